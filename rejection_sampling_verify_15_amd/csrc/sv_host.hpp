// Host-side helpers of the libspecverify C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace sv
