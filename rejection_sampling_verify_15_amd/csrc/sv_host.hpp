// Host-side helpers of the libspecverify C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include "specverify.h"

namespace sv {

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// What a cut search learnt of a row, for the verification after it: m is the
// row's largest logit and z the sum, over the logits the cut keeps, of
// exp((x - m) / T) in fp64.  All zero for a row not searched.
struct RowStat {
  double z;
  float m;
  uint32_t pad;
};
static_assert(sizeof(RowStat) == 16, "row stat size");

// The thresholds of a filtered chain call (sv_filter.hip): launches over the
// rows of the sampling requests, writing thr[b][row] = key + 1 of each cut
// (0: none).  `slots` is the zero-filled search area of
// filter_workspace_bytes(B, gamma, V, dtype) bytes, left zero-filled.  With
// `stats` (bf16 rows only; 16 bytes per row, zero-filled) every row that gets
// a cut also gets its largest logit and kept mass there.
// Returns an sv_status.
int launch_filter_rows(const void* target, const void* draft, const float* temperature, const int32_t* top_k,
                       const float* top_p, int B, int gamma, int V, int dtype, uint32_t* thr, void* stats,
                       void* slots, hipStream_t stream);
size_t filter_workspace_bytes(int B, int gamma, int V, int dtype);

// Value of a test control (sv_set_test_hook); 0 when unset.
long long test_hook(int hook);

// Poll bound of the bounded waits: `dflt`, or the SV_HOOK_SPIN_LIMIT control.
inline uint32_t spin_limit(uint32_t dflt) {
  const long long v = test_hook(SV_HOOK_SPIN_LIMIT);
  return v > 0 ? static_cast<uint32_t>(v < 0xffffffffLL ? v : 0xffffffffLL) : dflt;
}

// Hands out the event pair of the next timed launch while a timing session is
// open (sv_timing_begin); leaves both NULL otherwise.
void timing_slot(int kernel, hipEvent_t* start, hipEvent_t* stop);

// Every kernel launch of the library goes through here: a plain dispatch, with
// events attached to it during a timing session.
template <typename F, typename... Args>
inline void launch(int kernel, F fn, dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                   Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  timing_slot(kernel, &start, &stop);
  hipExtLaunchKernelGGL(fn, grid, block, shmem, stream, start, stop, 0u, args...);
}

}  // namespace sv
