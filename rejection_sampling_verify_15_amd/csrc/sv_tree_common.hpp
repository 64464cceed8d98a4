// Pieces shared by the token-tree kernels (naive sampling / greedy descent and
// multi-step speculative sampling): chunk geometry, the one-run-per-lane
// chunk load, and the tagged words their workgroups exchange.
#pragma once

#include "sv_device.hpp"

namespace sv {

__device__ inline bool tree_temp_ok(float t) { return isfinite(t) && (t == 0.0f || t >= 1.17549435e-38f); }

constexpr int kTreeChunk = 2048;           // logits per stream item
constexpr int kTreeChunkCache = 4;         // chunk words per lane in a choose item
constexpr int kTreeMaxChunks = kTreeChunkCache * kWave;
constexpr int kCtlStride = 16;             // control words per request: one 128-byte line
constexpr uint64_t kTreeMark = 1ull << 63;
constexpr uint32_t kTreeSpinLimit = 1u << 22;

// A chunk as one contiguous run of kRun logits per lane (lane l holds
// [c0 + l * kRun, c0 + (l + 1) * kRun)), so that a lane's sum is one stretch of
// the chunk's CDF.  Loaded as kItems groups of kPer logits from clamped
// addresses; groups past the row's end become -inf.
template <int DT, bool VEC, int CHUNK = kTreeChunk>
struct LaneRun {
  static constexpr int kPer = VEC ? Elem<DT>::kVec : 1;
  static constexpr int kItems = CHUNK / (kWave * kPer);
  static constexpr int kRun = kItems * kPer;
  uint32_t w[kItems][VEC ? 4 : 1];

  __device__ static inline int index(int c0, int j, int e) {
    return c0 + static_cast<int>(threadIdx.x) * kRun + j * kPer + e;
  }
  __device__ inline void load(const void* row, int c0, int c1) {
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      const int k0 = index(c0, j, 0);
      const int k = k0 < c1 ? k0 : c0;
      if constexpr (VEC) {
        // cached: the choose workgroup soon re-reads a run of the row
        const uint4 v = load_row16_cached(static_cast<const char*>(row) + static_cast<size_t>(k) * Elem<DT>::kBytes);
        w[j][0] = v.x; w[j][1] = v.y; w[j][2] = v.z; w[j][3] = v.w;
      } else if constexpr (DT == 0) {
        w[j][0] = static_cast<const uint16_t*>(row)[k];
      } else {
        w[j][0] = static_cast<const uint32_t*>(row)[k];
      }
    }
    constexpr uint32_t kNegInf = DT == 0 ? (VEC ? 0xff80ff80u : 0xff80u) : 0xff800000u;
#pragma unroll
    for (int j = 0; j < kItems; ++j)
      if (index(c0, j, 0) >= c1) {
#pragma unroll
        for (int q = 0; q < (VEC ? 4 : 1); ++q) w[j][q] = kNegInf;
      }
  }
  __device__ inline float at(int j, int e) const {
    if constexpr (VEC) {
      if constexpr (DT == 0) return __uint_as_float((e & 1) ? (w[j][e >> 1] & 0xffff0000u) : (w[j][e >> 1] << 16));
      else return __uint_as_float(w[j][e]);
    } else {
      if constexpr (DT == 0) return __uint_as_float(w[j][0] << 16);
      else return __uint_as_float(w[j][0]);
    }
  }
};

// [63] mark, [62:56] level + 1, [55:32] argmax (greedy), [31:0] max bits.
__device__ inline uint64_t tree_chunk_word(int level, float m, int idx) {
  return kTreeMark | (static_cast<uint64_t>(level + 1) << 56) |
         (static_cast<uint64_t>(static_cast<uint32_t>(idx) & 0xffffffu) << 32) | __float_as_uint(m);
}
__device__ inline bool chunk_at_level(uint64_t w, int level) {
  return (w >> 56) == (0x80ull | static_cast<uint64_t>(level + 1));
}

// The fp64 sums of a sampling chunk travel tagged: the sign bit set as the
// mark (the sums are >= 0) and level + 1 in the low 7 bits of the mantissa,
// which the reader clears (a relative change below 3e-14, far under what the
// draw needs).  The choose workgroup so tells this level's sums from an
// earlier level's without a flag, and the stream workgroup need not wait for
// their stores before it publishes its chunk word.
constexpr uint64_t kSumTag = 0x7full;
__device__ inline uint64_t tag_sum(double v, int level) {
  return ((static_cast<uint64_t>(__double_as_longlong(v)) & ~kSumTag) | static_cast<uint64_t>(level + 1)) | kTreeMark;
}
__device__ inline bool sum_at_level(uint64_t w, int level) {
  return (w & kTreeMark) != 0 && (w & kSumTag) == static_cast<uint64_t>(level + 1);
}
__device__ inline double sum_value(uint64_t w) {
  return __longlong_as_double(static_cast<long long>(w & ~(kTreeMark | kSumTag)));
}

}  // namespace sv
