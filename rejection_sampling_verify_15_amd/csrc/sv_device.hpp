// Device building blocks shared by the libspecverify kernels (gfx950, wave64).
//
// Rows are read with 16-byte loads (8 bf16 or 4 fp32 per lane) laid out so
// that load j of a wave (or workgroup) covers one contiguous span, every wave
// reading 1 KiB contiguous per instruction.  Rows that are not 16-byte
// aligned, or whose length is not a multiple of the vector width, take the
// scalar variant of the same loops.  The single-launch chain and tree
// kernels work in one-wave workgroups (RawSlice with NT = kWave); the
// multi-launch forms and the debug-probabilities kernels use 256-thread
// workgroups over kChunk-logit (row, chunk) items (Slice).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 16384;  // logits per (row, chunk) work item

__host__ __device__ inline int num_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// ---------------------------------------------------------------------------
// element access
// ---------------------------------------------------------------------------
// 16 bytes of a logit row, loaded non-temporally: every logit is read by one
// workgroup (the draw re-reads a row or two at most), so the lines need not
// stay in the caches.  Measured on the chain kernels: batched 36.8 -> 36.0 us,
// deep 288 -> 274 us.
// The pointer is taken as a global-memory one (address space 1), so the load
// is a global load rather than a flat one even where the compiler cannot
// trace the pointer back to a kernel argument.
typedef unsigned int U32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) U32x4* GlobalU32x4Ptr;
__device__ inline uint4 load_row16(const void* p) {
  const U32x4 v = __builtin_nontemporal_load((GlobalU32x4Ptr)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same load kept in the caches, for rows that are read again soon after.
__device__ inline uint4 load_row16_cached(const void* p) { return *static_cast<const uint4*>(p); }

template <int DT> struct Elem;

template <> struct Elem<0> {  // bf16 stored as raw 16-bit patterns
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  __device__ static inline float at(const void* row, int k) {
    const uint16_t b = static_cast<const uint16_t*>(row)[k];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
  __device__ static inline uint4 raw(const void* row, int k) {
    return load_row16(static_cast<const uint16_t*>(row) + k);
  }
  __device__ static inline void unpack(const uint4 w, float (&x)[kVec]) {
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(q[i] << 16);
      x[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
    }
  }
};

template <> struct Elem<1> {  // float32
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
  __device__ static inline float at(const void* row, int k) {
    return static_cast<const float*>(row)[k];
  }
  __device__ static inline uint4 raw(const void* row, int k) {
    return load_row16(static_cast<const float*>(row) + k);
  }
  __device__ static inline void unpack(const uint4 w, float (&x)[kVec]) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};

// Per-thread slice of one span of kThreads * kPer * ITEMS elements: ITEMS
// groups of kPer consecutive elements; group j of thread t starts at element
// c0 + (j * kThreads + t) * kPer.  A full span issues all its loads before any
// use (no branches between them, so they are in flight together); a partial
// span loads from a clamped, in-range address and masks the excess to -inf.
template <int DT, bool VEC, int ITEMS = kChunk / (kThreads * (VEC ? Elem<DT>::kVec : 1))>
struct Slice {
  static constexpr int kPer = VEC ? Elem<DT>::kVec : 1;
  static constexpr int kItems = ITEMS;
  static constexpr int kSpan = kThreads * kPer * ITEMS;
  float x[kItems][kPer];

  __device__ static inline int index(int c0, int j, int e) {
    return c0 + (j * kThreads + static_cast<int>(threadIdx.x)) * kPer + e;
  }

  // Loads [c0, c1) of `row` (c1 - c0 <= kSpan).
  __device__ inline void load(const void* row, int c0, int c1) {
    if (c1 - c0 == kSpan) {
      if constexpr (VEC) {
        uint4 w[kItems];
#pragma unroll
        for (int j = 0; j < kItems; ++j) w[j] = Elem<DT>::raw(row, index(c0, j, 0));
#pragma unroll
        for (int j = 0; j < kItems; ++j) Elem<DT>::unpack(w[j], x[j]);
      } else {
#pragma unroll
        for (int j = 0; j < kItems; ++j) x[j][0] = Elem<DT>::at(row, index(c0, j, 0));
      }
    } else {
      if constexpr (VEC) {
        uint4 w[kItems];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
          const int k0 = index(c0, j, 0);
          w[j] = Elem<DT>::raw(row, k0 < c1 ? k0 : c0);
        }
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
          Elem<DT>::unpack(w[j], x[j]);
          if (index(c0, j, 0) >= c1) {
#pragma unroll
            for (int e = 0; e < kPer; ++e) x[j][e] = -INFINITY;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
          const int k0 = index(c0, j, 0);
          const float v = Elem<DT>::at(row, k0 < c1 ? k0 : c0);
          x[j][0] = k0 < c1 ? v : -INFINITY;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// fp64 exponential of a non-positive argument
// ---------------------------------------------------------------------------
constexpr double kLog2e = 0x1.71547652b82fep+0;

// 2^t for t <= 0 (t = -inf gives 0; t a few ulps above 0 is fine too): t =
// n + f with n = rint(t) and |f| <= 1/2, 2^f = 1 + f q(f), and the result
// scaled by 2^n.  q is the degree-8 polynomial interpolating (2^f - 1) / f at
// the nine Chebyshev nodes of [-1/2, 1/2] (exp2_coefficients.py derives the
// constants); the relative error is at most 3.7e-14 (at f = -1/2), far inside
// the 1e-10 the inverse-CDF draw needs, and 2^0 is exactly 1.  No table, so no shared-memory
// reads on the dependent path of each exponential.
__host__ __device__ inline double exp2_neg(double t_in) {
  const double t = __builtin_fmax(t_in, -1100.0);
  const double n = __builtin_rint(t);
  const double f = t - n;  // exact, |f| <= 1/2
  double q = 0x1.b63880a30e9ffp-24;
  q = __builtin_fma(q, f, 0x1.63d136366db24p-20);
  q = __builtin_fma(q, f, 0x1.ffcb9515a8016p-17);
  q = __builtin_fma(q, f, 0x1.4308ac85aa947p-13);
  q = __builtin_fma(q, f, 0x1.5d87fe86fe88ep-10);
  q = __builtin_fma(q, f, 0x1.3b2ab7181b755p-7);
  q = __builtin_fma(q, f, 0x1.c6b08d7047e52p-5);
  q = __builtin_fma(q, f, 0x1.ebfbdff823cedp-3);
  q = __builtin_fma(q, f, 0x1.62e42fefa39efp-1);
  const double p = __builtin_fma(q, f, 1.0);
  return __builtin_ldexp(p, static_cast<int>(n));
}

// ---------------------------------------------------------------------------
// order-preserving keys of logits (consistent top-k / top-p thresholds)
// ---------------------------------------------------------------------------
// An unsigned key that orders like the float (both zeros map to +0's key, so
// they tie, as they compare equal); NaN is not a valid logit.
__device__ inline uint32_t order_key(float x) {
  const uint32_t u = x == 0.0f ? 0u : __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// A stored row threshold: 0 means no filter, otherwise key + 1.
__device__ inline float stored_threshold(uint32_t stored) {
  return stored ? key_value(stored - 1u) : -INFINITY;
}

// ---------------------------------------------------------------------------
// raw (still packed) slices for prefetching
// ---------------------------------------------------------------------------
// The element layout of Slice (for NT threads), kept as loaded (16-byte words, or single
// elements on the scalar path) so that two items can be in flight per thread
// at the cost of the raw words only; elements are unpacked where they are used.
template <int DT, bool VEC, int ITEMS, int NT = kThreads>
struct RawSlice {
  static constexpr int kPer = VEC ? Elem<DT>::kVec : 1;
  static constexpr int kItems = ITEMS;
  static constexpr int kSpan = NT * kPer * ITEMS;
  uint32_t w[ITEMS][VEC ? 4 : 1];

  __device__ static inline int index(int c0, int j, int e) {
    return c0 + (j * NT + static_cast<int>(threadIdx.x)) * kPer + e;
  }

  // Issues the loads of [c0, c1) of `row` (c1 - c0 <= kSpan) from clamped,
  // in-range addresses, with no branches between them.
  __device__ inline void load(const void* row, int c0, int c1) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int k0 = index(c0, j, 0);
      const int k = k0 < c1 ? k0 : c0;
      if constexpr (VEC) {
        const uint4 v = Elem<DT>::raw(row, k);
        w[j][0] = v.x; w[j][1] = v.y; w[j][2] = v.z; w[j][3] = v.w;
      } else if constexpr (DT == 0) {
        w[j][0] = static_cast<const uint16_t*>(row)[k];
      } else {
        w[j][0] = static_cast<const uint32_t*>(row)[k];
      }
    }
  }

  // Moves group j + 1 to group j (the last group keeps its words): a loop
  // that works on group 0 and shifts stays in registers without unrolling.
  __device__ inline void shift() {
#pragma unroll
    for (int j = 0; j + 1 < ITEMS; ++j)
#pragma unroll
      for (int q = 0; q < (VEC ? 4 : 1); ++q) w[j][q] = w[j + 1][q];
  }

  // Every element below `thr` becomes -inf (a consistent top-k / top-p
  // filter applied to the loaded words).
  __device__ inline void mask_below(float thr) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
#pragma unroll
      for (int q = 0; q < (VEC ? 4 : 1); ++q) {
        const uint32_t v = w[j][q];
        if constexpr (DT == 0 && VEC) {
          const uint32_t lo = __uint_as_float(v << 16) < thr ? 0xff80u : (v & 0xffffu);
          const uint32_t hi = __uint_as_float(v & 0xffff0000u) < thr ? 0xff800000u : (v & 0xffff0000u);
          w[j][q] = hi | lo;
        } else if constexpr (DT == 0) {
          w[j][q] = __uint_as_float(v << 16) < thr ? 0xff80u : v;
        } else {
          w[j][q] = __uint_as_float(v) < thr ? 0xff800000u : v;
        }
      }
  }

  // Element e of group j as float (no range check).
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

// Workgroup barrier that orders LDS accesses only: global loads still in
// flight (prefetched data) stay in flight across it.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// reductions
// ---------------------------------------------------------------------------
// (value, index) argmax with the lowest index among equal values.
struct ArgMax {
  float v;
  int i;
};

__device__ inline ArgMax argmax_combine(ArgMax a, ArgMax b) {
  return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

// Running (max, sum of exp2((x - max) * s)) pair of a softmax normaliser.
struct MaxSum {
  float m;
  float z;
};

__device__ inline float scale_to(float m_from, float m_to, float s) {
  return (m_from == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m_from - m_to) * s);
}

__device__ inline MaxSum maxsum_combine(MaxSum a, MaxSum b, float s) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return {m, 0.0f};
  return {m, a.z * scale_to(a.m, m, s) + b.z * scale_to(b.m, m, s)};
}

// ---------------------------------------------------------------------------
// cross-lane moves within a wave (DPP: register to register, no LDS round
// trip).  Controls use the gfx9 DPP encoding; lanes whose source is outside
// the pattern, or that a row mask leaves out, receive 0.
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadSwap1 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
  kDppQuadSwap2 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
  kDppRowMirror = 0x140,      // lane i <- 15 - i within each row of 16
  kDppRowHalfMirror = 0x141,  // lane i <- 7 - i within each half row
  kDppRowShr1 = 0x111,        // lane i <- i - 1 within the row
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,     // lane 15 of each row to the whole next row
  kDppRowBcast31 = 0x143,     // lane 31 to rows 2 and 3
  kDppWaveShr1 = 0x138,       // lane i <- i - 1 across the wave
};

template <int CTRL, int ROW_MASK = 0xf>
__device__ inline int lane_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, true);
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float lane_move(float v) {
  return __int_as_float(lane_move<CTRL, ROW_MASK>(__float_as_int(v)));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline double lane_move(double v) {
  struct Words { int lo, hi; };
  Words w = __builtin_bit_cast(Words, v);
  w.lo = lane_move<CTRL, ROW_MASK>(w.lo);
  w.hi = lane_move<CTRL, ROW_MASK>(w.hi);
  return __builtin_bit_cast(double, w);
}

__device__ inline int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ inline float read_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ inline double read_lane(double v, int lane) {
  struct Words { int lo, hi; };
  Words w = __builtin_bit_cast(Words, v);
  w.lo = __builtin_amdgcn_readlane(w.lo, lane);
  w.hi = __builtin_amdgcn_readlane(w.hi, lane);
  return __builtin_bit_cast(double, w);
}

// Reduction of one value per lane over the whole wave with an associative,
// commutative op; every lane receives the result.  Within each row of 16 the
// butterfly xor 1, xor 2, half mirror, mirror leaves the row's result in all
// its lanes; the four rows are then combined from lanes 0, 16, 32, 48.
template <typename T, typename Op>
__device__ inline T wave_allreduce(T v, Op op) {
  v = op(v, lane_move<kDppQuadSwap1>(v));
  v = op(v, lane_move<kDppQuadSwap2>(v));
  v = op(v, lane_move<kDppRowHalfMirror>(v));
  v = op(v, lane_move<kDppRowMirror>(v));
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}

template <typename T> __device__ inline T wave_sum(T v) {
  return wave_allreduce(v, [](T a, T b) { return a + b; });
}

__device__ inline int wave_min(int v) {
  return wave_allreduce(v, [](int a, int b) { return min(a, b); });
}

__device__ inline int wave_max_int(int v) {
  return wave_allreduce(v, [](int a, int b) { return max(a, b); });
}

__device__ inline float wave_max(float v) {
  return wave_allreduce(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ inline ArgMax wave_argmax(ArgMax a) {
  // the pair travels as two lanes' worth of moves per step
  auto step = [](ArgMax x, ArgMax y) { return argmax_combine(x, y); };
  a = step(a, ArgMax{lane_move<kDppQuadSwap1>(a.v), lane_move<kDppQuadSwap1>(a.i)});
  a = step(a, ArgMax{lane_move<kDppQuadSwap2>(a.v), lane_move<kDppQuadSwap2>(a.i)});
  a = step(a, ArgMax{lane_move<kDppRowHalfMirror>(a.v), lane_move<kDppRowHalfMirror>(a.i)});
  a = step(a, ArgMax{lane_move<kDppRowMirror>(a.v), lane_move<kDppRowMirror>(a.i)});
  const ArgMax r0{read_lane(a.v, 0), read_lane(a.i, 0)}, r1{read_lane(a.v, 16), read_lane(a.i, 16)};
  const ArgMax r2{read_lane(a.v, 32), read_lane(a.i, 32)}, r3{read_lane(a.v, 48), read_lane(a.i, 48)};
  return step(step(r0, r1), step(r2, r3));
}

__device__ inline MaxSum wave_maxsum(MaxSum a, float s) {
  auto step = [s](MaxSum x, MaxSum y) { return maxsum_combine(x, y, s); };
  a = step(a, MaxSum{lane_move<kDppQuadSwap1>(a.m), lane_move<kDppQuadSwap1>(a.z)});
  a = step(a, MaxSum{lane_move<kDppQuadSwap2>(a.m), lane_move<kDppQuadSwap2>(a.z)});
  a = step(a, MaxSum{lane_move<kDppRowHalfMirror>(a.m), lane_move<kDppRowHalfMirror>(a.z)});
  a = step(a, MaxSum{lane_move<kDppRowMirror>(a.m), lane_move<kDppRowMirror>(a.z)});
  const MaxSum r0{read_lane(a.m, 0), read_lane(a.z, 0)}, r1{read_lane(a.m, 16), read_lane(a.z, 16)};
  const MaxSum r2{read_lane(a.m, 32), read_lane(a.z, 32)}, r3{read_lane(a.m, 48), read_lane(a.z, 48)};
  return step(step(r0, r1), step(r2, r3));
}

// Inclusive prefix sum over the wave (lane order): a Hillis-Steele scan in
// each row (shifts 1, 2, 4, 8), then row 0's total into row 1 and row 2's
// into row 3, then the total of rows 0-1 into rows 2 and 3.
__device__ inline double wave_inclusive_sum(double v) {
  v += lane_move<kDppRowShr1>(v);
  v += lane_move<kDppRowShr2>(v);
  v += lane_move<kDppRowShr4>(v);
  v += lane_move<kDppRowShr8>(v);
  v += lane_move<kDppRowBcast15, 0xa>(v);
  v += lane_move<kDppRowBcast31, 0xc>(v);
  return v;
}

// Workgroup reductions through LDS; every thread receives the result.
__device__ inline ArgMax block_argmax(ArgMax a) {
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves];
  a = wave_argmax(a);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) { sv[w] = a.v; si[w] = a.i; }
  __syncthreads();
  ArgMax r{sv[0], si[0]};
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = argmax_combine(r, ArgMax{sv[i], si[i]});
  __syncthreads();
  return r;
}

__device__ inline MaxSum block_maxsum(MaxSum a, float s) {
  __shared__ float sm[kWaves];
  __shared__ float sz[kWaves];
  a = wave_maxsum(a, s);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) { sm[w] = a.m; sz[w] = a.z; }
  __syncthreads();
  MaxSum r{sm[0], sz[0]};
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = maxsum_combine(r, MaxSum{sm[i], sz[i]}, s);
  __syncthreads();
  return r;
}

template <int NV>
__device__ inline void block_sum_doubles(double (&v)[NV]) {
  __shared__ double sd[NV][kWaves];
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wave_sum(v[k]);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
#pragma unroll
    for (int k = 0; k < NV; ++k) sd[k][w] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += sd[k][i];
    v[k] = t;
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup of one double per thread (lanes in
// thread order); returns this thread's exclusive prefix and writes the total
// to *total.
__device__ inline double block_exclusive_scan(double v, double* total) {
  __shared__ double sw[kWaves];
  const int w = threadIdx.x / kWave;
  const double inc = wave_inclusive_sum(v);
  const double exc = lane_move<kDppWaveShr1>(inc);  // lane 0 receives 0
  if ((threadIdx.x % kWave) == kWave - 1) sw[w] = inc;
  __syncthreads();
  double before = 0.0, all = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) before += sw[i];
    all += sw[i];
  }
  __syncthreads();
  *total = all;
  return before + exc;
}

// ---------------------------------------------------------------------------
// hand-off between workgroups of one launch
// ---------------------------------------------------------------------------
// Data that one workgroup produces and another consumes within the same
// launch travels through agent-scope (whole-device) atomic accesses: the
// stores write through to the device-coherent level and the loads read from
// it, so neither depends on which XCD's L2 holds a copy.  A producer makes its
// stores visible by waiting for their completion before it counts itself in;
// the consumer that sees the final count issues its loads after that atomic
// returns.
__device__ inline void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void store_coherent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline double load_coherent_f64(const double* p) {
  return __longlong_as_double(static_cast<long long>(load_coherent(reinterpret_cast<const uint64_t*>(p))));
}
__device__ inline void store_coherent_f64(double* p, double v) {
  store_coherent(reinterpret_cast<uint64_t*>(p), static_cast<uint64_t>(__double_as_longlong(v)));
}

// Waits until every memory access this wave has issued is complete (on gfx9
// the vector-memory counter covers stores as well as loads); also a compiler
// barrier.
__device__ inline void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Counts the calling thread in on `counter` once its wave's coherent stores
// are complete; returns the count before this arrival.
__device__ inline uint32_t arrive(uint32_t* counter) {
  wait_memory();
  const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::: "memory");
  return old;
}

}  // namespace sv
