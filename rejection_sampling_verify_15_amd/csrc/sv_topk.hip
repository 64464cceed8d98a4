// Chain verification under a consistent top-k filter: every target and draft
// row of a sampling request keeps its min(k, V) largest logits (all logits
// equal to the k-th largest included) and drops the rest before the
// temperature softmax, the same rule on both sides, which keeps the method
// exact for the filtered target (close-reading notes 02, section 5.4).  The
// test and the draws are then those of the unfiltered call (Leviathan et
// al.'s Algorithm 1 as restated in the close-reading notes 02, section 4).
// See include/specverify.h for the contract.
//
// Two launches on the caller's stream, with no waits between workgroups:
//
//  1. topk_rows    one 512-thread workgroup per (request, row read), each
//                  wave owning a contiguous tile of the row.  The row's max
//                  and lowest-index argmax come first, with each thread's
//                  maximum per 16-byte step (bf16) or per batch of loads.
//                  For a sampling row the k-th largest thread maximum bounds
//                  the k-th largest logit from below (k threads hold a logit
//                  at least that large), so only the logits at or above it
//                  -- about k of them -- are collected in LDS with their
//                  indices, each lane reloading (through the caches) only
//                  the steps or batches whose maximum reaches the bound; the
//                  exact k-th largest value is found among them by a
//                  bit-by-bit search over order-preserving keys; each kept
//                  logit's rank by index places it in the row's kept list.  Should more than 512 logits pass the bound,
//                  a bisection over the whole row finds the value and one
//                  more visit compacts the kept logits in vocabulary order.
//                  With top-p, the threshold then rises to the largest kept
//                  logit whose softmax mass over the kept logits at or above
//                  it reaches p.
//  2. topk_decide  one wave per request: fp64 normalisers over the kept
//                  lists, the gamma-step test (tau = 1 if q' <= p' else
//                  p'/q', p' and q' zero below their row's threshold), and
//                  the residual or bonus draw by inverse CDF over the kept
//                  list of the draw's target row: max(0, p' - q') vanishes
//                  outside it, so no row is read again in full.  It returns
//                  the workspace it read to zero.
#include <algorithm>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {
namespace {

constexpr int kTopkMax = SV_MAX_TOPK;
constexpr int kTopkKept = SV_TOPK_MAX_KEPT;
constexpr int kRowThreads = 512;  // two workgroups per CU at this kernel's registers
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kCand = kRowThreads;   // logits the exact selection sorts at most
// steps of a tile visit whose loads are in flight together (bf16 unpacks to
// twice the registers; more of its steps spill)
constexpr int kInFlight = 16;
constexpr int kInFlightBf16 = 8;
constexpr int kMaxRowsTopk = 2 * SV_MAX_GAMMA + 1;
constexpr int kNoIndex = 0x7fffffff;

// One per (request, row).  A sampling row: its kept count, the threshold (the
// k-th largest logit), max and argmax; a greedy row: count 0 and its argmax.
// A row that was not read stays all zero.
struct TopkHead {
  int32_t count;
  float thr;
  float max;
  int32_t arg;
};
struct TopkEntry {
  int32_t idx;
  float val;
};

struct TopkArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;  // [B] or NULL: no top-p
  int B, gamma, V;
  int tile;  // logits per wave of a row workgroup (a multiple of its step)
  int32_t* out_tokens;
  int32_t* out_n;
  TopkHead* heads;   // [B][2*gamma+1]
  TopkEntry* lists;  // [B][2*gamma+1][kTopkKept], vocabulary order
  double* zs;        // [B][2*gamma+1] fp64 normaliser of each sampling row's kept logits
};

// T must be 0 (greedy) or a finite positive normal float.
__device__ inline bool topk_temp_ok(float t) { return isfinite(t) && (t == 0.0f || t >= 1.17549435e-38f); }

// Unsigned keys in the order of the floats (-0 just below +0; no NaNs).
__device__ inline uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_float(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

__device__ inline double exp_scaled_t(float x, float m, double l2t) {
  return exp2_neg((static_cast<double>(x) - static_cast<double>(m)) * l2t);
}

// The logits one wave of a row workgroup owns: [t0, t1), visited one wave
// step at a time; at step s lane l holds the kPer logits from
// t0 + s * kStep + l * kPer.  Every visit reads the tile through the caches,
// where the next visit finds it again.
template <int DT, bool VEC>
struct RowTile {
  static constexpr int kPer = VEC ? Elem<DT>::kVec : 1;
  static constexpr int kStep = kWave * kPer;
  const void* row;
  int t0, t1;

  static constexpr int kU = DT == 0 ? kInFlightBf16 : kInFlight;
  static constexpr int kBatch = kU * kStep;  // logits of a wave's batch of loads in flight
  __device__ inline int batches() const { return (t1 - t0 + kBatch - 1) / kBatch; }

  // f(i0, x, valid) for every step, every lane taking part (valid is false
  // past the tile), so f may use wave-wide operations; done(batch) after
  // each batch of kU steps.
  template <typename F>
  __device__ inline void each(F&& f) const {
    each(f, [](int) {});
  }
  template <typename F, typename D>
  __device__ inline void each(F&& f, D&& done) const {
    for (int bt = 0; bt < batches(); ++bt) {
      visit_batch(bt, f);
      done(bt);
    }
  }
  // The steps of batch bt only.
  template <typename F>
  __device__ inline void visit_batch(int bt, F&& f) const {
    const int lane = threadIdx.x % kWave;
    {
      const int base = t0 + bt * kBatch;
      if constexpr (VEC) {
        // the raw groups stay packed until their step is visited
        uint4 w[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i0 = base + u * kStep + lane * kPer;
          if (i0 < t1)
            w[u] = load_row16_cached(static_cast<const char*>(row) + static_cast<size_t>(i0) * Elem<DT>::kBytes);
          else
            w[u] = make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i0 = base + u * kStep + lane * kPer;
          float x[kPer];
          Elem<DT>::unpack(w[u], x);
          f(i0, x, i0 < t1);
        }
      } else {
        float x[kU][1];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i0 = base + u * kStep + lane;
          x[u][0] = i0 < t1 ? Elem<DT>::at(row, i0) : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) f(base + u * kStep + lane, x[u], base + u * kStep + lane < t1);
      }
    }
  }
};

// bf16 rows on the vector path also keep each step's maximum per thread in
// LDS (tiles of at most kMaxSteps steps), so the candidate visit reloads
// only the 16-byte groups that can hold a candidate, all at once.
constexpr int kMaxSteps = 32;
static_assert(kMaxSteps % kInFlightBf16 == 0, "a tile of kMaxSteps steps is whole batches");

// Per-thread maxima of the first visit's batches, kMaxSlots of them held
// in registers: with more batches, consecutive ones share a slot.
constexpr int kMaxSlots = 8;
struct BatchMax {
  float m[kMaxSlots];
  int per;  // batches per slot
  __device__ inline int slot(int bt) const { return bt / per; }
  __device__ inline void add(int bt, float v) {
    const int s = slot(bt);
#pragma unroll
    for (int i = 0; i < kMaxSlots; ++i)
      if (i == s) m[i] = fmaxf(m[i], v);
  }
};

// The kk-th largest of one key per thread (0 stands for none): the largest
// t with at least kk keys >= t.  The keys go through LDS to the first wave,
// which builds t from the top bit down, eight ballot counts per bit (no
// barrier per bit), and hands it back.  With low_bit = 16 every key is a
// bf16 value's: its low 16 bits are 0 for a positive value and all ones for
// a negative one, so only the top 16 bits are searched and the low ones
// follow from the sign.
__device__ inline uint32_t block_kth_key(uint32_t key, int kk, uint32_t* s_keys, uint32_t* s_ans, int low_bit) {
  s_keys[threadIdx.x] = key;
  __syncthreads();
  if (threadIdx.x < kWave) {
    constexpr int kPerLane = kRowThreads / kWave;
    uint32_t k8[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) k8[i] = s_keys[i * kWave + threadIdx.x];
    uint32_t ans = 0u;
    for (int bit = 31; bit >= low_bit; --bit) {
      const uint32_t c = ans | (1u << bit);
      int n = 0;
#pragma unroll
      for (int i = 0; i < kPerLane; ++i) n += __popcll(__ballot(k8[i] >= c));
      if (n >= kk) ans = c;
    }
    if (low_bit > 0 && ans != 0u && !(ans & 0x80000000u)) ans |= (1u << low_bit) - 1u;
    if (threadIdx.x == 0) *s_ans = ans;
  }
  __syncthreads();
  return *s_ans;
}

__device__ inline double block_sum_f64(double v, double* s_red) {
  const int w = threadIdx.x / kWave;
  v = wave_sum(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) s_red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) t += s_red[i];
  return t;
}

__device__ inline float block_max_f32(float v, float* s_red) {
  const int w = threadIdx.x / kWave;
  v = wave_max(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) s_red[w] = v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) t = fmaxf(t, s_red[i]);
  return t;
}

// Sum of one int per thread over the workgroup; every thread receives it.
__device__ inline int block_count(int v, int* s_red) {
  const int w = threadIdx.x / kWave;
  v = wave_sum(v);
  __syncthreads();  // s_red is free again
  if (threadIdx.x % kWave == 0) s_red[w] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) t += s_red[i];
  return t;
}

// TOPP: top_p is given (a separate instantiation, so that calls without it
// carry none of its work).
template <int DT, bool VEC, bool TOPP>
__global__ __launch_bounds__(kRowThreads) void topk_rows(TopkArgs a) {
  __shared__ uint32_t s_keys[kRowThreads];
  __shared__ uint32_t s_kth;
  constexpr bool kStepMax = DT == 0 && VEC;
  __shared__ uint16_t s_smax[kStepMax ? kMaxSteps * kRowThreads : 1];  // bf16: each step's maximum, per thread
  __shared__ float s_kv[kTopkKept];
  __shared__ int s_ki[kTopkKept];
  __shared__ double s_e[kTopkKept];
  __shared__ double s_dred[kRowWaves];
  __shared__ float s_fred[kRowWaves];
  __shared__ int s_nkept;
  __shared__ float s_cand[kCand];
  __shared__ int s_cidx[kCand];
  __shared__ TopkEntry s_keep[kRowWaves][kTopkKept];
  __shared__ int s_cnt[kRowWaves];
  __shared__ int s_red[kRowWaves];
  __shared__ float s_am_v[kRowWaves];
  __shared__ int s_am_i[kRowWaves];
  __shared__ int s_ncand;
  using Tile = RowTile<DT, VEC>;
  constexpr int kPer = Tile::kPer;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const int b = static_cast<int>(blockIdx.x / static_cast<unsigned>(R));
  const int k = static_cast<int>(blockIdx.x - static_cast<unsigned>(b) * R);
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int w = tid / kWave;
  const float T = a.temperature[b];
  if (!topk_temp_ok(T)) return;
  const bool sampling = T > 0.0f;
  if (!sampling && k > G) return;  // greedy requests read target rows only
  int kk = 0;
  float pp = 1.0f;
  if (sampling) {
    const int kr = a.top_k[b];
    if (kr < 1 || kr > kTopkMax) return;  // an invalid request: nothing is read
    kk = min(kr, a.V);
    if constexpr (TOPP) {
      pp = a.top_p[b];
      if (!(pp > 0.0f && pp <= 1.0f)) return;
    }
  }
  Tile tile;
  tile.row = k <= G ? static_cast<const char*>(a.target) +
                          (static_cast<size_t>(b) * (G + 1) + k) * static_cast<size_t>(a.V) * Elem<DT>::kBytes
                    : static_cast<const char*>(a.draft) +
                          (static_cast<size_t>(b) * G + (k - G - 1)) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
  tile.t0 = min(a.V, w * a.tile);
  tile.t1 = min(a.V, tile.t0 + a.tile);
  // 1) max, lowest-index argmax, this thread's own max, and its maximum per
  //    batch of loads (so the candidate visit re-reads only the batches
  //    that can hold a candidate)
  ArgMax best{-INFINITY, kNoIndex};
  BatchMax bm;
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i) bm.m[i] = -INFINITY;
  bm.per = (tile.batches() + kMaxSlots - 1) / kMaxSlots;
  if (bm.per < 1) bm.per = 1;
  float cur = -INFINITY;
  const bool by_step = kStepMax && tile.t1 - tile.t0 <= kMaxSteps * Tile::kStep;
  tile.each(
      [&](int i0, const float (&x)[kPer], bool valid) {
        float sm = -INFINITY;
        if (valid)
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            sm = fmaxf(sm, x[e]);
            if (x[e] > best.v || best.i == kNoIndex) best = ArgMax{x[e], i0 + e};
          }
        cur = fmaxf(cur, sm);
        if constexpr (kStepMax) {
          if (by_step) s_smax[((i0 - tile.t0) / Tile::kStep) * kRowThreads + tid] =
              static_cast<uint16_t>(__float_as_uint(sm) >> 16);
        }
      },
      [&](int bt) {
        bm.add(bt, cur);
        cur = -INFINITY;
      });
  const float own_max = best.v;
  ArgMax wb = wave_argmax(best);
  if (lane == 0) {
    s_am_v[w] = wb.v;
    s_am_i[w] = wb.i;
  }
  __syncthreads();
  ArgMax rb{-INFINITY, kNoIndex};
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) rb = argmax_combine(rb, ArgMax{s_am_v[i], s_am_i[i]});
  TopkHead* head = a.heads + static_cast<size_t>(b) * R + k;
  if (!sampling) {
    if (tid == 0) *head = TopkHead{0, -INFINITY, rb.v, rb.i};
    return;
  }
  // 2) a lower bound: the kk-th largest thread maximum
  if (tid == 0) {
    s_ncand = 0;
    s_nkept = 0;
  }
  constexpr int kLowBit = DT == 0 ? 16 : 0;  // bf16 keys vary in their top 16 bits only
  const float lowb = key_float(block_kth_key(order_key(own_max), kk, s_keys, &s_kth, kLowBit));
  // The end of every sampling row: the kept logits sit in s_kv / s_ki (in
  // any order) when there are at most kTopkKept of them.  With top-p the
  // threshold rises to the largest kept value whose mass (the kept logits at
  // or above it, under the temperature softmax over the kept ones) reaches
  // p; then every kept logit is written at its rank by index.
  auto finish = [&](int kept, float thr) {
    // each staged logit's weight on the scale of the row maximum
    const double l2t = kLog2e / static_cast<double>(T);
    double e = 0.0;
    if (kept <= kTopkKept && tid < s_nkept) e = exp_scaled_t(s_kv[tid], rb.v, l2t);
    if (TOPP && kept <= kTopkKept && pp < 1.0f) {
      if (tid < kept) s_e[tid] = e;
      const double z = block_sum_f64(e, s_dred);  // its barriers publish s_e
      float cand = -INFINITY;
      if (tid < kept) {
        const float my = s_kv[tid];
        double m = 0.0;
        for (int j = 0; j < kept; ++j) m += s_kv[j] >= my ? s_e[j] : 0.0;
        if (m >= static_cast<double>(pp) * z) cand = my;
      }
      const float vp = block_max_f32(cand, s_fred);
      if (vp > thr) {
        thr = vp;
        kept = block_count(tid < kept && s_kv[tid] >= vp ? 1 : 0, s_red);
      }
    }
    if (kept <= kTopkKept && tid < kTopkKept && s_kv[tid] >= thr && tid < s_nkept) {
      const int my = s_ki[tid];
      int rank = 0;
      if constexpr (TOPP) {
        for (int j = 0; j < s_nkept; ++j) rank += (s_kv[j] >= thr && s_ki[j] < my) ? 1 : 0;
      } else {  // every staged logit is kept
        for (int j = 0; j < s_nkept; ++j) rank += s_ki[j] < my ? 1 : 0;
      }
      a.lists[(static_cast<size_t>(b) * R + k) * kTopkKept + rank] = TopkEntry{my, s_kv[tid]};
    }
    // the normaliser of the kept logits, for the decision and the draw
    const double zk = block_sum_f64((kept <= kTopkKept && tid < s_nkept && s_kv[tid] >= thr) ? e : 0.0, s_dred);
    if (tid == 0) {
      *head = TopkHead{kept, thr, rb.v, rb.i};
      a.zs[static_cast<size_t>(b) * R + k] = zk;
    }
  };
  // 3) the logits at or above it, with their indices: only the batches
  //    whose maximum reaches the bound are read again, each lane its own,
  //    the lanes' first such batches together, then their second ones
  auto collect = [&](int i0, const float (&x)[kPer], bool valid) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (valid && x[e] >= lowb) {
        const int slot = atomicAdd(&s_ncand, 1);
        if (slot < kCand) {
          s_cand[slot] = x[e];
          s_cidx[slot] = i0 + e;
        }
      }
  };
  uint32_t need = 0u;
  if constexpr (kStepMax) {
    // the steps whose maximum reaches the bound, up to four reloaded at once
    if (by_step)
      for (int st = 0; st < kMaxSteps; ++st)
        if (__uint_as_float(static_cast<uint32_t>(s_smax[st * kRowThreads + tid]) << 16) >= lowb) need |= 1u << st;
    while (__ballot(need != 0u)) {  // empty unless by_step
      constexpr int kR = 4;
      int i0s[kR];
      uint4 wv[kR];
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        i0s[j] = -1;
        if (need) {
          i0s[j] = tile.t0 + __builtin_ctz(need) * Tile::kStep + lane * kPer;
          need &= need - 1u;
        }
        wv[j] = (i0s[j] >= 0 && i0s[j] < tile.t1)
                    ? load_row16_cached(static_cast<const char*>(tile.row) + static_cast<size_t>(i0s[j]) * Elem<DT>::kBytes)
                    : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        float x[kPer];
        Elem<DT>::unpack(wv[j], x);
        collect(i0s[j], x, i0s[j] >= 0 && i0s[j] < tile.t1);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxSlots; ++i)
    if (!(kStepMax && by_step) && bm.m[i] >= lowb) need |= 1u << i;
  while (__ballot(need != 0u)) {
    const int sl = need ? __builtin_ctz(need) : -1;
    need &= need - 1u;
    for (int q = 0; q < bm.per; ++q) {
      const int bt = sl * bm.per + q;
      if (sl < 0 || bt >= tile.batches()) continue;
      tile.visit_batch(bt, collect);
    }
  }
  __syncthreads();
  const int ncand = s_ncand;
  if (ncand <= kCand) {
    // every logit >= the threshold is a candidate: the kk-th largest
    // candidate is the threshold; the kept ones are gathered and each
    // written at its rank by index
    const bool mine = tid < ncand;
    const float cv = mine ? s_cand[tid] : -INFINITY;
    const int ci = mine ? s_cidx[tid] : kNoIndex;
    const float thr = key_float(block_kth_key(mine ? order_key(cv) : 0u, kk, s_keys, &s_kth, kLowBit));
    if (mine && cv >= thr) {
      const int slot = atomicAdd(&s_nkept, 1);
      if (slot < kTopkKept) {
        s_kv[slot] = cv;
        s_ki[slot] = ci;
      }
    }
    __syncthreads();
    finish(s_nkept, thr);
    return;
  }
  float thr;
  {
    // bisection over keys: the largest key t with at least kk logits >= t
    uint32_t lo = 0u, hi = order_key(rb.v) + 1u;
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      int c = 0;
      tile.each([&](int, const float (&x)[kPer], bool valid) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) c += (valid && order_key(x[e]) >= mid) ? 1 : 0;
      });
      if (block_count(c, s_red) >= kk) lo = mid;
      else hi = mid;
    }
    thr = key_float(lo);
  }
  // 4) the kept logits in vocabulary order: staged per wave, then copied out
  int wcount = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  tile.each([&](int i0, const float (&x)[kPer], bool valid) {
    int n = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) n += (valid && x[e] >= thr) ? 1 : 0;
    const uint64_t b0 = __ballot(n & 1), b1 = __ballot(n & 2), b2 = __ballot(n & 4), b3 = __ballot(n & 8);
    if (b0 | b1 | b2 | b3) {
      int pos = wcount + __popcll(b0 & below) + 2 * __popcll(b1 & below) + 4 * __popcll(b2 & below) +
                8 * __popcll(b3 & below);
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (valid && x[e] >= thr) {
          if (pos < kTopkKept) s_keep[w][pos] = TopkEntry{i0 + e, x[e]};
          ++pos;
        }
      wcount += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2) + 8 * __popcll(b3);
    }
  });
  if (lane == 0) s_cnt[w] = wcount;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int i = 0; i < kRowWaves; ++i) total += s_cnt[i];
  if (total <= kTopkKept) {
    for (int i = tid; i < total; i += kRowThreads) {
      int ww = 0, off = 0;
      while (i - off >= s_cnt[ww]) {
        off += s_cnt[ww];
        ++ww;
      }
      s_kv[i] = s_keep[ww][i - off].val;
      s_ki[i] = s_keep[ww][i - off].idx;
    }
  }
  if (tid == 0) s_nkept = min(total, kTopkKept);
  __syncthreads();
  finish(total, thr);
}

// One wave per request.
template <int DT>
__global__ __launch_bounds__(kWave) void topk_decide(TopkArgs a) {
  __shared__ TopkHead s_h[kMaxRowsTopk];
  __shared__ double s_z[kMaxRowsTopk];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const int V = a.V;
  TopkHead* hb = a.heads + static_cast<size_t>(b) * R;
  TopkEntry* lb = a.lists + static_cast<size_t>(b) * R * kTopkKept;
  for (int r = lane; r < R; r += kWave) s_h[r] = hb[r];
  __syncthreads();
  const float T = a.temperature[b];
  const bool tok_t = topk_temp_ok(T);
  const bool sampling = tok_t && T > 0.0f;
  int bad = !tok_t;
  if (sampling) {
    const int kr = a.top_k[b];
    bad |= (kr < 1 || kr > kTopkMax);
    if (a.top_p) {
      const float pr = a.top_p[b];
      bad |= !(pr > 0.0f && pr <= 1.0f);
    }
    for (int r = lane; r < R; r += kWave) bad |= s_h[r].count > kTopkKept;
  }
  int32_t x = -1;
  float u = 0.0f;
  if (lane < G) {
    x = a.tokens[static_cast<size_t>(b) * G + lane];
    bad |= (x < 0 || x >= V);
  }
  if (sampling && lane <= G) {
    u = a.uniforms[static_cast<size_t>(b) * (G + 1) + lane];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  // the logits of the draft tokens, loaded before the normalisers are formed
  float xt = 0.0f, xd = 0.0f;
  if (sampling && lane < G && x >= 0 && x < V) {
    xt = Elem<DT>::at(static_cast<const char*>(a.target) +
                          (static_cast<size_t>(b) * (G + 1) + lane) * static_cast<size_t>(V) * Elem<DT>::kBytes,
                      x);
    xd = Elem<DT>::at(static_cast<const char*>(a.draft) +
                          (static_cast<size_t>(b) * G + lane) * static_cast<size_t>(V) * Elem<DT>::kBytes,
                      x);
  }
  const bool any_bad = __any(bad);
  const double l2t = sampling ? kLog2e / static_cast<double>(T) : 0.0;
  int n = -1;
  int32_t drawn = -1;
  if (!any_bad) {
    if (sampling) {
      // the fp64 normalisers the row workgroups left
      for (int r = lane; r < R; r += kWave) s_z[r] = a.zs[static_cast<size_t>(b) * R + r];
      __syncthreads();
    }
    int ok = 1;
    if (lane < G) {
      if (!sampling) {
        ok = (x == s_h[lane].arg);
      } else {
        const TopkHead ht = s_h[lane], hd = s_h[G + 1 + lane];
        const double p = xt >= ht.thr ? exp_scaled_t(xt, ht.max, l2t) / s_z[lane] : 0.0;
        const double q = xd >= hd.thr ? exp_scaled_t(xd, hd.max, l2t) / s_z[G + 1 + lane] : 0.0;
        const double tau = (q <= p) ? 1.0 : p / q;
        ok = static_cast<double>(u) <= tau;
      }
    }
    const uint64_t fail = __ballot(lane < G && !ok);
    n = fail ? static_cast<int>(__builtin_ctzll(fail)) : G;
    if (!sampling) {
      drawn = s_h[n].arg;
    } else {
      // the draw over the kept list of target row n: lane l holds entries
      // 4l .. 4l+3 (vocabulary order runs lane by lane)
      constexpr int kPerLane = kTopkKept / kWave;
      const bool residual = n < G;
      const TopkHead ht = s_h[n];
      const TopkHead hd = residual ? s_h[G + 1 + n] : TopkHead{0, 0.0f, 0.0f, 0};
      const double rzt = 1.0 / s_z[n];
      const double rzd = residual ? 1.0 / s_z[G + 1 + n] : 0.0;
      const TopkEntry* e = lb + static_cast<size_t>(n) * kTopkKept;
      const char* drow = residual ? static_cast<const char*>(a.draft) +
                                        (static_cast<size_t>(b) * G + n) * static_cast<size_t>(V) * Elem<DT>::kBytes
                                  : nullptr;
      int idx[kPerLane];
      double pw[kPerLane], wk[kPerLane];
      double own = 0.0, own_p = 0.0;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const int pos = lane * kPerLane + j;
        idx[j] = kNoIndex;
        pw[j] = 0.0;
        wk[j] = 0.0;
        if (pos < ht.count && e[pos].idx >= 0 && e[pos].idx < V) {
          const TopkEntry t = e[pos];
          idx[j] = t.idx;
          pw[j] = exp_scaled_t(t.val, ht.max, l2t) * rzt;
          if (residual) {
            const float d = Elem<DT>::at(drow, t.idx);
            const double q = d >= hd.thr ? exp_scaled_t(d, hd.max, l2t) * rzd : 0.0;
            wk[j] = fmax(0.0, pw[j] - q);
          } else {
            wk[j] = pw[j];
          }
        }
        own += wk[j];
        own_p += pw[j];
      }
      double W = wave_sum(own);
      if (residual && !(W > 0.0)) {  // an empty residual: draw from p' of that position
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) wk[j] = pw[j];
        own = own_p;
        W = wave_sum(own);
      }
      const double target = static_cast<double>(read_lane(u, G)) * W;
      double run = lane_move<kDppWaveShr1>(wave_inclusive_sum(own));  // lane 0 receives 0
      int hit = kNoIndex, last = -1;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        run += wk[j];
        if (wk[j] > 0.0) {
          last = idx[j];
          if (hit == kNoIndex && run > target) hit = idx[j];
        }
      }
      hit = wave_min(hit);
      last = wave_max_int(last);
      drawn = hit != kNoIndex ? hit : last;
    }
  }
  if (lane <= G) {
    int32_t v = -1;
    if (!any_bad) v = lane < n ? x : (lane == n ? drawn : -1);
    a.out_tokens[static_cast<size_t>(b) * (G + 1) + lane] = v;
  }
  if (lane == 0) a.out_n[b] = any_bad ? -1 : n;
  // the workspace this request used back to zero: the kept lists written,
  // then the heads
  for (int r = 0; r < R; ++r) {
    const int c = s_h[r].count <= kTopkKept ? s_h[r].count : 0;
    uint64_t* z = reinterpret_cast<uint64_t*>(lb + static_cast<size_t>(r) * kTopkKept);
    for (int j = lane; j < c; j += kWave) z[j] = 0ull;
  }
  uint32_t* hz = reinterpret_cast<uint32_t*>(hb);
  for (int i = lane; i < R * 4; i += kWave) hz[i] = 0u;
  for (int r = lane; r < R; r += kWave) a.zs[static_cast<size_t>(b) * R + r] = 0.0;
}

struct TopkLayout {
  size_t heads, lists, zs, total;
};

TopkLayout topk_layout(int B, int gamma) {
  const size_t R = 2 * static_cast<size_t>(gamma) + 1;
  TopkLayout L{};
  size_t off = 0;
  L.heads = off;
  off = align_up(off + static_cast<size_t>(B) * R * sizeof(TopkHead));
  L.lists = off;
  off = align_up(off + static_cast<size_t>(B) * R * kTopkKept * sizeof(TopkEntry));
  L.zs = off;
  off = align_up(off + static_cast<size_t>(B) * R * sizeof(double));
  L.total = off;
  return L;
}

template <int DT, bool VEC>
void launch_topk(const TopkArgs& a, hipStream_t stream) {
  const unsigned rows = static_cast<unsigned>(a.B) * static_cast<unsigned>(2 * a.gamma + 1);
  if (a.top_p)
    launch(SV_K_TOPK_ROWS, topk_rows<DT, VEC, true>, dim3(rows), dim3(kRowThreads), 0, stream, a);
  else
    launch(SV_K_TOPK_ROWS, topk_rows<DT, VEC, false>, dim3(rows), dim3(kRowThreads), 0, stream, a);
  launch(SV_K_TOPK_DECIDE, topk_decide<DT>, dim3(static_cast<unsigned>(a.B)), dim3(kWave), 0, stream, a);
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" size_t sv_chain_topk_workspace_bytes(int B, int gamma, int V, int dtype) {
  (void)dtype;
  if (B < 0 || B > SV_MAX_BATCH || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return 0;
  return topk_layout(B, gamma).total;
}

extern "C" int spec_verify_chain_topk(const void* target_logits, const void* draft_logits,
                                      const int32_t* draft_tokens, const float* uniforms,
                                      const float* temperature, const int32_t* top_k, const float* top_p,
                                      int B, int gamma, int V,
                                      int dtype, int32_t* out_tokens, int32_t* out_num_accepted, void* workspace,
                                      size_t workspace_bytes, void* hip_stream) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || B > SV_MAX_BATCH || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!target_logits || !temperature || !uniforms || !top_k || !out_tokens || !out_num_accepted || !workspace)
    return SV_ERR_NULL;
  if (gamma > 0 && (!draft_tokens || !draft_logits)) return SV_ERR_NULL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || (gamma > 0 && !aligned(draft_logits, es))) return SV_ERR_ALIGN;
  const TopkLayout L = topk_layout(B, gamma);
  if (workspace_bytes < L.total || !aligned(workspace, 256)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  TopkArgs a{};
  a.target = target_logits;
  a.draft = gamma > 0 ? draft_logits : nullptr;
  a.tokens = draft_tokens;
  a.uniforms = uniforms;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.out_tokens = out_tokens;
  a.out_n = out_num_accepted;
  a.heads = reinterpret_cast<TopkHead*>(ws + L.heads);
  a.lists = reinterpret_cast<TopkEntry*>(ws + L.lists);
  a.zs = reinterpret_cast<double*>(ws + L.zs);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  const int per = vec ? kv : 1;
  const int step = kWave * per;
  const int per_wave = (V + kRowWaves - 1) / kRowWaves;
  a.tile = (per_wave + step - 1) / step * step;
  if (dtype == SV_BF16) {
    if (vec) launch_topk<0, true>(a, stream);
    else launch_topk<0, false>(a, stream);
  } else {
    if (vec) launch_topk<1, true>(a, stream);
    else launch_topk<1, false>(a, stream);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
