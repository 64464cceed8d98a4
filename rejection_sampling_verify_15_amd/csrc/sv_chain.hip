// Chain verification: the acceptance stage of one speculative-decoding round
// for a batch of requests (Leviathan et al.'s Algorithm 1 as restated in the
// close-reading notes 02, section 4, and CMU 15-779 lecture 17 notes, sections
// 2.2-2.4).  See include/specverify.h for the contract.
//
// Two launches on the caller's stream:
//
//  1. chain_row_stats  one workgroup per (request, row, chunk) of kChunk
//                      logits, request-major: the chunk max and, for sampling
//                      rows, the fp32 sum of exp2((x - max) * log2e / T); for
//                      greedy rows the argmax (lowest index).  The workgroup
//                      whose chunk holds a row's draft token also hands over
//                      that logit.  Draft rows of greedy requests are not
//                      read.  The last workgroup of a request to finish
//                      merges the request's partials in fp64, runs the
//                      gamma-step test (u <= tau, tau = 1 if q <= p else p / q;
//                      greedy: argmax equality), writes the accepted tokens
//                      and the count, and for a sampling request leaves the
//                      pending final draw for launch 2.  Early requests are
//                      decided while later ones still stream.
//  2. chain_units      one workgroup per (sampling request, draw unit) of
//                      kThreads * kPer logits: fp64 sums of exp((x - max) / T)
//                      of the draw's target and draft rows over the unit (all,
//                      and where p > q).  The last unit of a request to finish
//                      does the draw: fp64 normalisers, the residual (or bonus)
//                      weight of every unit, and an fp64 block scan of the
//                      crossing unit -- the smallest k with C_k > u * W.
//
// Whoever finishes last also returns the workspace words it consumed to zero.
//
// Precision: the accept test needs p(x)/q(x) to ~1e-6 and uses the fp32 chunk
// sums merged in fp64; the final draw uses fp64 exponentials and fp64
// normalisers summed in launch 2, so the inverse CDF matches an fp64
// reference except where u lies within a few ulps of a CDF step.
#include <stdlib.h>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
struct RowPartial {  // one (row, chunk), handed over as one 64-bit word
  float m;           // chunk max
  int32_t v;         // float bits of the exp-sum (sampling) or the argmax (greedy)
};

// Per (request, draw unit), fp64: sums over the unit of the target (t) and
// draft (d) exponentials, over all tokens and over the tokens with p > q.
enum : int { kUnitAllT = 0, kUnitAllD = 1, kUnitPosT = 2, kUnitPosD = 3, kUnitFields = 4 };
struct UnitRec {
  double f[kUnitFields];
};

// A sampling request's final draw, decided in launch 1 and drawn in launch 2.
struct Pending {
  int32_t valid;  // 1 while a draw is pending
  int32_t n;      // accepted drafts; the draw fills out_tokens[b][n]
  int32_t mode;   // kModeResidual / kModeBonus
  float u;        // u[b][gamma]
  float t;        // temperature
  float mt, md;   // maxima of the draw's target row and of draft row n
  int32_t pad;
  double zt, zd;  // their fp64-merged pass-1 normalisers
};

// A drawing request's Pending record travels to its units as kWireWords
// 64-bit words, each holding one 32-bit word of the record and, above it, the
// record's `valid` value.  The decider stores all words at once with
// device-coherent stores, in no particular order; a unit takes the record once
// every word it reads carries a nonzero mark.
constexpr int kWireWords = sizeof(Pending) / 4;
struct PendingWire {
  uint64_t w[kWireWords];
};

static_assert(sizeof(RowPartial) == 8, "row partials are one 64-bit word");
static_assert(sizeof(UnitRec) % 8 == 0 && sizeof(Pending) % 8 == 0, "records are cleared in 64-bit words");

enum : int32_t { kModeResidual = 1, kModeBonus = 2 };
enum : int32_t { kPendingDraw = 1, kPendingNone = 2 };  // Pending::valid once published

constexpr int kCounterStride = 32;  // uint32 words per request: one 128-byte line
constexpr int kUnitCounter = 0;     // draw units of the request that have counted in

struct ChainArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;
  int B, gamma, V, nchunk, nunit;
  int32_t* out_tokens;
  int32_t* out_n;
  RowPartial* partials;  // [B][2*gamma+1][nchunk]
  float* gathers;        // [B][2*gamma+1] logit of the draft token in each row
  PendingWire* pending;  // [B]
  UnitRec* units;        // [B][nunit]
  uint32_t* counters;    // [B][kCounterStride]
};

// T must be 0 (greedy) or a finite positive normal float.
__device__ inline bool temp_ok(float t) { return isfinite(t) && (t == 0.0f || t >= 1.17549435e-38f); }

template <int DT>
__device__ inline const void* row_ptr(const void* base, size_t row, int V) {
  return static_cast<const char*>(base) + row * static_cast<size_t>(V) * Elem<DT>::kBytes;
}

// exp((x - m) / T) for x <= m, in fp64, given l2t = log2(e) / T (the
// difference is taken in fp64, so it is exact for fp32 logits too).
__device__ inline double exp_scaled(float x, float m, double l2t) {
  return exp2_nonpos((static_cast<double>(x) - static_cast<double>(m)) * l2t);
}

// The same with the LDS table of the calling workgroup.
__device__ inline double exp_scaled(float x, float m, double l2t, const Exp2Table& tab) {
  return exp2_tab((static_cast<double>(x) - static_cast<double>(m)) * l2t, tab);
}

// Request classes: 0 samples with its draft rows or has gamma == 0 (it has a
// final draw), 1 is greedy or cannot sample (target rows only), 2 has an
// invalid temperature.
__device__ inline int request_class(const ChainArgs& a, float T) {
  if (!temp_ok(T)) return 2;
  if (T > 0.0f && (a.draft != nullptr || a.gamma == 0)) return 0;
  return 1;
}

// Rows of a request that are read: target rows, plus draft rows when sampling.
__device__ inline int needed_rows(const ChainArgs& a, float T) {
  return (T > 0.0f && a.draft != nullptr) ? 2 * a.gamma + 1 : a.gamma + 1;
}


// Thread t < kWireWords of the calling workgroup stores word t.
__device__ inline void publish_pending(PendingWire* wire, const Pending& d) {
  const int t = threadIdx.x;
  if (t < kWireWords) {
    struct Dwords { uint32_t v[kWireWords]; };
    const Dwords src = __builtin_bit_cast(Dwords, d);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < kWireWords; ++i)
      if (t == i) v = src.v[i];  // constant indices keep the record in registers
    const uint64_t mark = static_cast<uint64_t>(static_cast<uint32_t>(d.valid)) << 32;
    store_coherent(&wire->w[t], mark | v);
  }
}

// Upper bound on the polls of a unit waiting for its request's decision
// (about 2 s); the decision is always made by workgroups dispatched before the
// waiting one, so the bound only guards against a broken dispatch order.
constexpr uint32_t kSpinLimit = 1u << 22;

// Waits (thread 0 polls, the workgroup then reads the copy in LDS) until the
// decision of request b is published and returns it; valid = 0 means the
// wait gave up.
__device__ Pending wait_pending(const ChainArgs& a, int b) {
  __shared__ Pending s_p;
  if (threadIdx.x == 0) {
    const PendingWire* wire = a.pending + b;
    struct Dwords { uint32_t v[kWireWords]; };
    Dwords got{};
    bool whole = false;
    for (uint32_t spin = 0; !whole && spin < kSpinLimit; ++spin) {
      if ((load_coherent(&wire->w[0]) >> 32) != 0) {
        asm volatile("" ::: "memory");
        whole = true;
#pragma unroll
        for (int i = 0; i < kWireWords; ++i) {
          const uint64_t w = load_coherent(&wire->w[i]);
          whole = whole && (w >> 32) != 0;
          got.v[i] = static_cast<uint32_t>(w);
        }
      }
      if (!whole) __builtin_amdgcn_s_sleep(8);
    }
    Pending d = __builtin_bit_cast(Pending, got);
    if (!whole) d.valid = 0;
    s_p = d;
  }
  __syncthreads();
  const Pending d = s_p;
  __syncthreads();
  return d;
}

__device__ void write_invalid(const ChainArgs& a, int b) {
  const int G = a.gamma;
  for (int i = threadIdx.x; i <= G; i += kThreads) a.out_tokens[static_cast<size_t>(b) * (G + 1) + i] = -1;
  if (threadIdx.x == 0) a.out_n[b] = -1;
}

// ---------------------------------------------------------------------------
// the decision of request b
// ---------------------------------------------------------------------------
// Merges the request's chunk partials in fp64: one thread per group of chunks
// of a row takes the group max, then rescales every chunk sum to it (all
// exponentials independent of each other); one thread per row combines the
// groups the same way.  Then the drafts are tested in order; tokens [0, n]
// (all but a sampling request's slot n) and the count are written, a
// drawing request's outcome is published to its units, and the partials and
// gathered logits return to zero.
template <int DT>
__device__ void decide_and_publish(const ChainArgs& a, int b, const Exp2Table& tab) {
  constexpr int kMaxRows = 2 * SV_MAX_GAMMA + 1;
  __shared__ float s_gm[kThreads];
  __shared__ double s_gz[kThreads];
  __shared__ int32_t s_garg[kThreads];
  __shared__ float s_m[kMaxRows];
  __shared__ double s_z[kMaxRows];
  __shared__ int32_t s_arg[kMaxRows];
  __shared__ float s_xt[SV_MAX_GAMMA], s_xd[SV_MAX_GAMMA];
  __shared__ int32_t s_ok[SV_MAX_GAMMA];
  __shared__ int32_t s_n;
  __shared__ Pending s_pend;
  const int tid = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  const bool sampling = T > 0.0f;
  const double l2t = sampling ? kLog2e / static_cast<double>(T) : 0.0;
  const int nrows = needed_rows(a, T);
  // one round of loads: the chunk partials (in groups of chunks, one group per
  // thread), the draft tokens, their gathered logits and the uniforms
  const int gpr = max(1, min((a.nchunk + 3) / 4, kThreads / nrows));  // groups per row
  const int gs = (a.nchunk + gpr - 1) / gpr;                           // chunks per group
  int bad = 0;
  if (tid < G) {
    const int32_t x = a.tokens[static_cast<size_t>(b) * G + tid];
    bad |= (x < 0 || x >= a.V);
    if (sampling && a.draft != nullptr) {
      s_xt[tid] = a.gathers[static_cast<size_t>(b) * R + tid];
      s_xd[tid] = a.gathers[static_cast<size_t>(b) * R + G + 1 + tid];
    }
  }
  if (sampling && tid <= G) {
    const float u = a.uniforms[static_cast<size_t>(b) * (G + 1) + tid];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  if (sampling && G > 0 && a.draft == nullptr) bad = 1;
  if (tid < nrows * gpr) {
    const int r = tid / gpr;
    const int g = tid % gpr;
    const RowPartial* p = a.partials + (static_cast<size_t>(b) * R + r) * a.nchunk;
    const int cb = g * gs;
    const int ce = min(a.nchunk, cb + gs);
    float m = -INFINITY;
    double z = 0.0;
    ArgMax best{-INFINITY, 0x7fffffff};
    for (int c0 = cb; c0 < ce; c0 += 4) {
      RowPartial w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = p[min(c0 + i, ce - 1)];
      if (!sampling) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + i < ce) best = argmax_combine(best, ArgMax{w[i].m, w[i].v});
      } else {
        float m4 = m;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + i < ce) m4 = fmaxf(m4, w[i].m);
        if (m4 != -INFINITY) {
          double z4 = (m != -INFINITY) ? z * exp_scaled(m, m4, l2t, tab) : 0.0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c0 + i < ce && w[i].m != -INFINITY)
              z4 += static_cast<double>(__int_as_float(w[i].v)) * exp_scaled(w[i].m, m4, l2t, tab);
          m = m4;
          z = z4;
        }
      }
    }
    if (sampling) {
      s_gm[tid] = m;
      s_gz[tid] = z;
    } else {
      s_gm[tid] = best.v;
      s_garg[tid] = best.i;
    }
  }
  bad = __syncthreads_or(bad);
  if (!bad) {
    // combine the groups of each row
    if (tid < nrows) {
      if (!sampling) {
        ArgMax best{-INFINITY, 0x7fffffff};
        for (int g = 0; g < gpr; ++g)
          best = argmax_combine(best, ArgMax{s_gm[tid * gpr + g], s_garg[tid * gpr + g]});
        s_m[tid] = best.v;
        s_arg[tid] = best.i;
      } else {
        float m = -INFINITY;
        for (int g = 0; g < gpr; ++g) m = fmaxf(m, s_gm[tid * gpr + g]);
        double z = 0.0;
        for (int g = 0; g < gpr; ++g) {
          const float gm = s_gm[tid * gpr + g];
          if (gm != -INFINITY) z += s_gz[tid * gpr + g] * exp_scaled(gm, m, l2t, tab);
        }
        s_m[tid] = m;
        s_z[tid] = z;
      }
    }
    __syncthreads();
    if (tid < G) {
      const int32_t x = a.tokens[static_cast<size_t>(b) * G + tid];
      int ok;
      if (!sampling) {
        ok = (x == s_arg[tid]);
      } else {
        const double p = exp_scaled(s_xt[tid], s_m[tid], l2t, tab) / s_z[tid];
        const double q = exp_scaled(s_xd[tid], s_m[G + 1 + tid], l2t, tab) / s_z[G + 1 + tid];
        const double tau = (q <= p) ? 1.0 : p / q;
        const double u = static_cast<double>(a.uniforms[static_cast<size_t>(b) * (G + 1) + tid]);
        ok = (u <= tau);
      }
      s_ok[tid] = ok;
    }
    __syncthreads();
    if (tid == 0) {
      int n = 0;
      while (n < G && s_ok[n]) ++n;
      s_n = n;
      if (sampling) {
        Pending d{};
        d.valid = kPendingDraw;
        d.n = n;
        d.mode = n < G ? kModeResidual : kModeBonus;
        d.u = a.uniforms[static_cast<size_t>(b) * (G + 1) + G];
        d.t = T;
        d.mt = s_m[n];
        d.zt = s_z[n];
        if (n < G) {
          d.md = s_m[G + 1 + n];
          d.zd = s_z[G + 1 + n];
        }
        s_pend = d;
      }
    }
  }
  if (tid == 0 && bad) {
    Pending d{};
    d.valid = kPendingNone;
    s_pend = d;
  }
  __syncthreads();
  // a request with draw units hears the outcome in every case: the draw, or
  // that there is none
  if (request_class(a, T) == 0) publish_pending(a.pending + b, s_pend);
  // outputs: tokens [0, n), greedy: the argmax at slot n, the rest -1; slot n
  // of a sampling request is filled by its draw
  int32_t* out = a.out_tokens + static_cast<size_t>(b) * (G + 1);
  const int n = bad ? -1 : s_n;
  for (int i = tid; i <= G; i += kThreads) {
    int32_t v = -1;
    if (!bad) {
      if (sampling && i == n) continue;
      if (i < n) v = a.tokens[static_cast<size_t>(b) * G + i];
      else if (i == n) v = s_arg[n];
    }
    out[i] = v;
  }
  if (tid == 0) a.out_n[b] = n;
  // the workspace words of this request back to zero
  unsigned long long* pz = reinterpret_cast<unsigned long long*>(a.partials + static_cast<size_t>(b) * R * a.nchunk);
  for (int i = tid; i < nrows * a.nchunk; i += kThreads) pz[i] = 0ull;
  if (tid < R) a.gathers[static_cast<size_t>(b) * R + tid] = 0.0f;
}

// ---------------------------------------------------------------------------
// launch 1: streaming row statistics
// ---------------------------------------------------------------------------
// Persistent workgroups (as many as fit on the GPU) stride over the items
// (request, row, chunk) in request-major order.  Each keeps two items in
// flight: the loads of the next item are issued before the current one is
// reduced, and the reductions synchronise through LDS only, so the prefetch
// stays outstanding.  Per item: the chunk max and, for sampling rows, the fp32
// sum of exp2((x - max) * log2e / T); for greedy rows the argmax (lowest
// index); the chunk holding a row's draft token also stores that logit.  Rows
// that no decision needs (draft rows of greedy requests, requests with an
// invalid temperature) are skipped.

// Row chunk of one streaming item, and so of one row partial.
constexpr int kRowChunk = 4096;
__host__ __device__ inline int row_chunks(int V) { return (V + kRowChunk - 1) / kRowChunk; }

// Which rows of each request are streamed, 2 bits per request, kept in LDS.
constexpr int kMaxStreamBatch = SV_MAX_BATCH;
enum : uint32_t { kStreamTarget = 1u, kStreamDraft = 2u };

struct StreamFlags {
  uint32_t w[kMaxStreamBatch / 16];
  __device__ inline uint32_t get(int b) const { return (w[b >> 4] >> ((b & 15) * 2)) & 3u; }
};

template <int DT, bool VEC, int NT>
struct StreamItem {
  using Raw = RawSlice<DT, VEC, kRowChunk / (NT * (VEC ? Elem<DT>::kVec : 1)), NT>;
  Raw raw;
  float t;      // temperature of the request
  int32_t tok;  // draft token of the row (sampling rows below gamma), else -1
};

// Item order: request-major, rows (target 0..gamma, then draft), then chunks.
struct RowItem {
  int b, k, c;
};
__device__ inline RowItem decode_item(const ChainArgs& a, long long item) {
  const int per_req = (2 * a.gamma + 1) * a.nchunk;
  const int rem = static_cast<int>(item % per_req);
  return RowItem{static_cast<int>(item / per_req), rem / a.nchunk, rem % a.nchunk};
}

__device__ inline bool stream_needed(const ChainArgs& a, const StreamFlags& fl, long long item) {
  const RowItem r = decode_item(a, item);
  const int b = r.b, k = r.k;
  const uint32_t f = fl.get(b);
  return k <= a.gamma ? (f & kStreamTarget) != 0 : (f & kStreamDraft) != 0;
}

__device__ inline long long stream_next(const ChainArgs& a, const StreamFlags& fl, long long item, long long items) {
  while (item < items && !stream_needed(a, fl, item)) item += gridDim.x;
  return item;
}

template <int DT, bool VEC, int NT>
__device__ inline void stream_issue(const ChainArgs& a, long long item, StreamItem<DT, VEC, NT>& it) {
  const int G = a.gamma;
  const RowItem r = decode_item(a, item);
  const int b = r.b, k = r.k, c = r.c;
  const int pos = k <= G ? k : k - G - 1;
  const void* row = (k <= G) ? row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + k, a.V)
                             : row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + pos, a.V);
  const int c0 = c * kRowChunk;
  it.raw.load(row, c0, min(a.V, c0 + kRowChunk));
  it.t = a.temperature[b];
  it.tok = pos < G ? a.tokens[static_cast<size_t>(b) * G + pos] : -1;
}

// NT == kWave: one wave per workgroup, reductions within the wave only;
// otherwise the waves combine through LDS.
template <int DT, bool VEC, int NT>
__device__ inline void stream_reduce(const ChainArgs& a, long long item, const StreamItem<DT, VEC, NT>& it) {
  using Raw = typename StreamItem<DT, VEC, NT>::Raw;
  __shared__ float s_a[kWaves];
  __shared__ int s_i[kWaves];
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const RowItem r = decode_item(a, item);
  const int b = r.b, k = r.k, c = r.c;
  const int c0 = c * kRowChunk;
  const int c1 = min(a.V, c0 + kRowChunk);
  const bool sampling = it.t > 0.0f;
  auto val = [&](int j, int e) -> float { return it.raw.at(j, e); };
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
    for (int e = 0; e < Raw::kPer; ++e) m = fmaxf(m, val(j, e));
  const int w = threadIdx.x / kWave;
  const bool lane0 = (threadIdx.x % kWave) == 0;
  float out_m;
  int32_t out_v;
  if (!sampling) {
    // chunk max first; only the lanes holding it look for its lowest index
    const float wm = wave_max(m);
    float bm = wm;
    if constexpr (NT != kWave) {
      if (lane0) s_a[w] = wm;
      lds_barrier();
      bm = s_a[0];
#pragma unroll
      for (int i = 1; i < NT / kWave; ++i) bm = fmaxf(bm, s_a[i]);
    }
    int idx = 0x7fffffff;
    if (m == bm) {
#pragma unroll
      for (int j = Raw::kItems - 1; j >= 0; --j)
#pragma unroll
        for (int e = Raw::kPer - 1; e >= 0; --e) {
          const int kk = Raw::index(c0, j, e);
          if (kk < c1 && it.raw.at(j, e) == bm) idx = kk;
        }
    }
    int bi = wave_min(idx);
    if constexpr (NT != kWave) {
      lds_barrier();  // s_a has been read
      if (lane0) s_i[w] = bi;
      lds_barrier();
      bi = s_i[0];
#pragma unroll
      for (int i = 1; i < NT / kWave; ++i) bi = min(bi, s_i[i]);
    }
    out_m = bm;
    out_v = bi;
  } else {
    const float sc = 1.4426950408889634f / it.t;
    float z = 0.0f;
    if (m != -INFINITY) {
      const float msc = m * sc;
#pragma unroll
      for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
        for (int e = 0; e < Raw::kPer; ++e) z += __builtin_amdgcn_exp2f(__builtin_fmaf(val(j, e), sc, -msc));
    }
    MaxSum r = wave_maxsum(MaxSum{m, z}, sc);
    if constexpr (NT != kWave) {
      if (lane0) {
        s_a[w] = r.m;
        s_i[w] = __float_as_int(r.z);
      }
      lds_barrier();
      r = MaxSum{s_a[0], __int_as_float(s_i[0])};
#pragma unroll
      for (int i = 1; i < NT / kWave; ++i) r = maxsum_combine(r, MaxSum{s_a[i], __int_as_float(s_i[i])}, sc);
    }
    out_m = r.m;
    out_v = __float_as_int(r.z);
  }
  if (it.tok >= c0 && it.tok < c1) {  // the lane holding the draft token stores its logit
#pragma unroll
    for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
      for (int e = 0; e < Raw::kPer; ++e)
        if (Raw::index(c0, j, e) == it.tok) a.gathers[static_cast<size_t>(b) * R + k] = it.raw.at(j, e);
  }
  if (threadIdx.x == 0) {
    RowPartial p;
    p.m = out_m;
    p.v = out_v;
    a.partials[(static_cast<size_t>(b) * R + k) * a.nchunk + c] = p;
  }
  if constexpr (NT != kWave) lds_barrier();  // s_a / s_i are reused by the next item
}

// The last chunk of a row: words past the row's end (loaded from a clamped
// address) become -inf before the reduction.  Vector groups lie wholly inside
// or outside the row (V is a multiple of the vector width on that path).
template <int DT, bool VEC, int NT>
__device__ inline void stream_reduce_any(const ChainArgs& a, long long item, StreamItem<DT, VEC, NT>& it) {
  using Raw = typename StreamItem<DT, VEC, NT>::Raw;
  const int c0 = decode_item(a, item).c * kRowChunk;
  const int c1 = min(a.V, c0 + kRowChunk);
  if (c1 - c0 != Raw::kSpan) {
    constexpr uint32_t kNegInf = DT == 0 ? (VEC ? 0xff80ff80u : 0xff80u) : 0xff800000u;
#pragma unroll
    for (int j = 0; j < Raw::kItems; ++j)
      if (Raw::index(c0, j, 0) >= c1) {
#pragma unroll
        for (int q = 0; q < (VEC ? 4 : 1); ++q) it.raw.w[j][q] = kNegInf;
      }
  }
  stream_reduce<DT, VEC, NT>(a, item, it);
}

// One item per workgroup of one wave (no prefetch, no barriers): the grid
// covers every item.
constexpr int kOnceThreads = kWave;

template <int DT, bool VEC>
__global__ __launch_bounds__(kOnceThreads) void chain_stream_once(ChainArgs a) {
  constexpr int NT = kOnceThreads;
  const long long item = blockIdx.x;
  const RowItem r = decode_item(a, item);
  const int b = r.b, k = r.k;
  StreamItem<DT, VEC, NT> x;
  if (k <= a.gamma) {
    stream_issue<DT, VEC, NT>(a, item, x);  // target rows: the loads do not wait for the temperature
    if (!temp_ok(x.t)) return;
  } else {
    const float T = a.temperature[b];
    if (!(temp_ok(T) && T > 0.0f && a.draft != nullptr)) return;
    stream_issue<DT, VEC, NT>(a, item, x);
  }
  stream_reduce_any<DT, VEC, NT>(a, item, x);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_stream(ChainArgs a) {
  __shared__ StreamFlags s_flags;
  for (int i = threadIdx.x; i < (a.B + 15) / 16; i += kThreads) {
    uint32_t word = 0;
    for (int q = 0; q < 16; ++q) {
      const int b = i * 16 + q;
      if (b >= a.B) break;
      const float T = a.temperature[b];
      uint32_t f = 0;
      if (temp_ok(T)) f = kStreamTarget | ((T > 0.0f && a.draft != nullptr) ? kStreamDraft : 0u);
      word |= f << (q * 2);
    }
    s_flags.w[i] = word;
  }
  __syncthreads();
  const long long items = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  long long ia = stream_next(a, s_flags, blockIdx.x, items);
  if (ia >= items) return;
  StreamItem<DT, VEC, kThreads> x, y;
  stream_issue<DT, VEC, kThreads>(a, ia, x);
  for (;;) {
    const long long ib = stream_next(a, s_flags, ia + gridDim.x, items);
    if (ib < items) stream_issue<DT, VEC, kThreads>(a, ib, y);
    stream_reduce_any<DT, VEC, kThreads>(a, ia, x);
    if (ib >= items) break;
    const long long ic = stream_next(a, s_flags, ib + gridDim.x, items);
    if (ic < items) stream_issue<DT, VEC, kThreads>(a, ic, x);
    stream_reduce_any<DT, VEC, kThreads>(a, ib, y);
    if (ic >= items) break;
    ia = ic;
  }
}

// ---------------------------------------------------------------------------
// launch 2: draw units, and the draw by the last unit of each request
// ---------------------------------------------------------------------------
// A draw unit is kUnitItems vector groups per thread: 2048 * kUnitItems logits
// on the bf16 vector path.
constexpr int kUnitItems = 2;
template <int DT, bool VEC>
using UnitSlice = Slice<DT, VEC, kUnitItems>;

// Weight of a unit in the final draw (rzt, rzd: reciprocal normalisers).
__device__ inline double unit_weight(double pos_t, double pos_d, double all_t, bool residual,
                                     double rzt, double rzd) {
  return residual ? (pos_t * rzt - pos_d * rzd) : all_t;
}

__device__ inline double unit_field(const UnitRec* r, int f) { return load_coherent_f64(&r->f[f]); }

// The draw of request b from its unit records: fp64 normalisers, the weight W
// of the draw (residual mass, or the target normaliser for a bonus draw), the
// unit where the running weight first exceeds u * W, then an fp64 block scan
// of that unit's logits for the token.
template <int DT, bool VEC>
__device__ void draw_token(const ChainArgs& a, int b, const Pending& d, const Exp2Table& tab) {
  using S = UnitSlice<DT, VEC>;
  __shared__ int s_unit, s_first, s_lastpos, s_hit, s_lasttok;
  __shared__ double s_before;
  // the last unit of a request draws while other units still compute: let
  // its waves issue first on their SIMDs
  __builtin_amdgcn_s_setprio(3);
  const int G = a.gamma;
  const int tid = threadIdx.x;
  const UnitRec* ur = a.units + static_cast<size_t>(b) * a.nunit;
  // 1) one round of loads; with at most kThreads units (the usual case) each
  //    thread keeps its unit's sums in registers for the scan below
  const bool one_batch = a.nunit <= kThreads;
  double mine[kUnitFields] = {0.0, 0.0, 0.0, 0.0};
  double tot[kUnitFields] = {0.0, 0.0, 0.0, 0.0};
  for (int i = tid; i < a.nunit; i += kThreads) {
#pragma unroll
    for (int f = 0; f < kUnitFields; ++f) {
      const double v = unit_field(ur + i, f);
      tot[f] += v;
      if (one_batch) mine[f] = v;
    }
  }
  block_sum_doubles<kUnitFields>(tot);
  // p = e_t / zt and q = e_d / zd are formed with the reciprocals throughout
  const double rzt = 1.0 / tot[kUnitAllT], rzd = 1.0 / tot[kUnitAllD];
  // an empty residual (p and q equal up to rounding) draws from p of that
  // position instead
  const bool residual = d.mode == kModeResidual && (tot[kUnitPosT] * rzt - tot[kUnitPosD] * rzd > 0.0);
  auto weight_of = [&](int i) -> double {
    if (one_batch) return unit_weight(mine[kUnitPosT], mine[kUnitPosD], mine[kUnitAllT], residual, rzt, rzd);
    return unit_weight(unit_field(ur + i, kUnitPosT), unit_field(ur + i, kUnitPosD),
                       unit_field(ur + i, kUnitAllT), residual, rzt, rzd);
  };
  double W;
  {
    double ws[1] = {0.0};
    for (int i = tid; i < a.nunit; i += kThreads) ws[0] += weight_of(i);
    block_sum_doubles<1>(ws);
    W = ws[0];
  }
  const double target = static_cast<double>(d.u) * W;
  // 2) crossing unit: block scan of the unit weights in unit order
  if (tid == 0) { s_unit = -1; s_lastpos = -1; }
  __syncthreads();
  double carry = 0.0;
  for (int base = 0; base < a.nunit; base += kThreads) {
    const int i = base + tid;
    const double wu = i < a.nunit ? weight_of(i) : 0.0;
    double total;
    const double before = carry + block_exclusive_scan(wu, &total);
    if (tid == 0) s_first = 0x7fffffff;
    __syncthreads();
    const int lp = wave_max_int((i < a.nunit && wu > 0.0) ? i : -1);
    const int fi = wave_min((i < a.nunit && before + wu > target) ? i : 0x7fffffff);
    if ((tid % kWave) == 0) {
      atomicMax(&s_lastpos, lp);
      atomicMin(&s_first, fi);
    }
    __syncthreads();
    if (s_first != 0x7fffffff && i == s_first) {
      s_unit = i;
      s_before = before;
    }
    __syncthreads();
    carry += total;
    if (s_unit >= 0) break;
  }
  if (s_unit < 0) {  // rounding left u * W at the very top: take the last positive unit
    const int lp = s_lastpos < 0 ? 0 : s_lastpos;
    double bsum[1] = {0.0};
    for (int i = tid; i < lp; i += kThreads) bsum[0] += weight_of(i);
    block_sum_doubles<1>(bsum);
    if (tid == 0) { s_unit = lp; s_before = bsum[0]; }
    __syncthreads();
  }
  // 3) fp64 block scans of the crossing unit, one per vector group (group j
  //    of all threads precedes group j + 1); thread t owns kPer logits of each
  const int c0 = s_unit * S::kSpan;
  const int c1 = min(a.V, c0 + S::kSpan);
  const double l2t = kLog2e / static_cast<double>(d.t);
  const int trow = d.mode == kModeResidual ? d.n : G;
  S st;
  st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow, a.V), c0, c1);
  S sd;
  if (residual) sd.load(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V), c0, c1);
  if (tid == 0) { s_hit = 0x7fffffff; s_lasttok = -1; }
  int hit = 0x7fffffff;
  int last_pos = -1;
  double run0 = s_before;
#pragma unroll
  for (int j = 0; j < S::kItems; ++j) {
    double wk[S::kPer];
    if (residual) {
#pragma unroll
      for (int e = 0; e < S::kPer; ++e)
        wk[e] = fmax(0.0, exp_scaled(st.x[j][e], d.mt, l2t, tab) * rzt - exp_scaled(sd.x[j][e], d.md, l2t, tab) * rzd);
    } else {
#pragma unroll
      for (int e = 0; e < S::kPer; ++e) wk[e] = exp_scaled(st.x[j][e], d.mt, l2t, tab);
    }
    double own = 0.0;
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) {
      own += wk[e];
      if (wk[e] > 0.0) last_pos = S::index(c0, j, e);
    }
    double total;
    double run = run0 + block_exclusive_scan(own, &total);
    run0 += total;
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) {
      run += wk[e];
      if (hit == 0x7fffffff && wk[e] > 0.0 && run > target) hit = S::index(c0, j, e);
    }
  }
  hit = wave_min(hit);
  last_pos = wave_max_int(last_pos);
  if ((tid % kWave) == 0) {
    atomicMin(&s_hit, hit);
    atomicMax(&s_lasttok, last_pos);
  }
  __syncthreads();
  if (tid == 0)
    a.out_tokens[static_cast<size_t>(b) * (G + 1) + d.n] = (s_hit != 0x7fffffff) ? s_hit : s_lasttok;
  __syncthreads();
  __builtin_amdgcn_s_setprio(0);
}

// Requests for unit items: with few requests, unit items are handed out only
// to the requests that can have a final draw (class 0), in request order, so
// that greedy and invalid requests occupy no workgroups; otherwise request =
// item / nunit.  The ranking reads only the temperatures, which no workgroup
// changes (the pending records are cleared as draws finish).
constexpr int kCompactMaxBatch = 256;

// The p-th class-0 request (0-based, request order), or -1.
__device__ int nth_drawing_request(const ChainArgs& a, int p) {
  __shared__ int s_cnt[kWaves];
  __shared__ int s_b;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int w = tid / kWave;
  if (tid == 0) s_b = -1;
  const int i = tid;
  const bool v = i < a.B && request_class(a, a.temperature[i]) == 0;
  const uint64_t m = __ballot(v);
  if (lane == 0) s_cnt[w] = __popcll(m);
  __syncthreads();
  int before = __popcll(m & ((1ull << lane) - 1ull));
#pragma unroll
  for (int k = 0; k < kWaves; ++k)
    if (k < w) before += s_cnt[k];
  if (v && before == p) s_b = i;
  __syncthreads();
  return s_b;
}

// Unit `unit` of request b (a class-0 request): waits for the decision, then
// adds its share of the final draw and counts itself in; the last unit of the
// request draws and returns the request's draw records to zero.
template <int DT, bool VEC>
__device__ void unit_work(const ChainArgs& a, int b, int unit, const Exp2Table& tab) {
  using S = UnitSlice<DT, VEC>;
  __shared__ double s_w[4][kWaves];
  __shared__ int s_last;
  const int G = a.gamma;
  const Pending d = wait_pending(a, b);
  if (d.valid == 0 && threadIdx.x == 0) a.out_n[b] = -1;  // gave up waiting
  const bool draw = d.valid == kPendingDraw;
  UnitRec* rec = a.units + static_cast<size_t>(b) * a.nunit + unit;
  if (draw) {
    const double l2t = kLog2e / static_cast<double>(d.t);
    const int c0 = unit * S::kSpan;
    const int c1 = min(a.V, c0 + S::kSpan);
    const bool residual = d.mode == kModeResidual;
    const int trow = residual ? d.n : G;
    S st;
    st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow, a.V), c0, c1);
    double pos_t = 0.0, pos_d = 0.0, all_t = 0.0, all_d = 0.0;
    if (residual) {
      S sd;
      sd.load(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V), c0, c1);
#pragma unroll
      for (int j = 0; j < S::kItems; ++j)
#pragma unroll
        for (int e = 0; e < S::kPer; ++e) {
          const double et = exp_scaled(st.x[j][e], d.mt, l2t, tab);
          const double ed = exp_scaled(sd.x[j][e], d.md, l2t, tab);
          all_t += et;
          all_d += ed;
          if (et * d.zd > ed * d.zt) {  // p > q under the pass-1 normalisers
            pos_t += et;
            pos_d += ed;
          }
        }
    } else {
#pragma unroll
      for (int j = 0; j < S::kItems; ++j)
#pragma unroll
        for (int e = 0; e < S::kPer; ++e) all_t += exp_scaled(st.x[j][e], d.mt, l2t, tab);
    }
    pos_t = wave_sum(pos_t);
    pos_d = wave_sum(pos_d);
    all_t = wave_sum(all_t);
    all_d = wave_sum(all_d);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) {
      s_w[kUnitPosT][w] = pos_t;
      s_w[kUnitPosD][w] = pos_d;
      s_w[kUnitAllT][w] = all_t;
      s_w[kUnitAllD][w] = all_d;
    }
    __syncthreads();
    // wave 0 hands the record over (one field per lane)
    if (threadIdx.x < kUnitFields) {
      double v = 0.0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) v += s_w[threadIdx.x][i];
      store_coherent_f64(&rec->f[threadIdx.x], v);
    }
  }
  if (threadIdx.x == 0)
    s_last = arrive(a.counters + static_cast<size_t>(b) * kCounterStride + kUnitCounter) ==
             static_cast<uint32_t>(a.nunit - 1);
  __syncthreads();
  if (s_last) {
    if (draw) {
      draw_token<DT, VEC>(a, b, d, tab);
      unsigned long long* wz = reinterpret_cast<unsigned long long*>(a.units + static_cast<size_t>(b) * a.nunit);
      const int nw = a.nunit * static_cast<int>(sizeof(UnitRec) / 8);
      for (int i = threadIdx.x; i < nw; i += kThreads) wz[i] = 0ull;
    }
    if (threadIdx.x < kWireWords) a.pending[b].w[threadIdx.x] = 0ull;
    if (threadIdx.x == 0) store_coherent(a.counters + static_cast<size_t>(b) * kCounterStride + kUnitCounter, 0u);
  }
  __syncthreads();  // LDS is reused by the next item
}

// Unit item of the separate unit launch: with few requests the unit items go
// only to class-0 requests; otherwise request = item / nunit.
template <int DT, bool VEC>
__device__ void unit_item(const ChainArgs& a, long long item, const Exp2Table& tab) {
  const int unit = static_cast<int>(item % a.nunit);
  int b;
  if (a.B <= kCompactMaxBatch) {
    static_assert(kCompactMaxBatch <= kThreads, "one temperature per thread");
    b = nth_drawing_request(a, static_cast<int>(item / a.nunit));
    if (b < 0) return;
  } else {
    b = static_cast<int>(item / a.nunit);
    if (request_class(a, a.temperature[b]) != 0) return;
  }
  unit_work<DT, VEC>(a, b, unit, tab);
}


// ---------------------------------------------------------------------------
// launch 2: decisions, draw units and draws
// ---------------------------------------------------------------------------
// Blocks [0, B) decide request b.  The blocks after them are unit items, each
// waiting only for the decision of its own request, made by a lower-numbered
// block: workgroups are dispatched in block order, so that block is running
// or done and the wait ends.  With B <= kCompactMaxBatch the unit items go to
// the requests that draw, in request order, and the rest exit at once.
template <int DT>
__device__ void decide_request(const ChainArgs& a, int b, const Exp2Table& tab) {
  if (request_class(a, a.temperature[b]) == 2) write_invalid(a, b);  // nothing was streamed
  else decide_and_publish<DT>(a, b, tab);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_draw(ChainArgs a) {
  __shared__ Exp2Table tab;
  exp2_table_init(tab);
  __syncthreads();
  const long long blk = blockIdx.x;
  if (blk < a.B) decide_request<DT>(a, static_cast<int>(blk), tab);
  else unit_item<DT, VEC>(a, blk - a.B, tab);
}

// Very large shapes: decisions and units in launches of their own, each with
// a capped grid whose workgroups stride over the items (no unit waits: every
// decision is made by the time the unit launch starts).
template <int DT>
__global__ __launch_bounds__(kThreads) void chain_decide(ChainArgs a) {
  __shared__ Exp2Table tab;
  exp2_table_init(tab);
  __syncthreads();
  for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
    decide_request<DT>(a, b, tab);
    __syncthreads();
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_units(ChainArgs a) {
  __shared__ Exp2Table tab;
  exp2_table_init(tab);
  __syncthreads();
  const long long items = static_cast<long long>(a.B) * a.nunit;
  for (long long item = blockIdx.x; item < items; item += gridDim.x) unit_item<DT, VEC>(a, item, tab);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct ChainLayout {
  size_t partials, gathers, pending, units, counters, total;
};

static int units_for(int V, int kper) {
  const int span = kThreads * kper;
  return (V + span - 1) / span;
}

// Sized for the largest draw-unit count (scalar path: kThreads logits per unit).
static ChainLayout chain_layout(int B, int gamma, int V) {
  ChainLayout L{};
  const size_t nchunk = static_cast<size_t>(row_chunks(V));
  const size_t R = 2 * static_cast<size_t>(gamma) + 1;
  const size_t nunit = static_cast<size_t>(units_for(V, 1));
  size_t off = 0;
  L.partials = off; off = align_up(off + static_cast<size_t>(B) * R * nchunk * sizeof(RowPartial));
  L.gathers = off;  off = align_up(off + static_cast<size_t>(B) * R * sizeof(float));
  L.pending = off;  off = align_up(off + static_cast<size_t>(B) * sizeof(PendingWire));
  L.units = off;    off = align_up(off + static_cast<size_t>(B) * nunit * sizeof(UnitRec));
  L.counters = off; off = align_up(off + static_cast<size_t>(B) * kCounterStride * sizeof(uint32_t));
  L.total = off;
  return L;
}

// Grids of launch 2 in its split form are capped; their workgroups stride.
constexpr long long kMaxGrid = 1 << 20;

// Workgroups of chain_stream that fit on the current device at once.
template <int DT, bool VEC>
static long long stream_capacity() {
  static long long cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_stream<DT, VEC>, kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1)
      return 1024;
    cached[dev] = static_cast<long long>(per_cu) * cus;
  }
  return cached[dev];
}

// Test hook: a positive value in this environment variable caps every grid
// at that many workgroups and selects the split form of launch 2.
static long long test_grid_cap() {
  const char* v = getenv("SV_CHAIN_TEST_GRID_CAP");
  return v ? atoll(v) : 0;
}

template <int DT, bool VEC>
static int launch_chain(ChainArgs a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  a.nunit = units_for(a.V, UnitSlice<DT, VEC>::kPer * kUnitItems);
  const long long units = static_cast<long long>(a.B) * a.nunit;
  const long long cap = test_grid_cap();
  long long sg = stream_capacity<DT, VEC>();
  if (cap > 0 && cap < sg) sg = cap;
  if (getenv("SV_CHAIN_STREAM_PERSISTENT") != nullptr || items > kMaxGrid || cap > 0)
    launch(SV_K_CHAIN_STREAM, chain_stream<DT, VEC>, dim3(static_cast<unsigned>(items < sg ? items : sg)),
           dim3(kThreads), 0, stream, a);
  else
    launch(SV_K_CHAIN_STREAM, chain_stream_once<DT, VEC>, dim3(static_cast<unsigned>(items)), dim3(kOnceThreads), 0,
           stream, a);
  if (cap <= 0 && a.B + units <= kMaxGrid) {
    launch(SV_K_CHAIN_DRAW, chain_draw<DT, VEC>, dim3(static_cast<unsigned>(a.B + units)), dim3(kThreads), 0,
           stream, a);
  } else {
    const long long g = cap > 0 ? cap : kMaxGrid;
    launch(SV_K_CHAIN_DECIDE, chain_decide<DT>, dim3(static_cast<unsigned>(a.B < g ? a.B : g)), dim3(kThreads), 0,
           stream, a);
    launch(SV_K_CHAIN_UNITS, chain_units<DT, VEC>, dim3(static_cast<unsigned>(units < g ? units : g)),
           dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_chain_workspace_bytes(int B, int gamma, int V, int dtype) {
  (void)dtype;
  if (B < 0 || B > SV_MAX_BATCH || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB)
    return 0;
  return chain_layout(B, gamma, V).total;
}

extern "C" int spec_verify_chain(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 const float* temperature, int B, int gamma, int V, int dtype,
                                 int32_t* out_tokens, int32_t* out_num_accepted,
                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || B > SV_MAX_BATCH || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!target_logits || !temperature || !uniforms || !out_tokens || !out_num_accepted || !workspace)
    return SV_ERR_NULL;
  if (gamma > 0 && !draft_tokens) return SV_ERR_NULL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || (draft_logits && !aligned(draft_logits, es))) return SV_ERR_ALIGN;
  const ChainLayout L = chain_layout(B, gamma, V);
  if (workspace_bytes < L.total || !aligned(workspace, 256)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  ChainArgs a{};
  a.target = target_logits;
  a.draft = gamma > 0 ? draft_logits : nullptr;
  a.tokens = draft_tokens;
  a.uniforms = uniforms;
  a.temperature = temperature;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.nchunk = row_chunks(V);
  a.out_tokens = out_tokens;
  a.out_n = out_num_accepted;
  a.partials = reinterpret_cast<RowPartial*>(ws + L.partials);
  a.gathers = reinterpret_cast<float*>(ws + L.gathers);
  a.pending = reinterpret_cast<PendingWire*>(ws + L.pending);
  a.units = reinterpret_cast<UnitRec*>(ws + L.units);
  a.counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_chain<0, true>(a, stream) : launch_chain<0, false>(a, stream);
  return vec ? launch_chain<1, true>(a, stream) : launch_chain<1, false>(a, stream);
}
