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

static_assert(sizeof(RowPartial) == 8, "row partials are one 64-bit word");
static_assert(sizeof(UnitRec) % 8 == 0 && sizeof(Pending) % 8 == 0, "records are cleared in 64-bit words");

enum : int32_t { kModeResidual = 1, kModeBonus = 2 };

constexpr int kCounterStride = 32;  // uint32 words per request: one 128-byte line
constexpr int kRowCounter = 0;      // row-statistics workgroups arrived (launch 1)
constexpr int kUnitCounter = 16;    // draw units arrived (launch 2)

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
  Pending* pending;      // [B]
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

__device__ inline uint64_t pack_partial(float m, int32_t v) {
  return static_cast<uint64_t>(__float_as_uint(m)) | (static_cast<uint64_t>(static_cast<uint32_t>(v)) << 32);
}

__device__ inline RowPartial load_partial(const RowPartial* p) {
  const uint64_t w = load_coherent(reinterpret_cast<const uint64_t*>(p));
  return RowPartial{__uint_as_float(static_cast<uint32_t>(w)), static_cast<int32_t>(w >> 32)};
}

__device__ void write_invalid(const ChainArgs& a, int b) {
  const int G = a.gamma;
  for (int i = threadIdx.x; i <= G; i += kThreads) a.out_tokens[static_cast<size_t>(b) * (G + 1) + i] = -1;
  if (threadIdx.x == 0) a.out_n[b] = -1;
}

// ---------------------------------------------------------------------------
// the decision of request b, made by the last row-statistics workgroup
// ---------------------------------------------------------------------------
// Merges the request's chunk partials (fp64, online rescaling), tests the
// drafts in order, writes tokens [0, n] (all but a sampling request's slot
// n) and the count, records a sampling request's pending draw, and zeroes the
// partials, gathered logits and counter.
template <int DT>
__device__ void decide_and_publish(const ChainArgs& a, int b) {
  constexpr int kMaxRows = 2 * SV_MAX_GAMMA + 1;
  // one workgroup per request does this while others stream: let its waves
  // issue first on their SIMDs
  __builtin_amdgcn_s_setprio(3);
  __shared__ float s_gm[kThreads];
  __shared__ double s_gz[kThreads];
  __shared__ int32_t s_garg[kThreads];
  __shared__ float s_m[kMaxRows];
  __shared__ double s_z[kMaxRows];
  __shared__ int32_t s_arg[kMaxRows];
  __shared__ float s_xt[SV_MAX_GAMMA], s_xd[SV_MAX_GAMMA];
  __shared__ int32_t s_ok[SV_MAX_GAMMA];
  __shared__ int32_t s_n;
  const int tid = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  const bool sampling = T > 0.0f;
  const double l2t = sampling ? kLog2e / static_cast<double>(T) : 0.0;
  const int nrows = needed_rows(a, T);
  const uint32_t* gathers = reinterpret_cast<const uint32_t*>(a.gathers) + static_cast<size_t>(b) * R;
  // one round of loads: the chunk partials (in groups of chunks, one group per
  // thread), the draft tokens, their gathered logits and the uniforms
  const int gpr = max(1, min((a.nchunk + 3) / 4, kThreads / nrows));  // groups per row
  const int gs = (a.nchunk + gpr - 1) / gpr;                           // chunks per group
  int bad = 0;
  if (tid < G) {
    const int32_t x = a.tokens[static_cast<size_t>(b) * G + tid];
    bad |= (x < 0 || x >= a.V);
    if (sampling && a.draft != nullptr) {
      s_xt[tid] = __uint_as_float(load_coherent(gathers + tid));
      s_xd[tid] = __uint_as_float(load_coherent(gathers + G + 1 + tid));
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
      for (int i = 0; i < 4; ++i) w[i] = load_partial(p + min(c0 + i, ce - 1));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c0 + i >= ce) continue;
        if (!sampling) {
          best = argmax_combine(best, ArgMax{w[i].m, w[i].v});
        } else if (w[i].m != -INFINITY) {
          if (w[i].m > m) {
            if (m != -INFINITY) z *= exp_scaled(m, w[i].m, l2t);
            m = w[i].m;
          }
          z += static_cast<double>(__int_as_float(w[i].v)) * exp_scaled(w[i].m, m, l2t);
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
          if (gm != -INFINITY) z += s_gz[tid * gpr + g] * exp_scaled(gm, m, l2t);
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
        const double p = exp_scaled(s_xt[tid], s_m[tid], l2t) / s_z[tid];
        const double q = exp_scaled(s_xd[tid], s_m[G + 1 + tid], l2t) / s_z[G + 1 + tid];
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
        d.valid = 1;
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
        a.pending[b] = d;
      }
    }
    __syncthreads();
  }
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
  if (tid == 0) store_coherent(a.counters + static_cast<size_t>(b) * kCounterStride + kRowCounter, 0u);
  __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// launch 1: row statistics
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void row_stats_item(const ChainArgs& a, long long item) {
  __shared__ float s_wm[kWaves];
  __shared__ float s_gather;
  __shared__ int s_last;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const int per_req = R * a.nchunk;
  const int b = static_cast<int>(item / per_req);
  const int rem = static_cast<int>(item % per_req);
  const int k = rem / a.nchunk;  // target rows 0..G, then draft rows
  const int c = rem % a.nchunk;
  const float T = a.temperature[b];
  const int cls = request_class(a, T);
  if (cls == 2) {  // nothing is read for this request
    if (k == 0 && c == 0) write_invalid(a, b);
    return;
  }
  const bool sampling = T > 0.0f;
  if (k > G && !(sampling && a.draft != nullptr)) return;  // draft rows are read only when sampling
  const int pos = k <= G ? k : k - G - 1;                    // draft position of this row
  const void* row = (k <= G) ? row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + k, a.V)
                             : row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + pos, a.V);
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  const int32_t tok = (sampling && pos < G) ? a.tokens[static_cast<size_t>(b) * G + pos] : -1;
  const bool has_gather = tok >= c0 && tok < c1;
  Slice<DT, VEC> s;
  s.load(row, c0, c1);
  if (has_gather) {
#pragma unroll
    for (int j = 0; j < s.kItems; ++j)
#pragma unroll
      for (int e = 0; e < s.kPer; ++e)
        if (s.index(c0, j, e) == tok) s_gather = s.x[j][e];
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < s.kItems; ++j)
#pragma unroll
    for (int e = 0; e < s.kPer; ++e) m = fmaxf(m, s.x[j][e]);
  float out_m;
  int32_t out_v;
  if (!sampling) {
    // chunk max first; only threads holding it look for its lowest index
    const float wm = wave_max(m);
    if ((threadIdx.x % kWave) == 0) s_wm[threadIdx.x / kWave] = wm;
    __syncthreads();
    float bm = s_wm[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) bm = fmaxf(bm, s_wm[i]);
    int idx = 0x7fffffff;
    if (m == bm) {
#pragma unroll
      for (int j = s.kItems - 1; j >= 0; --j)
#pragma unroll
        for (int e = s.kPer - 1; e >= 0; --e) {
          const int kk = s.index(c0, j, e);
          if (s.x[j][e] == bm && kk < c1) idx = kk;
        }
    }
    const ArgMax best = block_argmax(ArgMax{bm, idx});
    out_m = bm;
    out_v = best.i;
  } else {
    const float sc = 1.4426950408889634f / T;
    float z = 0.0f;
    if (m != -INFINITY) {
      const float msc = m * sc;
#pragma unroll
      for (int j = 0; j < s.kItems; ++j)
#pragma unroll
        for (int e = 0; e < s.kPer; ++e) z += __builtin_amdgcn_exp2f(__builtin_fmaf(s.x[j][e], sc, -msc));
    }
    const MaxSum ms = block_maxsum(MaxSum{m, z}, sc);
    out_m = ms.m;
    out_v = __float_as_int(ms.z);
  }
  // hand the partial (and the gathered logit) over; the last workgroup of the
  // request decides it
  if (threadIdx.x == 0) {
    store_coherent(reinterpret_cast<uint64_t*>(a.partials + (static_cast<size_t>(b) * R + k) * a.nchunk + c),
                   pack_partial(out_m, out_v));
    if (has_gather)
      store_coherent(reinterpret_cast<uint32_t*>(a.gathers) + static_cast<size_t>(b) * R + k,
                     __float_as_uint(s_gather));
    const uint32_t total = static_cast<uint32_t>(needed_rows(a, T) * a.nchunk);
    s_last = arrive(a.counters + static_cast<size_t>(b) * kCounterStride + kRowCounter) == total - 1;
  }
  __syncthreads();
  if (s_last) decide_and_publish<DT>(a, b);
  __syncthreads();  // LDS is reused by the next item
}

// LOOP: more items than workgroups, which stride over them.  Without the loop
// nothing is hoisted across items, which keeps the register count (and so the
// occupancy of the streaming part) where a single item needs it.
template <int DT, bool VEC, bool LOOP>
__global__ __launch_bounds__(kThreads) void chain_row_stats(ChainArgs a) {
  if constexpr (LOOP) {
    const long long items = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
    for (long long item = blockIdx.x; item < items; item += gridDim.x) row_stats_item<DT, VEC>(a, item);
  } else {
    row_stats_item<DT, VEC>(a, blockIdx.x);
  }
}

// ---------------------------------------------------------------------------
// launch 2: draw units, and the draw by the last unit of each request
// ---------------------------------------------------------------------------
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
__device__ void draw_token(const ChainArgs& a, int b, const Pending& d) {
  using S = Slice<DT, VEC, 1>;
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
  // 3) fp64 block scan of the crossing unit: thread t owns kPer logits
  const int c0 = s_unit * S::kSpan;
  const int c1 = min(a.V, c0 + S::kSpan);
  const double l2t = kLog2e / static_cast<double>(d.t);
  const int trow = d.mode == kModeResidual ? d.n : G;
  S st;
  st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow, a.V), c0, c1);
  double wk[S::kPer];
  if (residual) {
    S sd;
    sd.load(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V), c0, c1);
#pragma unroll
    for (int e = 0; e < S::kPer; ++e)
      wk[e] = fmax(0.0, exp_scaled(st.x[0][e], d.mt, l2t) * rzt - exp_scaled(sd.x[0][e], d.md, l2t) * rzd);
  } else {
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) wk[e] = exp_scaled(st.x[0][e], d.mt, l2t);
  }
  double own = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int e = 0; e < S::kPer; ++e) {
    own += wk[e];
    if (wk[e] > 0.0) last_pos = S::index(c0, 0, e);
  }
  if (tid == 0) { s_hit = 0x7fffffff; s_lasttok = -1; }
  double total;
  double run = s_before + block_exclusive_scan(own, &total);
  int hit = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < S::kPer; ++e) {
    run += wk[e];
    if (hit == 0x7fffffff && wk[e] > 0.0 && run > target) hit = S::index(c0, 0, e);
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

template <int DT, bool VEC>
__device__ void unit_item(const ChainArgs& a, long long item) {
  using S = Slice<DT, VEC, 1>;
  __shared__ double s_w[4][kWaves];
  __shared__ int s_last;
  __shared__ Pending s_pending;
  const int unit = static_cast<int>(item % a.nunit);
  const int G = a.gamma;
  int b;
  if (a.B <= kCompactMaxBatch) {
    static_assert(kCompactMaxBatch <= kThreads, "one temperature per thread");
    b = nth_drawing_request(a, static_cast<int>(item / a.nunit));
    if (b < 0) return;
  } else {
    b = static_cast<int>(item / a.nunit);
    if (request_class(a, a.temperature[b]) != 0) return;
  }
  if (threadIdx.x == 0) s_pending = a.pending[b];  // cleared only after this unit has arrived
  __syncthreads();
  const Pending d = s_pending;
  if (d.valid != 1) return;  // invalid request: launch 1 wrote its outputs
  // this unit's share of the final draw
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
    for (int e = 0; e < S::kPer; ++e) {
      const double et = exp_scaled(st.x[0][e], d.mt, l2t);
      const double ed = exp_scaled(sd.x[0][e], d.md, l2t);
      all_t += et;
      all_d += ed;
      if (et * d.zd > ed * d.zt) {  // p > q under the pass-1 normalisers
        pos_t += et;
        pos_d += ed;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) all_t += exp_scaled(st.x[0][e], d.mt, l2t);
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
  // wave 0 hands the record over (one field per lane) and counts the unit in
  if (threadIdx.x < kUnitFields) {
    double v = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) v += s_w[threadIdx.x][i];
    store_coherent_f64(&a.units[static_cast<size_t>(b) * a.nunit + unit].f[threadIdx.x], v);
  }
  if (threadIdx.x == 0)
    s_last = arrive(a.counters + static_cast<size_t>(b) * kCounterStride + kUnitCounter) ==
             static_cast<uint32_t>(a.nunit - 1);
  __syncthreads();
  if (s_last) {
    draw_token<DT, VEC>(a, b, d);
    unsigned long long* wz = reinterpret_cast<unsigned long long*>(a.units + static_cast<size_t>(b) * a.nunit);
    const int nw = a.nunit * static_cast<int>(sizeof(UnitRec) / 8);
    for (int i = threadIdx.x; i < nw; i += kThreads) wz[i] = 0ull;
    unsigned long long* pz = reinterpret_cast<unsigned long long*>(a.pending + b);
    if (threadIdx.x < static_cast<int>(sizeof(Pending) / 8)) pz[threadIdx.x] = 0ull;
    if (threadIdx.x == 0) store_coherent(a.counters + static_cast<size_t>(b) * kCounterStride + kUnitCounter, 0u);
  }
  __syncthreads();  // LDS is reused by the next item
}

// The draw of the last unit needs more registers than the unit sums; holding
// the kernel to 64 registers keeps eight waves per SIMD for the sums at the
// cost of a few spills on the draw path.
template <int DT, bool VEC, bool LOOP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void chain_units(ChainArgs a) {
  if constexpr (LOOP) {
    const long long items = static_cast<long long>(a.B) * a.nunit;
    for (long long item = blockIdx.x; item < items; item += gridDim.x) unit_item<DT, VEC>(a, item);
  } else {
    unit_item<DT, VEC>(a, blockIdx.x);
  }
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
  const size_t nchunk = static_cast<size_t>(num_chunks(V));
  const size_t R = 2 * static_cast<size_t>(gamma) + 1;
  const size_t nunit = static_cast<size_t>(units_for(V, 1));
  size_t off = 0;
  L.partials = off; off = align_up(off + static_cast<size_t>(B) * R * nchunk * sizeof(RowPartial));
  L.gathers = off;  off = align_up(off + static_cast<size_t>(B) * R * sizeof(float));
  L.pending = off;  off = align_up(off + static_cast<size_t>(B) * sizeof(Pending));
  L.units = off;    off = align_up(off + static_cast<size_t>(B) * nunit * sizeof(UnitRec));
  L.counters = off; off = align_up(off + static_cast<size_t>(B) * kCounterStride * sizeof(uint32_t));
  L.total = off;
  return L;
}

// Grids of the two launches are capped; their workgroups stride over the
// remaining items.
constexpr long long kMaxGrid = 1 << 20;

template <int DT, bool VEC>
static int launch_chain(ChainArgs a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  a.nunit = units_for(a.V, Slice<DT, VEC, 1>::kPer);
  const long long units = static_cast<long long>(a.B) * a.nunit;
  if (items <= kMaxGrid)
    launch(SV_K_CHAIN_ROW_STATS, chain_row_stats<DT, VEC, false>, dim3(static_cast<unsigned>(items)), dim3(kThreads),
           0, stream, a);
  else
    launch(SV_K_CHAIN_ROW_STATS, chain_row_stats<DT, VEC, true>, dim3(static_cast<unsigned>(kMaxGrid)), dim3(kThreads),
           0, stream, a);
  if (units <= kMaxGrid)
    launch(SV_K_CHAIN_UNITS, chain_units<DT, VEC, false>, dim3(static_cast<unsigned>(units)), dim3(kThreads), 0,
           stream, a);
  else
    launch(SV_K_CHAIN_UNITS, chain_units<DT, VEC, true>, dim3(static_cast<unsigned>(kMaxGrid)), dim3(kThreads), 0,
           stream, a);
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
  a.nchunk = num_chunks(V);
  a.out_tokens = out_tokens;
  a.out_n = out_num_accepted;
  a.partials = reinterpret_cast<RowPartial*>(ws + L.partials);
  a.gathers = reinterpret_cast<float*>(ws + L.gathers);
  a.pending = reinterpret_cast<Pending*>(ws + L.pending);
  a.units = reinterpret_cast<UnitRec*>(ws + L.units);
  a.counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_chain<0, true>(a, stream) : launch_chain<0, false>(a, stream);
  return vec ? launch_chain<1, true>(a, stream) : launch_chain<1, false>(a, stream);
}
