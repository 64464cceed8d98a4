// Chain verification: the acceptance stage of one speculative-decoding round
// for a batch of requests (Leviathan et al.'s Algorithm 1 as restated in the
// close-reading notes 02, section 4, and CMU 15-779 lecture 17 notes, sections
// 2.2-2.4).  See include/specverify.h for the contract.
//
// Three launches on the caller's stream; every dependency between workgroups
// is a launch boundary, so all reads are plain loads:
//
//  1. chain_row_stats  one workgroup per needed (row, chunk) of kChunk logits:
//                      the chunk max and, for sampling rows, the fp32 sum of
//                      exp2((x - max) * log2e / T); for greedy rows the argmax
//                      (lowest index).  The workgroup whose chunk holds a
//                      row's draft token also records that logit.  Draft rows
//                      of greedy requests are not read.
//  2. chain_units      one workgroup per (request, draw unit) of kThreads*kPer
//                      logits.  Each re-derives its request's decision from the
//                      row partials in one round of loads (fp64 merge; the
//                      gamma-step test u <= tau, tau = 1 if q <= p else p / q;
//                      greedy: argmax equality); unit 0 writes the accepted
//                      tokens and count.  For a sampling request each unit then
//                      sums, in fp64, exp((x - max) / T) of the final draw's
//                      target and draft rows over its span (all, and where
//                      p > q), also per 64-lane sub-span.
//  3. chain_finalize   one workgroup per request: fp64 normalisers from the
//                      unit sums, the residual (or bonus) weight of every unit
//                      and sub-span, an fp64 scan of the crossing sub-span -- the
//                      smallest k with C_k > u * W -- and returns every
//                      workspace word the request used to zero.
//
// Precision: the accept test needs p(x)/q(x) to ~1e-6 and uses the fp32 row
// normalisers; the final draw uses fp64 exponentials and fp64 normalisers
// summed in launch 2, so the inverse CDF matches an fp64 reference except
// where u lies within a few ulps of a CDF step.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
struct RowPartial {  // one (row, chunk), packed in one 64-bit word
  float m;           // chunk max
  int32_t v;         // float bits of the exp-sum (sampling) or the argmax (greedy)
};

struct UnitRec {     // per (request, draw unit), fp64
  double st_all, sd_all, st_pos, sd_pos;
  double w_pos_t[kWaves], w_pos_d[kWaves], w_all_t[kWaves];
};

static_assert(sizeof(RowPartial) == 8, "row partials are one 64-bit word");
static_assert(sizeof(UnitRec) % 8 == 0, "unit records are cleared in 64-bit words");

enum : int32_t { kModeResidual = 1, kModeBonus = 2 };

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
  UnitRec* units;        // [B][nunit]
};

// T must be 0 (greedy) or a finite positive normal float.
__device__ inline bool temp_ok(float t) { return isfinite(t) && (t == 0.0f || t >= 1.17549435e-38f); }

template <int DT>
__device__ inline const void* row_ptr(const void* base, size_t row, int V) {
  return static_cast<const char*>(base) + row * static_cast<size_t>(V) * Elem<DT>::kBytes;
}

__device__ inline double exp_scaled(float x, float m, double inv_t) {
  return exp(static_cast<double>(x - m) * inv_t);
}

// Request classes: 0 samples with its draft rows (it has a final draw), 1 is
// greedy or cannot sample (target rows only), 2 has an invalid temperature.
__device__ inline int request_class(const ChainArgs& a, float T) {
  if (!temp_ok(T)) return 2;
  if (T > 0.0f && (a.draft != nullptr || a.gamma == 0)) return 0;
  return 1;
}

// Rows of a request that are read: target rows, plus draft rows when sampling.
__device__ inline int needed_rows(const ChainArgs& a, float T) {
  return (T > 0.0f && a.draft != nullptr) ? 2 * a.gamma + 1 : a.gamma + 1;
}

// ---------------------------------------------------------------------------
// launch 1: row statistics
// ---------------------------------------------------------------------------
// Workgroups [0, B*(gamma+1)*nchunk) cover the target rows and the rest the
// draft rows, so the workgroups that skip (draft rows of greedy requests)
// come last.
template <int DT, bool VEC>
__device__ void row_stats_item(const ChainArgs& a, long long item) {
  __shared__ float s_wm[kWaves];
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const long long ntgt = static_cast<long long>(a.B) * (G + 1) * a.nchunk;
  int b, k, c;
  if (item < ntgt) {
    b = static_cast<int>(item / ((G + 1) * a.nchunk));
    const int rem = static_cast<int>(item % ((G + 1) * a.nchunk));
    k = rem / a.nchunk;
    c = rem % a.nchunk;
  } else {
    const long long i2 = item - ntgt;
    b = static_cast<int>(i2 / (G * a.nchunk));
    const int rem = static_cast<int>(i2 % (G * a.nchunk));
    k = G + 1 + rem / a.nchunk;
    c = rem % a.nchunk;
  }
  const float T = a.temperature[b];
  if (!temp_ok(T)) return;
  const bool sampling = T > 0.0f;
  if (k > G && !(sampling && a.draft != nullptr)) return;  // draft rows are read only when sampling
  const int pos = k <= G ? k : k - G - 1;                    // draft position of this row
  const void* row = (k <= G) ? row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + k, a.V)
                             : row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + pos, a.V);
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  const int32_t tok = (sampling && pos < G) ? a.tokens[static_cast<size_t>(b) * G + pos] : -1;
  Slice<DT, VEC> s;
  s.load(row, c0, c1);
  if (tok >= c0 && tok < c1) {
#pragma unroll
    for (int j = 0; j < s.kItems; ++j)
#pragma unroll
      for (int e = 0; e < s.kPer; ++e)
        if (s.index(c0, j, e) == tok) a.gathers[static_cast<size_t>(b) * R + k] = s.x[j][e];
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < s.kItems; ++j)
#pragma unroll
    for (int e = 0; e < s.kPer; ++e) m = fmaxf(m, s.x[j][e]);
  RowPartial out;
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
    out.m = bm;
    out.v = best.i;
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
    out.m = ms.m;
    out.v = __float_as_int(ms.z);
  }
  if (threadIdx.x == 0) a.partials[(static_cast<size_t>(b) * R + k) * a.nchunk + c] = out;
  __syncthreads();  // s_wm is reused by the next item
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_row_stats(ChainArgs a) {
  const long long items = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  for (long long item = blockIdx.x; item < items; item += gridDim.x) row_stats_item<DT, VEC>(a, item);
}

// ---------------------------------------------------------------------------
// the decision of request b, derived by a whole workgroup from the partials
// ---------------------------------------------------------------------------
struct Decision {
  int32_t bad;        // invalid token / uniform / missing draft logits
  int32_t n;          // accepted drafts
  int32_t mode;       // kModeResidual / kModeBonus (sampling)
  int32_t final_tok;  // greedy: the emitted argmax
  float mt, md;       // maxima of the final draw's target / draft rows
  double zt, zd;      // their fp64-merged pass-1 normalisers
  float u, t;         // u[b][gamma], temperature
};

template <int DT>
__device__ Decision decide(const ChainArgs& a, int b) {
  constexpr int kMaxRows = 2 * SV_MAX_GAMMA + 1;
  __shared__ float s_gm[kThreads];
  __shared__ double s_gz[kThreads];
  __shared__ int32_t s_garg[kThreads];
  __shared__ float s_m[kMaxRows];
  __shared__ double s_z[kMaxRows];
  __shared__ int32_t s_arg[kMaxRows];
  __shared__ float s_xt[SV_MAX_GAMMA], s_xd[SV_MAX_GAMMA];
  __shared__ int32_t s_ok[SV_MAX_GAMMA];
  __shared__ Decision s_dec;
  const int tid = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  const bool sampling = T > 0.0f;
  const double inv_t = sampling ? 1.0 / static_cast<double>(T) : 0.0;
  const int nrows = needed_rows(a, T);
  // one round of loads: the chunk partials (in groups of chunks, one group per
  // thread), the draft tokens, their gathered logits and the uniforms
  const int gpr = max(1, min((a.nchunk + 7) / 8, kThreads / nrows));  // groups per row
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
    for (int c0 = cb; c0 < ce; c0 += 8) {
      RowPartial w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = p[min(c0 + i, ce - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (c0 + i >= ce) continue;
        if (!sampling) {
          best = argmax_combine(best, ArgMax{w[i].m, w[i].v});
        } else if (w[i].m != -INFINITY) {
          if (w[i].m > m) {
            if (m != -INFINITY) z *= exp(static_cast<double>(m - w[i].m) * inv_t);
            m = w[i].m;
          }
          z += static_cast<double>(__int_as_float(w[i].v)) * exp_scaled(w[i].m, m, inv_t);
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
          if (gm != -INFINITY) z += s_gz[tid * gpr + g] * exp_scaled(gm, m, inv_t);
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
        const double p = exp_scaled(s_xt[tid], s_m[tid], inv_t) / s_z[tid];
        const double q = exp_scaled(s_xd[tid], s_m[G + 1 + tid], inv_t) / s_z[G + 1 + tid];
        const double tau = (q <= p) ? 1.0 : p / q;
        const double u = static_cast<double>(a.uniforms[static_cast<size_t>(b) * (G + 1) + tid]);
        ok = (u <= tau);
      }
      s_ok[tid] = ok;
    }
    __syncthreads();
  }
  if (tid == 0) {
    Decision d{};
    d.bad = bad;
    if (!bad) {
      int n = 0;
      while (n < G && s_ok[n]) ++n;
      d.n = n;
      d.t = T;
      if (!sampling) {
        d.final_tok = s_arg[n];
      } else {
        d.mode = n < G ? kModeResidual : kModeBonus;
        d.mt = s_m[n];
        d.zt = s_z[n];
        if (n < G) {
          d.md = s_m[G + 1 + n];
          d.zd = s_z[G + 1 + n];
        }
        d.u = a.uniforms[static_cast<size_t>(b) * (G + 1) + G];
      }
    }
    s_dec = d;
  }
  __syncthreads();
  const Decision d = s_dec;
  __syncthreads();
  return d;
}

// Accepted tokens, count, and for greedy requests the final token; slot n of
// a sampling request is left to the launch that draws it.
__device__ void write_outputs(const ChainArgs& a, int b, const Decision& d, bool sampling) {
  const int G = a.gamma;
  int32_t* out = a.out_tokens + static_cast<size_t>(b) * (G + 1);
  for (int i = threadIdx.x; i <= G; i += kThreads) {
    int32_t v = -1;
    if (!d.bad) {
      if (sampling && i == d.n) continue;
      if (i < d.n) v = a.tokens[static_cast<size_t>(b) * G + i];
      else if (i == d.n) v = d.final_tok;
    }
    out[i] = v;
  }
  if (threadIdx.x == 0) a.out_n[b] = d.bad ? -1 : d.n;
}

// ---------------------------------------------------------------------------
// launch 2: decisions and draw-unit sums
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void unit_item(const ChainArgs& a, long long item) {
  using S = Slice<DT, VEC, 1>;
  __shared__ double s_w[4][kWaves];
  const int b = static_cast<int>(item / a.nunit);
  const int unit = static_cast<int>(item % a.nunit);
  const int G = a.gamma;
  const float T = a.temperature[b];
  const int cls = request_class(a, T);
  if (cls == 2) {  // nothing was read for this request
    if (unit == 0) {
      for (int i = threadIdx.x; i <= G; i += kThreads) a.out_tokens[static_cast<size_t>(b) * (G + 1) + i] = -1;
      if (threadIdx.x == 0) a.out_n[b] = -1;
    }
    return;
  }
  if (cls == 1 && unit != 0) return;
  const Decision d = decide<DT>(a, b);
  if (unit == 0) write_outputs(a, b, d, cls == 0);
  if (cls != 0 || d.bad) return;
  // this unit's share of the final draw
  const double inv_t = 1.0 / static_cast<double>(d.t);
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
      const double et = exp_scaled(st.x[0][e], d.mt, inv_t);
      const double ed = exp_scaled(sd.x[0][e], d.md, inv_t);
      all_t += et;
      all_d += ed;
      if (et * d.zd > ed * d.zt) {  // p > q under the pass-1 normalisers
        pos_t += et;
        pos_d += ed;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) all_t += exp_scaled(st.x[0][e], d.mt, inv_t);
  }
  pos_t = wave_sum(pos_t);
  pos_d = wave_sum(pos_d);
  all_t = wave_sum(all_t);
  all_d = wave_sum(all_d);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    s_w[0][w] = pos_t;
    s_w[1][w] = pos_d;
    s_w[2][w] = all_t;
    s_w[3][w] = all_d;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    UnitRec r;
    r.st_pos = r.sd_pos = r.st_all = r.sd_all = 0.0;
    for (int i = 0; i < kWaves; ++i) {
      r.w_pos_t[i] = s_w[0][i];
      r.w_pos_d[i] = s_w[1][i];
      r.w_all_t[i] = s_w[2][i];
      r.st_pos += s_w[0][i];
      r.sd_pos += s_w[1][i];
      r.st_all += s_w[2][i];
      r.sd_all += s_w[3][i];
    }
    a.units[static_cast<size_t>(b) * a.nunit + unit] = r;
  }
  __syncthreads();  // s_w is reused by the next item
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_units(ChainArgs a) {
  const long long items = static_cast<long long>(a.B) * a.nunit;
  for (long long item = blockIdx.x; item < items; item += gridDim.x) unit_item<DT, VEC>(a, item);
}

// ---------------------------------------------------------------------------
// launch 3: the final draw, and the workspace back to zero
// ---------------------------------------------------------------------------
// Weight of a unit (or of one of its sub-spans) in the final draw.
__device__ inline double unit_weight(double pos_t, double pos_d, double all_t, bool residual,
                                     double zt, double zd) {
  return residual ? (pos_t / zt - pos_d / zd) : all_t;
}

template <int DT, bool VEC>
__device__ void draw_token(const ChainArgs& a, int b, const Decision& d) {
  using S = Slice<DT, VEC, 1>;
  __shared__ int s_unit, s_sub, s_first, s_lastpos;
  __shared__ double s_before;
  const int G = a.gamma;
  const int tid = threadIdx.x;
  const UnitRec* ur = a.units + static_cast<size_t>(b) * a.nunit;
  // 1) normalisers: fp64 sums of exp((x - max) / T) over every unit.  With at
  //    most kThreads units (the usual case) each thread keeps its unit's sums
  //    in registers for the scan below.
  const bool one_batch = a.nunit <= kThreads;
  double my_all_t = 0.0, my_pos_t = 0.0, my_pos_d = 0.0;
  double tot[2] = {0.0, 0.0};
  for (int i = tid; i < a.nunit; i += kThreads) {
    const double at = ur[i].st_all, ad = ur[i].sd_all;
    tot[0] += at;
    tot[1] += ad;
    if (one_batch) { my_all_t = at; my_pos_t = ur[i].st_pos; my_pos_d = ur[i].sd_pos; }
  }
  block_sum_doubles<2>(tot);
  const double zt = tot[0], zd = tot[1];
  auto weight_of = [&](int i, bool resid) -> double {
    if (one_batch) return unit_weight(my_pos_t, my_pos_d, my_all_t, resid, zt, zd);
    return unit_weight(ur[i].st_pos, ur[i].sd_pos, ur[i].st_all, resid, zt, zd);
  };
  // 2) an empty residual (p and q equal up to rounding) draws from p of that
  //    position instead
  bool residual = d.mode == kModeResidual;
  if (residual) {
    double ws[1] = {0.0};
    for (int i = tid; i < a.nunit; i += kThreads) ws[0] += weight_of(i, true);
    block_sum_doubles<1>(ws);
    if (!(ws[0] > 0.0)) residual = false;
  }
  double W;
  {
    double ws[1] = {0.0};
    for (int i = tid; i < a.nunit; i += kThreads) ws[0] += weight_of(i, residual);
    block_sum_doubles<1>(ws);
    W = ws[0];
  }
  const double target = static_cast<double>(d.u) * W;
  // 3) crossing unit: block scan of the unit weights in unit order
  if (tid == 0) { s_unit = -1; s_lastpos = -1; }
  __syncthreads();
  double carry = 0.0;
  for (int base = 0; base < a.nunit; base += kThreads) {
    const int i = base + tid;
    const double wu = i < a.nunit ? weight_of(i, residual) : 0.0;
    double total;
    const double before = carry + block_exclusive_scan(wu, &total);
    if (tid == 0) s_first = 0x7fffffff;
    __syncthreads();
    if (i < a.nunit && wu > 0.0) atomicMax(&s_lastpos, i);
    if (i < a.nunit && before + wu > target) atomicMin(&s_first, i);
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
    for (int i = tid; i < lp; i += kThreads) bsum[0] += weight_of(i, residual);
    block_sum_doubles<1>(bsum);
    if (tid == 0) { s_unit = lp; s_before = bsum[0]; }
    __syncthreads();
  }
  // 4) crossing sub-span inside the unit
  if (tid == 0) {
    const UnitRec& u = ur[s_unit];
    double ws[kWaves];
#pragma unroll
    for (int i = 0; i < kWaves; ++i) ws[i] = unit_weight(u.w_pos_t[i], u.w_pos_d[i], u.w_all_t[i], residual, zt, zd);
    double run = s_before;
    int sub = -1, lastsub = -1;
    double before_sub = run;
    for (int i = 0; i < kWaves; ++i) {
      if (ws[i] > 0.0) lastsub = i;
      if (sub < 0 && run + ws[i] > target) { sub = i; before_sub = run; }
      run += ws[i];
    }
    if (sub < 0) {
      sub = lastsub < 0 ? 0 : lastsub;
      before_sub = s_before;
      for (int i = 0; i < sub; ++i) before_sub += ws[i];
    }
    s_sub = sub;
    s_before = before_sub;
  }
  __syncthreads();
  // 5) fp64 scan of the crossing sub-span by one wave; lane l owns kPer logits
  if (tid < kWave) {
    const int lane = tid;
    const int k0 = s_unit * S::kSpan + (s_sub * kWave + lane) * S::kPer;
    const double inv_t = 1.0 / static_cast<double>(d.t);
    const int trow = d.mode == kModeResidual ? d.n : G;
    const void* tr = row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow, a.V);
    const void* dr = residual ? row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V) : nullptr;
    double wk[S::kPer];
    double mine = 0.0;
    int last_pos = -1;
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) {
      const int k = k0 + e;
      double x = 0.0;
      if (k < a.V) {
        const double et = exp_scaled(Elem<DT>::at(tr, k), d.mt, inv_t);
        x = residual ? fmax(0.0, et / zt - exp_scaled(Elem<DT>::at(dr, k), d.md, inv_t) / zd) : et;
      }
      wk[e] = x;
      mine += x;
      if (x > 0.0) last_pos = k;
    }
    double inc = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double t = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += t;
    }
    double exc = __shfl_up(inc, 1, kWave);
    if (lane == 0) exc = 0.0;
    double run = s_before + exc;
    int hit = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < S::kPer; ++e) {
      run += wk[e];
      if (hit == 0x7fffffff && wk[e] > 0.0 && run > target) hit = k0 + e;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      hit = min(hit, __shfl_xor(hit, o, kWave));
      last_pos = max(last_pos, __shfl_xor(last_pos, o, kWave));
    }
    if (lane == 0) a.out_tokens[static_cast<size_t>(b) * (G + 1) + d.n] = (hit != 0x7fffffff) ? hit : last_pos;
  }
  __syncthreads();
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_finalize(ChainArgs a) {
  const int b = blockIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  const int cls = request_class(a, T);
  if (cls == 2) return;  // nothing of this request is in the workspace
  if (cls == 0) {
    const Decision d = decide<DT>(a, b);
    if (!d.bad) {
      draw_token<DT, VEC>(a, b, d);
      unsigned long long* w = reinterpret_cast<unsigned long long*>(a.units + static_cast<size_t>(b) * a.nunit);
      const int nw = a.nunit * static_cast<int>(sizeof(UnitRec) / 8);
      for (int i = threadIdx.x; i < nw; i += kThreads) w[i] = 0ull;
    }
  }
  // the request's row partials and gathered logits back to zero
  const int nrows = needed_rows(a, T);
  unsigned long long* p = reinterpret_cast<unsigned long long*>(a.partials + static_cast<size_t>(b) * R * a.nchunk);
  for (int i = threadIdx.x; i < nrows * a.nchunk; i += kThreads) p[i] = 0ull;
  if (static_cast<int>(threadIdx.x) < R) a.gathers[static_cast<size_t>(b) * R + threadIdx.x] = 0.0f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct ChainLayout {
  size_t partials, gathers, units, total;
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
  L.units = off;    off = align_up(off + static_cast<size_t>(B) * nunit * sizeof(UnitRec));
  L.total = off;
  return L;
}

// Grids of the two streaming launches are capped; their workgroups stride over
// the remaining items.
constexpr long long kMaxGrid = 1 << 20;

template <int DT, bool VEC>
static int launch_chain(ChainArgs a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  a.nunit = units_for(a.V, Slice<DT, VEC, 1>::kPer);
  const long long units = static_cast<long long>(a.B) * a.nunit;
  launch(SV_K_CHAIN_ROW_STATS, chain_row_stats<DT, VEC>, dim3(static_cast<unsigned>(items < kMaxGrid ? items : kMaxGrid)),
         dim3(kThreads), 0, stream, a);
  launch(SV_K_CHAIN_UNITS, chain_units<DT, VEC>, dim3(static_cast<unsigned>(units < kMaxGrid ? units : kMaxGrid)),
         dim3(kThreads), 0, stream, a);
  launch(SV_K_CHAIN_FINALIZE, chain_finalize<DT, VEC>, dim3(static_cast<unsigned>(a.B)), dim3(kThreads), 0, stream, a);
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
  a.units = reinterpret_cast<UnitRec*>(ws + L.units);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_chain<0, true>(a, stream) : launch_chain<0, false>(a, stream);
  return vec ? launch_chain<1, true>(a, stream) : launch_chain<1, false>(a, stream);
}
