// Chain verification: the acceptance stage of one speculative-decoding round
// for a batch of requests (Leviathan et al.'s Algorithm 1 as restated in the
// close-reading notes 02, section 4, and CMU 15-779 lecture 17 notes, sections
// 2.2-2.4).  See include/specverify.h for the contract.
//
// One cooperative launch of a persistent kernel.  Every workgroup walks the
// row items (request, row, chunk) grid-stride; the workgroup whose item
// completes a request's rows takes that request's decision and raises the
// request's flag.  The final draw of a sampling request is split into draw
// units; unit q (request q / nunit) belongs to workgroup q mod grid, which
// runs it as soon as the request's flag is up -- between its own row items,
// or after them.  The workgroup completing a request's last unit locates and
// emits the drawn token.  Workgroups only ever wait on per-request flags,
// never on a shared counter, so no memory line is polled by the whole grid.
//
//  row item   kChunk logits of one needed row: the chunk max and, for sampling
//             rows, sum exp2((x - max) * log2e / T) in fp32; for greedy rows
//             the argmax (lowest index).  Draft rows of greedy requests and
//             all rows of requests with an invalid temperature are not read.
//  decision   fp64 merge of the chunk partials; the gamma-step accept test
//             (u <= tau, tau = 1 if q <= p else p / q, p and q from the
//             gathered logits); greedy: argmax equality.  Writes the accepted
//             tokens and count, and for greedy requests the final token.
//  draw unit  kThreads * kPer logits of the final draw's row(s): fp64 sums of
//             exp((x - max) / T) for the target and draft rows (all, and where
//             p > q), also per 64-lane sub-span.
//  finalise   fp64 normalisers from the units; cumulative residual (or bonus)
//             weight per unit and sub-span; an fp64 scan of the crossing
//             sub-span: the smallest k with C_k > u * W.
//
// Cross-workgroup data (partials, decisions, the draw queue) is written with
// agent-scope coherent stores, drained with s_waitcnt before the arrival
// atomic, and read with agent-scope coherent loads, so no L2 write-back or
// invalidate is issued.  Every wait is bounded.  Every word of the workspace
// is returned to zero by the workgroup that consumes it, so a completed call
// leaves the whole workspace zeroed whatever the next call's shape.
#include "sv_device.hpp"
#include "sv_host.hpp"

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

namespace sv {

// ---------------------------------------------------------------------------
// coherent accesses between workgroups (agent scope)
// ---------------------------------------------------------------------------
template <typename T> __device__ inline void cstore(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T> __device__ inline T cload(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int cadd(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline bool ccas(int* p, int expected, int desired) {
  return __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_RELAXED,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every earlier store of this wave has completed (reached the coherence point).
__device__ inline void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

constexpr int kSpinLimit = 1 << 22;  // bound of every wait (~0.2 s with s_sleep)
constexpr int kLine = 32;            // ints per padded counter (128 bytes)

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
struct RowPartial {  // one (row, chunk)
  float m;           // chunk max
  int32_t v;         // float bits of the exp-sum (sampling) or the argmax (greedy)
};

enum : int32_t { kModeResidual = 1, kModeBonus = 2 };

struct DecisionRec {  // per sampling request, read by its draw units
  int32_t mode, n;
  float mt, md;       // maxima of the final draw's target / draft rows
  double zt, zd;      // pass-1 normalisers of those rows (fp64 merge)
  float u, t;
};

struct UnitRec {      // per (request, draw unit), fp64
  double st_all, sd_all, st_pos, sd_pos;
  double w_pos_t[kWaves], w_pos_d[kWaves], w_all_t[kWaves];
};

static_assert(sizeof(RowPartial) == 8, "row partials are cleared as one 64-bit word");
static_assert(sizeof(DecisionRec) % 8 == 0 && sizeof(UnitRec) % 8 == 0,
              "records are cleared in 64-bit words");

enum : int { kFlagNone = 0, kFlagDraw = 1, kFlagDone = 2 };  // per-request flag values

struct ChainArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;
  int B, gamma, V, nchunk, nunit, nslots;
  int32_t* out_tokens;
  int32_t* out_n;
  RowPartial* partials;    // [B][2*gamma+1][nchunk]
  int* cnt_rows;           // [B][kLine]
  int* cnt_units;          // [B][kLine]
  int* flag;               // [B][kLine] kFlagNone / kFlagDraw / kFlagDone
  DecisionRec* decisions;  // [B]
  UnitRec* units;          // [B][nunit]
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

// Returns the chunk partials of one row to zero once they have been consumed.
__device__ inline void clear_row_partials(RowPartial* p, int nchunk) {
  for (int c = 0; c < nchunk; ++c) cstore(reinterpret_cast<unsigned long long*>(p + c), 0ull);
}

// Rows of request b that are read: target rows, plus draft rows when sampling.
__device__ inline int needed_rows(const ChainArgs& a, float T) {
  return (T > 0.0f && a.draft != nullptr) ? 2 * a.gamma + 1 : a.gamma + 1;
}

// ---------------------------------------------------------------------------
// decision of request b (whole workgroup)
// ---------------------------------------------------------------------------
template <int DT>
__device__ void decide(const ChainArgs& a, int b) {
  constexpr int kMaxRows = 2 * SV_MAX_GAMMA + 1;
  __shared__ float s_m[kMaxRows];
  __shared__ double s_z[kMaxRows];
  __shared__ int32_t s_arg[kMaxRows];
  __shared__ float s_xt[SV_MAX_GAMMA], s_xd[SV_MAX_GAMMA];
  __shared__ int32_t s_ok[SV_MAX_GAMMA];
  const int tid = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  const bool sampling = T > 0.0f;
  // validity of tokens and uniforms; gather the draft tokens' logits
  int bad = 0;
  if (tid < G) {
    const int32_t x = a.tokens[static_cast<size_t>(b) * G + tid];
    bad |= (x < 0 || x >= a.V);
    if (!bad && sampling && a.draft != nullptr) {
      s_xt[tid] = Elem<DT>::at(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + tid, a.V), x);
      s_xd[tid] = Elem<DT>::at(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + tid, a.V), x);
    }
  }
  if (sampling && tid <= G) {
    const float u = a.uniforms[static_cast<size_t>(b) * (G + 1) + tid];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  if (sampling && G > 0 && a.draft == nullptr) bad = 1;
  bad = __syncthreads_or(bad);
  int32_t* out = a.out_tokens + static_cast<size_t>(b) * (G + 1);
  if (bad) {
    for (int i = tid; i <= G; i += kThreads) out[i] = -1;
    if (tid < needed_rows(a, T))
      clear_row_partials(a.partials + (static_cast<size_t>(b) * R + tid) * a.nchunk, a.nchunk);
    if (tid == 0) {
      a.out_n[b] = -1;
      drain_stores();
      cstore(&a.flag[b * kLine], int(kFlagDone));
    }
    return;
  }
  // merge the chunk partials of every needed row (one thread per row, eight
  // coherent loads in flight at a time)
  const double inv_t = sampling ? 1.0 / static_cast<double>(T) : 0.0;
  const int nrows = needed_rows(a, T);
  if (tid < nrows) {
    const RowPartial* p = a.partials + (static_cast<size_t>(b) * R + tid) * a.nchunk;
    if (!sampling) {
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int c0 = 0; c0 < a.nchunk; c0 += 8) {
        float pm[8];
        int32_t pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = min(c0 + i, a.nchunk - 1);
          pm[i] = cload(&p[c].m);
          pv[i] = cload(&p[c].v);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c0 + i < a.nchunk) best = argmax_combine(best, ArgMax{pm[i], pv[i]});
      }
      s_m[tid] = best.v;
      s_arg[tid] = best.i;
      clear_row_partials(const_cast<RowPartial*>(p), a.nchunk);
    } else {
      float m = -INFINITY;
      double z = 0.0;
      for (int c0 = 0; c0 < a.nchunk; c0 += 8) {
        float pm[8], pz[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = min(c0 + i, a.nchunk - 1);
          pm[i] = cload(&p[c].m);
          pz[i] = __int_as_float(cload(&p[c].v));
        }
        float mm = m;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c0 + i < a.nchunk) mm = fmaxf(mm, pm[i]);
        if (mm != m && m != -INFINITY) z *= exp(static_cast<double>(m - mm) * inv_t);
        m = mm;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c0 + i < a.nchunk && pm[i] != -INFINITY)
            z += static_cast<double>(pz[i]) * exp_scaled(pm[i], m, inv_t);
      }
      s_m[tid] = m;
      s_z[tid] = z;
      clear_row_partials(const_cast<RowPartial*>(p), a.nchunk);
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
  int n = 0;
  while (n < G && s_ok[n]) ++n;
  // slot n of a sampling request belongs to the workgroup that finalises its
  // draw (one writer per output word)
  for (int i = tid; i <= G; i += kThreads) {
    if (sampling && i == n) continue;
    int32_t v = -1;
    if (i < n) v = a.tokens[static_cast<size_t>(b) * G + i];
    else if (i == n) v = s_arg[n];
    out[i] = v;
  }
  if (tid == 0) {
    a.out_n[b] = n;
    if (sampling) {
      DecisionRec* d = a.decisions + b;
      cstore(&d->mode, n < G ? int32_t(kModeResidual) : int32_t(kModeBonus));
      cstore(&d->n, int32_t(n));
      cstore(&d->mt, s_m[n]);
      cstore(&d->zt, s_z[n]);
      if (n < G) {
        cstore(&d->md, s_m[G + 1 + n]);
        cstore(&d->zd, s_z[G + 1 + n]);
      }
      cstore(&d->u, a.uniforms[static_cast<size_t>(b) * (G + 1) + G]);
      cstore(&d->t, T);
    }
    // the decision record is complete before the flag rises
    drain_stores();
    cstore(&a.flag[b * kLine], sampling ? int(kFlagDraw) : int(kFlagDone));
  }
}

// ---------------------------------------------------------------------------
// one row item
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void row_item(const ChainArgs& a, int b, int k, int c, float T) {
  __shared__ int s_last;
  __shared__ float s_wm[kWaves];
  const bool sampling = T > 0.0f;
  const void* row = (k <= a.gamma)
      ? row_ptr<DT>(a.target, static_cast<size_t>(b) * (a.gamma + 1) + k, a.V)
      : row_ptr<DT>(a.draft, static_cast<size_t>(b) * a.gamma + (k - a.gamma - 1), a.V);
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  Slice<DT, VEC> s;
  s.load(row, c0, c1);
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < s.kItems; ++j)
#pragma unroll
    for (int e = 0; e < s.kPer; ++e) m = fmaxf(m, s.x[j][e]);
  RowPartial out{};
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
  if (threadIdx.x == 0) {
    RowPartial* dst = a.partials + (static_cast<size_t>(b) * (2 * a.gamma + 1) + k) * a.nchunk + c;
    cstore(&dst->m, out.m);
    cstore(&dst->v, out.v);
    drain_stores();
    const int need = needed_rows(a, T) * a.nchunk;
    const int old = cadd(&a.cnt_rows[b * kLine], 1);
    s_last = (old == need - 1);
    if (old == need - 1) cstore(&a.cnt_rows[b * kLine], 0);
  }
  __syncthreads();
  const int last = s_last;
  __syncthreads();
  if (last) decide<DT>(a, b);
}

// ---------------------------------------------------------------------------
// draw units
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void finalize(const ChainArgs& a, int b, const DecisionRec& d);

// Draw unit `unit` of request b, whose flag was seen as `f`: kFlagDone units
// only arrive; kFlagDraw units accumulate their weights first.  The last unit
// to arrive finalises the draw (kFlagDraw) and returns the request's counters
// and flag to zero.
template <int DT, bool VEC>
__device__ void draw_unit(const ChainArgs& a, int b, int unit, int f) {
  using S = Slice<DT, VEC, 1>;
  __shared__ int s_last;
  __shared__ DecisionRec s_d;
  __shared__ double s_w[4][kWaves];
  const int G = a.gamma;
  if (f != kFlagDraw) {
    if (threadIdx.x == 0) {
      const int old = cadd(&a.cnt_units[b * kLine], 1);
      if (old == a.nunit - 1) {
        cstore(&a.cnt_units[b * kLine], 0);
        cstore(&a.flag[b * kLine], int(kFlagNone));
      }
    }
    __syncthreads();
    return;
  }
  if (threadIdx.x == 0) {
    const DecisionRec* dr = a.decisions + b;
    s_d.mode = cload(&dr->mode);
    s_d.n = cload(&dr->n);
    s_d.mt = cload(&dr->mt);
    s_d.md = cload(&dr->md);
    s_d.zt = cload(&dr->zt);
    s_d.zd = cload(&dr->zd);
    s_d.u = cload(&dr->u);
    s_d.t = cload(&dr->t);
  }
  __syncthreads();
  DecisionRec d = s_d;
  // keep every row index in range whatever the record holds
  if (d.n < 0 || d.n > G) d.n = G;
  if (d.n == G) d.mode = kModeBonus;
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
    UnitRec* ur = a.units + static_cast<size_t>(b) * a.nunit + unit;
    double u_all_t = 0, u_all_d = 0, u_pos_t = 0, u_pos_d = 0;
    for (int i = 0; i < kWaves; ++i) {
      u_pos_t += s_w[0][i];
      u_pos_d += s_w[1][i];
      u_all_t += s_w[2][i];
      u_all_d += s_w[3][i];
      cstore(&ur->w_pos_t[i], s_w[0][i]);
      cstore(&ur->w_pos_d[i], s_w[1][i]);
      cstore(&ur->w_all_t[i], s_w[2][i]);
    }
    cstore(&ur->st_all, u_all_t);
    cstore(&ur->sd_all, u_all_d);
    cstore(&ur->st_pos, u_pos_t);
    cstore(&ur->sd_pos, u_pos_d);
    drain_stores();
    const int old = cadd(&a.cnt_units[b * kLine], 1);
    s_last = (old == a.nunit - 1);
  }
  __syncthreads();
  const int last = s_last;
  __syncthreads();
  if (last) {
    finalize<DT, VEC>(a, b, d);
    if (threadIdx.x == 0) {
      cstore(&a.cnt_units[b * kLine], 0);
      cstore(&a.flag[b * kLine], int(kFlagNone));
    }
  }
}

// Weight of a unit (or of one of its sub-spans) in the final draw.
__device__ inline double unit_weight(double pos_t, double pos_d, double all_t, bool residual,
                                     double zt, double zd) {
  return residual ? (pos_t / zt - pos_d / zd) : all_t;
}

template <int DT, bool VEC>
__device__ void finalize(const ChainArgs& a, int b, const DecisionRec& d) {
  using S = Slice<DT, VEC, 1>;
  __shared__ int s_unit, s_sub, s_found;
  __shared__ double s_before;
  const int G = a.gamma;
  const UnitRec* ur = a.units + static_cast<size_t>(b) * a.nunit;
  // fp64 normalisers of the two rows
  double tot[2] = {0.0, 0.0};
  for (int i = threadIdx.x; i < a.nunit; i += kThreads) {
    tot[0] += cload(&ur[i].st_all);
    tot[1] += cload(&ur[i].sd_all);
  }
  block_sum_doubles<2>(tot);
  const double zt = tot[0], zd = tot[1];
  bool residual = d.mode == kModeResidual;
  // total weight; an empty residual (p and q equal up to rounding) draws from
  // p of that position instead
  double W;
  {
    double ws[1] = {0.0};
    for (int i = threadIdx.x; i < a.nunit; i += kThreads)
      ws[0] += unit_weight(cload(&ur[i].st_pos), cload(&ur[i].sd_pos), cload(&ur[i].st_all),
                           residual, zt, zd);
    block_sum_doubles<1>(ws);
    W = ws[0];
    if (residual && !(W > 0.0)) {
      residual = false;
      W = zt;
    }
  }
  const double target = static_cast<double>(d.u) * W;
  // crossing unit: block scan over units in batches of kThreads
  if (threadIdx.x == 0) { s_found = 0; s_unit = -1; }
  __syncthreads();
  double carry = 0.0;
  int last_pos_unit = -1;
  for (int base = 0; base < a.nunit; base += kThreads) {
    const int i = base + static_cast<int>(threadIdx.x);
    double wu = 0.0;
    if (i < a.nunit)
      wu = unit_weight(cload(&ur[i].st_pos), cload(&ur[i].sd_pos), cload(&ur[i].st_all), residual, zt, zd);
    double total;
    const double before = carry + block_exclusive_scan(wu, &total);
    if (i < a.nunit && wu > 0.0) last_pos_unit = i;
    const bool hit = i < a.nunit && before + wu > target;
    // the first hitting thread wins
    __shared__ int s_first;
    if (threadIdx.x == 0) s_first = 0x7fffffff;
    __syncthreads();
    if (hit && !s_found) atomicMin(&s_first, i);
    __syncthreads();
    if (!s_found && s_first != 0x7fffffff && i == s_first) {
      s_unit = i;
      s_before = before;
    }
    __syncthreads();
    if (threadIdx.x == 0 && s_unit >= 0) s_found = 1;
    __syncthreads();
    carry += total;
    if (s_found) break;
  }
  if (!s_found) {  // rounding left u * W at the very top: take the last positive unit
    __shared__ int s_lp;
    if (threadIdx.x == 0) s_lp = -1;
    __syncthreads();
    if (last_pos_unit >= 0) atomicMax(&s_lp, last_pos_unit);
    __syncthreads();
    const int lp = s_lp < 0 ? 0 : s_lp;
    double bsum[1] = {0.0};
    for (int i = threadIdx.x; i < lp; i += kThreads)
      bsum[0] += unit_weight(cload(&ur[i].st_pos), cload(&ur[i].sd_pos), cload(&ur[i].st_all), residual, zt, zd);
    block_sum_doubles<1>(bsum);
    if (threadIdx.x == 0) { s_unit = lp; s_before = bsum[0]; }
    __syncthreads();
  }
  // crossing sub-span inside the unit
  if (threadIdx.x == 0) {
    const UnitRec* u = ur + s_unit;
    double ws[kWaves];
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
      ws[i] = unit_weight(cload(&u->w_pos_t[i]), cload(&u->w_pos_d[i]), cload(&u->w_all_t[i]),
                          residual, zt, zd);
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
  // fp64 scan of the crossing sub-span by one wave; lane l owns kPer elements
  if (static_cast<int>(threadIdx.x) < kWave) {
    const int lane = threadIdx.x;
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
    if (lane == 0) {
      const int tok = (hit != 0x7fffffff) ? hit : last_pos;
      a.out_tokens[static_cast<size_t>(b) * (G + 1) + d.n] = tok;
    }
  }
  __syncthreads();
  // every unit of this request has arrived and read the decision: return the
  // request's unit records and decision record to zero
  {
    unsigned long long* w = reinterpret_cast<unsigned long long*>(a.units + static_cast<size_t>(b) * a.nunit);
    const int nw = a.nunit * static_cast<int>(sizeof(UnitRec) / 8);
    for (int i = threadIdx.x; i < nw; i += kThreads) cstore(w + i, 0ull);
    unsigned long long* dw = reinterpret_cast<unsigned long long*>(a.decisions + b);
    if (static_cast<int>(threadIdx.x) < static_cast<int>(sizeof(DecisionRec) / 8)) cstore(dw + threadIdx.x, 0ull);
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// Flag of request b as seen by thread 0, broadcast to the workgroup.
__device__ inline int read_flag(const ChainArgs& a, int b) {
  __shared__ int s_f;
  if (threadIdx.x == 0) s_f = cload(&a.flag[b * kLine]);
  __syncthreads();
  const int f = s_f;
  __syncthreads();
  return f;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_fused(ChainArgs a) {
  const int R = 2 * a.gamma + 1;
  const int per_req = R * a.nchunk;
  const int nunits = a.B * a.nunit;
  int q = blockIdx.x;  // this workgroup's next draw unit
  // phase 1: row items, grid-stride; after each, run this workgroup's next
  // draw unit if its request is already decided
  for (int it = blockIdx.x; it < a.nslots; it += gridDim.x) {
    const int b = it / per_req;
    const int rem = it % per_req;
    const int k = rem / a.nchunk;
    const int c = rem % a.nchunk;
    const float T = a.temperature[b];
    if (!temp_ok(T)) {
      if (k == 0 && c == 0) {  // the whole request is invalid
        for (int i = threadIdx.x; i <= a.gamma; i += kThreads)
          a.out_tokens[static_cast<size_t>(b) * (a.gamma + 1) + i] = -1;
        if (threadIdx.x == 0) {
          a.out_n[b] = -1;
          cstore(&a.flag[b * kLine], int(kFlagDone));
        }
      }
      continue;
    }
    if (k >= needed_rows(a, T)) continue;  // draft rows are not read for this request
    row_item<DT, VEC>(a, b, k, c, T);
    if (q < nunits) {
      const int qb = q / a.nunit;
      const int f = read_flag(a, qb);
      if (f != kFlagNone) {
        draw_unit<DT, VEC>(a, qb, q % a.nunit, f);
        q += gridDim.x;
      }
    }
  }
  // phase 2: the remaining draw units, each as soon as its request is decided
  for (; q < nunits; q += gridDim.x) {
    const int qb = q / a.nunit;
    int f = read_flag(a, qb);
    for (int spins = 0, nap = 1; f == kFlagNone && spins < kSpinLimit; ++spins) {
      if (nap < 16) {
        __builtin_amdgcn_s_sleep(1);
        nap <<= 1;
      } else {
        __builtin_amdgcn_s_sleep(16);
      }
      f = read_flag(a, qb);
    }
    draw_unit<DT, VEC>(a, qb, q % a.nunit, f == kFlagNone ? int(kFlagDone) : f);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct ChainLayout {
  size_t partials, cnt_rows, cnt_units, flag, decisions, units, total;
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
  L.partials = off;  off = align_up(off + static_cast<size_t>(B) * R * nchunk * sizeof(RowPartial));
  L.cnt_rows = off;  off = align_up(off + static_cast<size_t>(B) * kLine * sizeof(int));
  L.cnt_units = off; off = align_up(off + static_cast<size_t>(B) * kLine * sizeof(int));
  L.flag = off;      off = align_up(off + static_cast<size_t>(B) * kLine * sizeof(int));
  L.decisions = off; off = align_up(off + static_cast<size_t>(B) * sizeof(DecisionRec));
  L.units = off;     off = align_up(off + static_cast<size_t>(B) * nunit * sizeof(UnitRec));
  L.total = off;
  return L;
}

// Co-resident workgroups of one kernel on the current device (cached per device).
template <int DT, bool VEC>
static int coresident_blocks() {
  static std::mutex mu;
  static std::vector<std::pair<int, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.first == dev) return e.second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_fused<DT, VEC>, kThreads, 0) != hipSuccess)
    return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  const int n = per_cu * cus;
  cache.emplace_back(dev, n);
  return n;
}

template <int DT, bool VEC>
static int launch_chain(ChainArgs a, hipStream_t stream) {
  const int cap = coresident_blocks<DT, VEC>();
  if (cap <= 0) return SV_ERR_HIP;
  const long long slots = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  if (slots > 0x7fffffffLL) return SV_ERR_SHAPE;
  a.nslots = static_cast<int>(slots);
  a.nunit = units_for(a.V, Slice<DT, VEC, 1>::kPer);
  if (static_cast<long long>(a.B) * a.nunit > 0x7fffffffLL) return SV_ERR_SHAPE;
  const int grid = static_cast<int>(std::min<long long>(cap, std::max<long long>(1, slots)));
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&chain_fused<DT, VEC>), dim3(grid),
                                 dim3(kThreads), args, 0, stream) != hipSuccess)
    return SV_ERR_HIP;
  return SV_OK;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_chain_workspace_bytes(int B, int gamma, int V, int dtype) {
  (void)dtype;
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return 0;
  return chain_layout(B, gamma, V).total;
}

extern "C" int spec_verify_chain(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 const float* temperature, int B, int gamma, int V, int dtype,
                                 int32_t* out_tokens, int32_t* out_num_accepted,
                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return SV_ERR_SHAPE;
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
  a.cnt_rows = reinterpret_cast<int*>(ws + L.cnt_rows);
  a.cnt_units = reinterpret_cast<int*>(ws + L.cnt_units);
  a.flag = reinterpret_cast<int*>(ws + L.flag);
  a.decisions = reinterpret_cast<DecisionRec*>(ws + L.decisions);
  a.units = reinterpret_cast<UnitRec*>(ws + L.units);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_chain<0, true>(a, stream) : launch_chain<0, false>(a, stream);
  return vec ? launch_chain<1, true>(a, stream) : launch_chain<1, false>(a, stream);
}
