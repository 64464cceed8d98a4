// Chain verification: the acceptance stage of one speculative-decoding round
// for a batch of requests (Leviathan et al.'s Algorithm 1 as restated in the
// close-reading notes 02, section 4, and CMU 15-779 lecture 17 notes, sections
// 2.2-2.4).  See include/specverify.h for the contract.
//
// Three launches on the caller's stream:
//  1. chain_row_stats   one workgroup per needed (row, chunk): the chunk max
//                       and, for sampling rows, sum exp2((x - max) * log2e/T)
//                       in fp32; for greedy rows the argmax (lowest index).
//                       Draft rows of greedy requests are not read.
//  2. chain_decide_draw one workgroup per (request, chunk): every workgroup of
//                       a request merges the row partials (fp64), runs the
//                       gamma-step accept test and derives the same decision;
//                       chunk 0 writes the accepted tokens and the count; for
//                       sampling requests each workgroup accumulates, in fp64,
//                       the final draw's weights over its chunk.
//  3. chain_final_draw  one workgroup per request: locates the chunk where the
//                       running weight crosses u * W and scans it in fp64.
//
// Precision: the accept test needs p(x)/q(x) to ~1e-6 and uses the fp32
// normalisers of pass 1.  The final draw is computed from fp64 exponentials
// of the same rows with fp64 normalisers taken in the draw pass itself, so
// the inverse CDF matches an fp64 reference except where u lies within a few
// ulps of a CDF step.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

struct RowPartial {  // one (row, chunk)
  float m;           // chunk max
  int32_t arg;       // lowest index of the max (greedy rows)
  float z;           // sum of exp2((x - m) * log2e / T) (sampling rows)
  float pad;
};

enum : int32_t { kModeDone = 0, kModeResidual = 1, kModeBonus = 2 };

struct DecisionRec {  // per request, written by chunk 0 of pass 2
  int32_t mode;
  int32_t n;
  float mt, md;      // row maxima of the final draw's rows
  double zt, zd;     // pass-1 normalisers of those rows (fp64 merge)
  float u;           // u[b][gamma]
  float t;           // temperature
  double pad;
};

struct DrawPartial {  // per (request, chunk) of the final draw
  double st_all, sd_all, st_pos, sd_pos;
};

struct ChainArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;
  int B, gamma, V, nchunk;
  int32_t* out_tokens;
  int32_t* out_n;
  RowPartial* partials;
  DecisionRec* decisions;
  DrawPartial* draws;
};

// T must be 0 (greedy) or a finite positive normal float.
__device__ inline bool temp_ok(float t) { return isfinite(t) && (t == 0.0f || t >= 1.17549435e-38f); }

template <int DT>
__device__ inline const void* row_ptr(const void* base, size_t row, int V) {
  constexpr size_t es = DT == 0 ? 2 : 4;
  return static_cast<const char*>(base) + row * static_cast<size_t>(V) * es;
}

// ---------------------------------------------------------------------------
// pass 1: row statistics
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_row_stats(ChainArgs a) {
  const int R = 2 * a.gamma + 1;
  const int item = blockIdx.x;
  const int c = item % a.nchunk;
  const int r = item / a.nchunk;
  const int b = r / R;
  const int k = r % R;
  const float T = a.temperature[b];
  if (!temp_ok(T)) return;
  const bool sampling = T > 0.0f;
  const void* row;
  if (k <= a.gamma) {
    row = row_ptr<DT>(a.target, static_cast<size_t>(b) * (a.gamma + 1) + k, a.V);
  } else {
    if (!sampling || a.draft == nullptr) return;
    row = row_ptr<DT>(a.draft, static_cast<size_t>(b) * a.gamma + (k - a.gamma - 1), a.V);
  }
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  Slice<DT, VEC> s;
  s.load(row, c0, c1);
  RowPartial out{};
  if (!sampling) {
    ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
    for (int j = 0; j < s.kItems; ++j)
#pragma unroll
      for (int e = 0; e < s.kPer; ++e) {
        const int idx = s.index(c0, j, e);
        if (idx < c1) best = argmax_combine(best, ArgMax{s.x[j][e], idx});
      }
    best = block_argmax(best);
    out.m = best.v;
    out.arg = best.i;
  } else {
    const float sc = 1.4426950408889634f / T;
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < s.kItems; ++j)
#pragma unroll
      for (int e = 0; e < s.kPer; ++e) m = fmaxf(m, s.x[j][e]);
    float z = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int j = 0; j < s.kItems; ++j)
#pragma unroll
        for (int e = 0; e < s.kPer; ++e) z += __builtin_amdgcn_exp2f((s.x[j][e] - m) * sc);
    }
    const MaxSum ms = block_maxsum(MaxSum{m, z}, sc);
    out.m = ms.m;
    out.z = ms.z;
  }
  if (threadIdx.x == 0) a.partials[static_cast<size_t>(r) * a.nchunk + c] = out;
}

// ---------------------------------------------------------------------------
// the per-request decision (every workgroup of a request computes it)
// ---------------------------------------------------------------------------
struct Decision {
  int32_t mode;   // kModeDone / kModeResidual / kModeBonus, or -1 invalid
  int32_t n;
  int32_t final_token;  // greedy: the argmax token; else unused
  float mt, md;
  double zt, zd;
  float u, t;
};

__device__ inline double exp_scaled(float x, float m, double inv_t) {
  return exp(static_cast<double>(x - m) * inv_t);
}

template <int DT>
__device__ Decision decide_request(const ChainArgs& a, int b) {
  __shared__ float s_m[2 * SV_MAX_GAMMA + 1];
  __shared__ double s_z[2 * SV_MAX_GAMMA + 1];
  __shared__ int32_t s_arg[2 * SV_MAX_GAMMA + 1];
  __shared__ int32_t s_ok[SV_MAX_GAMMA + 1];
  __shared__ Decision s_dec;
  const int tid = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  const bool tok_ok_t = temp_ok(T);
  const bool sampling = tok_ok_t && T > 0.0f;
  // validity of tokens and uniforms
  int bad = 0;
  if (tid < G) {
    const int32_t x = a.tokens[static_cast<size_t>(b) * G + tid];
    bad |= (x < 0 || x >= a.V);
  }
  if (sampling && tid <= G) {
    const float u = a.uniforms[static_cast<size_t>(b) * (G + 1) + tid];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  if (sampling && G > 0 && a.draft == nullptr) bad = 1;
  bad = __syncthreads_or(bad);
  if (!tok_ok_t || bad) {
    Decision d{};
    d.mode = -1;
    return d;
  }
  // merge the chunk partials of every needed row
  const int nrows = sampling ? R : G + 1;
  if (tid < nrows) {
    const RowPartial* p = a.partials + (static_cast<size_t>(b) * R + tid) * a.nchunk;
    if (!sampling) {
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int c = 0; c < a.nchunk; ++c) best = argmax_combine(best, ArgMax{p[c].m, p[c].arg});
      s_m[tid] = best.v;
      s_arg[tid] = best.i;
    } else {
      float m = -INFINITY;
      for (int c = 0; c < a.nchunk; ++c) m = fmaxf(m, p[c].m);
      const double inv_t = 1.0 / static_cast<double>(T);
      double z = 0.0;
      for (int c = 0; c < a.nchunk; ++c)
        if (p[c].m != -INFINITY) z += static_cast<double>(p[c].z) * exp_scaled(p[c].m, m, inv_t);
      s_m[tid] = m;
      s_z[tid] = z;
    }
  }
  __syncthreads();
  // per-position accept flags
  if (tid < G) {
    const int32_t x = a.tokens[static_cast<size_t>(b) * G + tid];
    int ok;
    if (!sampling) {
      ok = (x == s_arg[tid]);
    } else {
      const double inv_t = 1.0 / static_cast<double>(T);
      const float xt = Elem<DT>::at(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + tid, a.V), x);
      const float xd = Elem<DT>::at(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + tid, a.V), x);
      const double p = exp_scaled(xt, s_m[tid], inv_t) / s_z[tid];
      const double q = exp_scaled(xd, s_m[G + 1 + tid], inv_t) / s_z[G + 1 + tid];
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
    Decision d{};
    d.n = n;
    d.t = T;
    if (!sampling) {
      d.mode = kModeDone;
      d.final_token = s_arg[n];
    } else {
      d.u = a.uniforms[static_cast<size_t>(b) * (G + 1) + G];
      d.mt = s_m[n];
      d.zt = s_z[n];
      if (n < G) {
        d.mode = kModeResidual;
        d.md = s_m[G + 1 + n];
        d.zd = s_z[G + 1 + n];
      } else {
        d.mode = kModeBonus;
      }
    }
    s_dec = d;
  }
  __syncthreads();
  const Decision d = s_dec;
  __syncthreads();
  return d;
}

// ---------------------------------------------------------------------------
// pass 2: decision + fp64 weight sums of the final draw over one chunk
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_decide_draw(ChainArgs a) {
  const int b = blockIdx.x / a.nchunk;
  const int c = blockIdx.x % a.nchunk;
  const int G = a.gamma;
  const Decision d = decide_request<DT>(a, b);
  if (c == 0) {
    int32_t* out = a.out_tokens + static_cast<size_t>(b) * (G + 1);
    for (int i = threadIdx.x; i <= G; i += kThreads) {
      int32_t v = -1;
      if (d.mode >= 0) {
        if (i < d.n) v = a.tokens[static_cast<size_t>(b) * G + i];
        else if (i == d.n && d.mode == kModeDone) v = d.final_token;
      }
      out[i] = v;
    }
    if (threadIdx.x == 0) {
      a.out_n[b] = d.mode >= 0 ? d.n : -1;
      DecisionRec rec{};
      rec.mode = d.mode;
      rec.n = d.n;
      rec.mt = d.mt;
      rec.md = d.md;
      rec.zt = d.zt;
      rec.zd = d.zd;
      rec.u = d.u;
      rec.t = d.t;
      a.decisions[b] = rec;
    }
  }
  if (d.mode != kModeResidual && d.mode != kModeBonus) return;
  const double inv_t = 1.0 / static_cast<double>(d.t);
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (d.mode == kModeBonus) {
    Slice<DT, VEC> st;
    st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + G, a.V), c0, c1);
#pragma unroll
    for (int j = 0; j < st.kItems; ++j)
#pragma unroll
      for (int e = 0; e < st.kPer; ++e) acc[0] += exp_scaled(st.x[j][e], d.mt, inv_t);
  } else {
    Slice<DT, VEC> st, sd;
    st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + d.n, a.V), c0, c1);
    sd.load(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V), c0, c1);
#pragma unroll
    for (int j = 0; j < st.kItems; ++j)
#pragma unroll
      for (int e = 0; e < st.kPer; ++e) {
        const double et = exp_scaled(st.x[j][e], d.mt, inv_t);
        const double ed = exp_scaled(sd.x[j][e], d.md, inv_t);
        acc[0] += et;
        acc[1] += ed;
        if (et * d.zd > ed * d.zt) {  // p > q under the pass-1 normalisers
          acc[2] += et;
          acc[3] += ed;
        }
      }
  }
  block_sum_doubles<4>(acc);
  if (threadIdx.x == 0)
    a.draws[static_cast<size_t>(b) * a.nchunk + c] = DrawPartial{acc[0], acc[1], acc[2], acc[3]};
}

// ---------------------------------------------------------------------------
// pass 3: locate the crossing chunk, scan it in fp64
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void chain_final_draw(ChainArgs a) {
  __shared__ int s_chunk;
  __shared__ double s_before, s_target, s_zt, s_zd;
  __shared__ int s_hit, s_last;
  const int b = blockIdx.x;
  const int G = a.gamma;
  const DecisionRec rec = a.decisions[b];
  if (rec.mode != kModeResidual && rec.mode != kModeBonus) return;
  const DrawPartial* dp = a.draws + static_cast<size_t>(b) * a.nchunk;
  // the residual's target row is the rejected position's; the bonus uses row gamma
  const int trow_index = rec.mode == kModeResidual ? rec.n : G;
  __shared__ int s_resid;
  if (threadIdx.x == 0) {
    double zt = 0.0, zd = 0.0;
    for (int c = 0; c < a.nchunk; ++c) { zt += dp[c].st_all; zd += dp[c].sd_all; }
    bool residual = rec.mode == kModeResidual;
    double W = 0.0;
    if (residual) {
      for (int c = 0; c < a.nchunk; ++c) W += dp[c].st_pos / zt - dp[c].sd_pos / zd;
      // an empty residual (p and q equal up to rounding) draws from p of that position
      if (!(W > 0.0)) residual = false;
    }
    if (!residual) {
      W = 0.0;
      for (int c = 0; c < a.nchunk; ++c) W += dp[c].st_all;
    }
    const double target = static_cast<double>(rec.u) * W;
    double run = 0.0;
    int hit = -1, last = -1;
    double before = 0.0;
    for (int c = 0; c < a.nchunk; ++c) {
      const double wc = residual ? (dp[c].st_pos / zt - dp[c].sd_pos / zd) : dp[c].st_all;
      if (wc > 0.0) last = c;
      if (hit < 0 && run + wc > target) { hit = c; before = run; }
      run += wc;
    }
    if (hit < 0) {  // rounding left u * W at the very top: use the last positive chunk
      hit = last < 0 ? 0 : last;
      before = 0.0;
      for (int c = 0; c < hit; ++c)
        before += residual ? (dp[c].st_pos / zt - dp[c].sd_pos / zd) : dp[c].st_all;
    }
    s_resid = residual ? 1 : 0;
    s_chunk = hit;
    s_before = before;
    s_target = target;
    s_zt = zt;
    s_zd = zd;
    s_hit = 0x7fffffff;
    s_last = -1;
  }
  __syncthreads();
  const int c0 = s_chunk * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  // each thread scans kChunk / kThreads consecutive elements
  constexpr int kPerThread = kChunk / kThreads;
  const int k0 = c0 + static_cast<int>(threadIdx.x) * kPerThread;
  const double inv_t = 1.0 / static_cast<double>(rec.t);
  const bool residual = s_resid != 0;
  const void* trow = row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow_index, a.V);
  const void* drow = residual ? row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + rec.n, a.V) : nullptr;
  double w[kPerThread];
  double mine = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int k = k0 + i;
    double wk = 0.0;
    if (k < c1) {
      const double et = exp_scaled(Elem<DT>::at(trow, k), rec.mt, inv_t);
      if (residual) {
        const double ed = exp_scaled(Elem<DT>::at(drow, k), rec.md, inv_t);
        wk = fmax(0.0, et / s_zt - ed / s_zd);
      } else {
        wk = et;
      }
    }
    w[i] = wk;
    mine += wk;
    if (wk > 0.0) last_pos = k;
  }
  double total;
  double run = s_before + block_exclusive_scan(mine, &total);
  int hit = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    run += w[i];
    if (hit == 0x7fffffff && w[i] > 0.0 && run > s_target) hit = k0 + i;
  }
  if (hit != 0x7fffffff) atomicMin(&s_hit, hit);
  if (last_pos >= 0) atomicMax(&s_last, last_pos);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tok = (s_hit != 0x7fffffff) ? s_hit : s_last;
    a.out_tokens[static_cast<size_t>(b) * (G + 1) + rec.n] = tok;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct ChainLayout {
  size_t partials, decisions, draws, total;
};

static ChainLayout chain_layout(int B, int gamma, int V) {
  ChainLayout L{};
  const size_t nchunk = static_cast<size_t>(num_chunks(V));
  const size_t R = 2 * static_cast<size_t>(gamma) + 1;
  L.partials = 0;
  L.decisions = align_up(L.partials + static_cast<size_t>(B) * R * nchunk * sizeof(RowPartial));
  L.draws = align_up(L.decisions + static_cast<size_t>(B) * sizeof(DecisionRec));
  L.total = align_up(L.draws + static_cast<size_t>(B) * nchunk * sizeof(DrawPartial));
  return L;
}

template <int DT, bool VEC>
static int launch_chain(const ChainArgs& a, hipStream_t stream) {
  const int R = 2 * a.gamma + 1;
  const long long n1 = static_cast<long long>(a.B) * R * a.nchunk;
  const long long n2 = static_cast<long long>(a.B) * a.nchunk;
  if (n1 > 0x7fffffffLL || n2 > 0x7fffffffLL) return SV_ERR_SHAPE;
  hipLaunchKernelGGL((chain_row_stats<DT, VEC>), dim3(static_cast<unsigned>(n1)), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL((chain_decide_draw<DT, VEC>), dim3(static_cast<unsigned>(n2)), dim3(kThreads), 0, stream, a);
  hipLaunchKernelGGL((chain_final_draw<DT>), dim3(static_cast<unsigned>(a.B)), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
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
  a.decisions = reinterpret_cast<DecisionRec*>(ws + L.decisions);
  a.draws = reinterpret_cast<DrawPartial*>(ws + L.draws);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_chain<0, true>(a, stream) : launch_chain<0, false>(a, stream);
  return vec ? launch_chain<1, true>(a, stream) : launch_chain<1, false>(a, stream);
}
