// Debug probabilities of the chain verification step: p_i(x_i), q_i(x_i), the
// residual mass sum_k max(0, p_i - q_i) (close-reading notes 02, section 5.1:
// it equals 1 - sum_k min(p_i, q_i)) and the log-normalisers, for every draft
// position.  Not on the hot path: three launches, fp64 residual pass.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

struct ProbPartial {  // one (row, chunk) of pass 1
  float m;
  float z;
};

struct ProbsArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* temperature;
  int B, gamma, V, nchunk;
  float *p_at, *q_at, *resid, *lse_t, *lse_d;
  ProbPartial* partials;  // [B][2*gamma+1][nchunk]
  double* resid_part;     // [B][gamma][nchunk]
};

__device__ inline bool probs_temp_ok(float t) { return isfinite(t) && t >= 1.17549435e-38f; }

template <int DT>
__device__ inline const void* prow(const void* base, size_t row, int V) {
  constexpr size_t es = DT == 0 ? 2 : 4;
  return static_cast<const char*>(base) + row * static_cast<size_t>(V) * es;
}

__device__ inline const void* probs_row_of(const ProbsArgs& a, int b, int k, int dt) {
  const size_t es = dt == 0 ? 2 : 4;
  if (k <= a.gamma)
    return static_cast<const char*>(a.target) +
           (static_cast<size_t>(b) * (a.gamma + 1) + k) * static_cast<size_t>(a.V) * es;
  return static_cast<const char*>(a.draft) +
         (static_cast<size_t>(b) * a.gamma + (k - a.gamma - 1)) * static_cast<size_t>(a.V) * es;
}

// pass 1: (max, sum exp2((x - max) * log2e / T)) per (row, chunk)
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void probs_row_stats(ProbsArgs a) {
  const int R = 2 * a.gamma + 1;
  const int c = blockIdx.x % a.nchunk;
  const int r = blockIdx.x / a.nchunk;
  const int b = r / R;
  const int k = r % R;
  const float T = a.temperature[b];
  if (!probs_temp_ok(T)) return;
  const void* row = probs_row_of(a, b, k, DT);
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  Slice<DT, VEC> s;
  s.load(row, c0, c1);
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
  if (threadIdx.x == 0) a.partials[static_cast<size_t>(r) * a.nchunk + c] = ProbPartial{ms.m, ms.z};
}

// fp64 merge of one row's chunk partials: returns (max, normaliser relative to max)
__device__ inline void merge_row(const ProbPartial* p, int nchunk, double inv_t, float* m_out,
                                 double* z_out) {
  float m = -INFINITY;
  for (int c = 0; c < nchunk; ++c) m = fmaxf(m, p[c].m);
  double z = 0.0;
  for (int c = 0; c < nchunk; ++c)
    if (p[c].m != -INFINITY) z += static_cast<double>(p[c].z) * exp(static_cast<double>(p[c].m - m) * inv_t);
  *m_out = m;
  *z_out = z;
}

// pass 2: residual mass of draft position i over one chunk
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void probs_residual(ProbsArgs a) {
  __shared__ float s_m[2];
  __shared__ double s_z[2];
  const int c = blockIdx.x % a.nchunk;
  const int bi = blockIdx.x / a.nchunk;
  const int b = bi / a.gamma;
  const int i = bi % a.gamma;
  const int R = 2 * a.gamma + 1;
  const float T = a.temperature[b];
  if (!probs_temp_ok(T)) return;
  const double inv_t = 1.0 / static_cast<double>(T);
  if (threadIdx.x < 2) {
    const int k = threadIdx.x == 0 ? i : a.gamma + 1 + i;
    merge_row(a.partials + (static_cast<size_t>(b) * R + k) * a.nchunk, a.nchunk, inv_t,
              &s_m[threadIdx.x], &s_z[threadIdx.x]);
  }
  __syncthreads();
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  Slice<DT, VEC> st, sd;
  st.load(probs_row_of(a, b, i, DT), c0, c1);
  sd.load(probs_row_of(a, b, a.gamma + 1 + i, DT), c0, c1);
  double acc[1] = {0.0};
#pragma unroll
  for (int j = 0; j < st.kItems; ++j)
#pragma unroll
    for (int e = 0; e < st.kPer; ++e) {
      const double p = exp(static_cast<double>(st.x[j][e] - s_m[0]) * inv_t) / s_z[0];
      const double q = exp(static_cast<double>(sd.x[j][e] - s_m[1]) * inv_t) / s_z[1];
      acc[0] += fmax(0.0, p - q);
    }
  block_sum_doubles<1>(acc);
  if (threadIdx.x == 0) a.resid_part[static_cast<size_t>(bi) * a.nchunk + c] = acc[0];
}

// pass 3: per request, gather and finalise
template <int DT>
__global__ __launch_bounds__(kThreads) void probs_finalize(ProbsArgs a) {
  const int b = blockIdx.x;
  const int R = 2 * a.gamma + 1;
  const float T = a.temperature[b];
  const bool ok = probs_temp_ok(T);
  const double inv_t = ok ? 1.0 / static_cast<double>(T) : 0.0;
  const float nanf = __int_as_float(0x7fc00000);
  for (int k = threadIdx.x; k < R; k += kThreads) {
    float m = 0.0f;
    double z = 0.0;
    if (ok) merge_row(a.partials + (static_cast<size_t>(b) * R + k) * a.nchunk, a.nchunk, inv_t, &m, &z);
    const float lse = ok ? static_cast<float>(static_cast<double>(m) * inv_t + log(z)) : nanf;
    if (k <= a.gamma) {
      if (a.lse_t) a.lse_t[static_cast<size_t>(b) * (a.gamma + 1) + k] = lse;
    } else {
      if (a.lse_d) a.lse_d[static_cast<size_t>(b) * a.gamma + (k - a.gamma - 1)] = lse;
    }
    if (k < a.gamma) {
      // position i = k: p at the draft token, residual mass
      float pv = nanf, qv = nanf, rv = nanf;
      if (ok) {
        double r = 0.0;
        const double* rp = a.resid_part + (static_cast<size_t>(b) * a.gamma + k) * a.nchunk;
        for (int c = 0; c < a.nchunk; ++c) r += rp[c];
        rv = static_cast<float>(r);
        const int32_t x = a.tokens[static_cast<size_t>(b) * a.gamma + k];
        if (x >= 0 && x < a.V) {
          float md;
          double zd;
          merge_row(a.partials + (static_cast<size_t>(b) * R + a.gamma + 1 + k) * a.nchunk, a.nchunk,
                    inv_t, &md, &zd);
          const float xt = Elem<DT>::at(prow<DT>(a.target, static_cast<size_t>(b) * (a.gamma + 1) + k, a.V), x);
          const float xd = Elem<DT>::at(prow<DT>(a.draft, static_cast<size_t>(b) * a.gamma + k, a.V), x);
          pv = static_cast<float>(exp(static_cast<double>(xt - m) * inv_t) / z);
          qv = static_cast<float>(exp(static_cast<double>(xd - md) * inv_t) / zd);
        }
      }
      a.p_at[static_cast<size_t>(b) * a.gamma + k] = pv;
      a.q_at[static_cast<size_t>(b) * a.gamma + k] = qv;
      a.resid[static_cast<size_t>(b) * a.gamma + k] = rv;
    }
  }
  // the request's partials back to zero once every thread has read its rows
  // (thread k also reads draft row gamma + 1 + k)
  __syncthreads();
  ProbPartial* pp = a.partials + static_cast<size_t>(b) * R * a.nchunk;
  for (int i = threadIdx.x; i < R * a.nchunk; i += kThreads) pp[i] = ProbPartial{};
  double* rp = a.resid_part + static_cast<size_t>(b) * a.gamma * a.nchunk;
  for (int i = threadIdx.x; i < a.gamma * a.nchunk; i += kThreads) rp[i] = 0.0;
}

struct ProbsLayout {
  size_t partials, resid, total;
};

static ProbsLayout probs_layout(int B, int gamma, int V) {
  ProbsLayout L{};
  const size_t nchunk = static_cast<size_t>(num_chunks(V));
  L.partials = 0;
  L.resid = align_up(static_cast<size_t>(B) * (2 * static_cast<size_t>(gamma) + 1) * nchunk * sizeof(ProbPartial));
  L.total = align_up(L.resid + static_cast<size_t>(B) * gamma * nchunk * sizeof(double));
  return L;
}

template <int DT, bool VEC>
static int launch_probs(const ProbsArgs& a, hipStream_t stream) {
  const long long n1 = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  const long long n2 = static_cast<long long>(a.B) * a.gamma * a.nchunk;
  if (n1 > 0x7fffffffLL || n2 > 0x7fffffffLL) return SV_ERR_SHAPE;
  launch(SV_K_PROBS_ROW_STATS, probs_row_stats<DT, VEC>, dim3(static_cast<unsigned>(n1)), dim3(kThreads), 0, stream, a);
  if (n2 > 0)
    launch(SV_K_PROBS_RESIDUAL, probs_residual<DT, VEC>, dim3(static_cast<unsigned>(n2)), dim3(kThreads), 0, stream, a);
  launch(SV_K_PROBS_FINALIZE, probs_finalize<DT>, dim3(static_cast<unsigned>(a.B)), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_probs_workspace_bytes(int B, int gamma, int V, int dtype) {
  (void)dtype;
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return 0;
  return probs_layout(B, gamma, V).total;
}

extern "C" int spec_probs_debug(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const float* temperature, int B,
                                int gamma, int V, int dtype, float* p_at_draft, float* q_at_draft,
                                float* residual_mass, float* target_lse, float* draft_lse,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB) return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!target_logits || !temperature || !workspace) return SV_ERR_NULL;
  if (gamma > 0 && (!draft_logits || !draft_tokens || !p_at_draft || !q_at_draft || !residual_mass))
    return SV_ERR_NULL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || (draft_logits && !aligned(draft_logits, es))) return SV_ERR_ALIGN;
  const ProbsLayout L = probs_layout(B, gamma, V);
  if (workspace_bytes < L.total || !aligned(workspace, 256)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  ProbsArgs a{};
  a.target = target_logits;
  a.draft = gamma > 0 ? draft_logits : nullptr;
  a.tokens = draft_tokens;
  a.temperature = temperature;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.nchunk = num_chunks(V);
  a.p_at = p_at_draft;
  a.q_at = q_at_draft;
  a.resid = residual_mass;
  a.lse_t = target_lse;
  a.lse_d = draft_lse;
  a.partials = reinterpret_cast<ProbPartial*>(ws + L.partials);
  a.resid_part = reinterpret_cast<double*>(ws + L.resid);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_probs<0, true>(a, stream) : launch_probs<0, false>(a, stream);
  return vec ? launch_probs<1, true>(a, stream) : launch_probs<1, false>(a, stream);
}
