// Thresholds of the general consistent filter (top-k and/or top-p over the
// whole vocabulary, the same rule on the target and the draft rows: the
// close-reading notes 02, section 5.4).  One 512-thread workgroup per
// (request, row) of a sampling request finds the row's threshold t and
// stores order_key(t) + 1 (0: nothing is cut); the chain kernel then treats
// every logit below t as -inf.  See include/specverify.h for the contract.
//
// Both cuts are searches over order-preserving keys (16-bit for bf16 logits,
// whose keys differ only in their top half, 32-bit for fp32), four-way: each
// pass over the row (from the caches after the first) evaluates three probe
// keys at once, with only a block reduction, no atomics.
//  - top-k: the largest key kt with #{keys >= kt} >= min(k, V) is the k-th
//    largest logit (every logit equal to it is kept);
//  - top-p: over the keys >= kt, with Z the softmax mass of those logits, the
//    largest key kp with mass(keys >= kp) >= p * Z is the cut value v*.
// The masses are fp32 exponentials summed in fp64, so a cut can differ from
// an fp64 reference only where p lies within about 1e-7 of the mass at the
// cut.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {
namespace {

constexpr int kFilterThreads = 512;
constexpr int kFilterWaves = kFilterThreads / kWave;

struct FilterArgs {
  const void* target;
  const void* draft;
  const float* temperature;
  const int32_t* top_k;  // [B] or NULL
  const float* top_p;    // [B] or NULL
  int B, gamma, V;
  uint32_t* thr;         // [B][2 * gamma + 1]: key + 1, 0 = no cut
};

__device__ inline bool filter_temp_ok(float t) { return isfinite(t) && t >= 1.17549435e-38f; }

// Search key of a logit: bf16 keys differ only in their top 16 bits.
template <int DT>
__device__ inline uint32_t search_key(float x) {
  return DT == 0 ? (order_key(x) >> 16) : order_key(x);
}
// The full key of a search key (for bf16: the low half of a bf16 value's key
// is 0 for a positive value and 0xffff for a negative one).
template <int DT>
__device__ inline uint32_t full_key(uint32_t k) {
  return DT == 0 ? ((k << 16) | ((k & 0x8000u) ? 0u : 0xffffu)) : k;
}

// Visits every element of the row: fn(x) per element, vector loads where the
// row allows them.
template <int DT, bool VEC, typename F>
__device__ inline void for_row(const void* row, int V, F&& fn) {
  if constexpr (VEC) {
    constexpr int kv = Elem<DT>::kVec;
    const int nv = V / kv;
#pragma unroll 4
    for (int i = threadIdx.x; i < nv; i += kFilterThreads) {
      float x[kv];
      Elem<DT>::unpack(Elem<DT>::raw(row, i * kv), x);
#pragma unroll
      for (int e = 0; e < kv; ++e) fn(x[e]);
    }
  } else {
#pragma unroll 4
    for (int i = threadIdx.x; i < V; i += kFilterThreads) fn(Elem<DT>::at(row, i));
  }
}

// Block-wide sums of NV values (every thread gets the totals).
template <typename T, int NV>
__device__ inline void block_sum(T (&v)[NV], T (*s)[NV]) {
#pragma unroll
  for (int k = 0; k < NV; ++k) v[k] = wave_sum(v[k]);
  const int w = threadIdx.x / kWave;
  __syncthreads();  // the previous pass has read s
  if (threadIdx.x % kWave == 0)
#pragma unroll
    for (int k = 0; k < NV; ++k) s[w][k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    T t = s[0][k];
    for (int i = 1; i < kFilterWaves; ++i) t += s[i][k];
    v[k] = t;
  }
}

// The largest key kk in [lo, hi) whose weight W(kk) = sum of w(x) over the
// row's elements with key >= kk (and key >= floor) reaches `want`, given
// W(lo) >= want (hi is one past the largest key).  w(x) = 1 (counts, fp64 is
// exact for them) or the exponential.
template <int DT, bool VEC, bool kMass>
__device__ uint32_t search(const void* row, int V, uint32_t lo, uint32_t hi, uint32_t floor, double want,
                           float sc, float msc) {
  __shared__ double s[kFilterWaves][3];
  while (hi - lo > 1u) {
    const uint64_t span = static_cast<uint64_t>(hi) - lo;
    uint32_t q[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) q[i] = lo + static_cast<uint32_t>((span * static_cast<uint64_t>(i + 1)) / 4u);
    double acc[3] = {0.0, 0.0, 0.0};
    for_row<DT, VEC>(row, V, [&](float x) {
      const uint32_t k = search_key<DT>(x);
      if (k < floor) return;
      double wgt = 1.0;
      if constexpr (kMass) wgt = static_cast<double>(__builtin_amdgcn_exp2f(__builtin_fmaf(x, sc, -msc)));
#pragma unroll
      for (int i = 0; i < 3; ++i) acc[i] += k >= q[i] ? wgt : 0.0;
    });
    block_sum<double, 3>(acc, s);
    // W is non-increasing in the key: keep the last probe that still reaches
    // `want` as lo and the first one that does not as hi
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (q[i] <= lo || q[i] >= hi) continue;
      if (acc[i] >= want) lo = q[i];
      else { hi = q[i]; break; }
    }
  }
  return lo;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kFilterThreads) void filter_rows(FilterArgs a) {
  __shared__ uint32_t s_k[kFilterWaves][2];
  __shared__ double s_z[kFilterWaves][1];
  const int R = 2 * a.gamma + 1;
  const int b = static_cast<int>(blockIdx.x) / R;
  const int r = static_cast<int>(blockIdx.x) - b * R;
  const float T = a.temperature[b];
  if (!filter_temp_ok(T)) return;  // greedy or invalid: no cut
  if (r > a.gamma && a.draft == nullptr) return;
  int k = a.V;
  if (a.top_k) {
    k = a.top_k[b];
    if (k < 1) return;  // invalid request: the decide item reports it
    k = min(k, a.V);
  }
  float p = 1.0f;
  if (a.top_p) {
    p = a.top_p[b];
    if (!(p > 0.0f && p <= 1.0f)) return;
  }
  const bool cut_k = k < a.V, cut_p = p < 1.0f;
  if (!cut_k && !cut_p) return;
  const size_t es = Elem<DT>::kBytes;
  const void* row = r <= a.gamma
      ? static_cast<const char*>(a.target) + (static_cast<size_t>(b) * (a.gamma + 1) + r) * a.V * es
      : static_cast<const char*>(a.draft) + (static_cast<size_t>(b) * a.gamma + (r - a.gamma - 1)) * a.V * es;
  // the row's smallest and largest keys
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for_row<DT, VEC>(row, a.V, [&](float x) {
    const uint32_t kk = search_key<DT>(x);
    kmin = min(kmin, kk);
    kmax = max(kmax, kk);
  });
  // wave reductions on ints: flipping the top bit maps unsigned order to signed
  kmin = static_cast<uint32_t>(wave_min(static_cast<int>(kmin ^ 0x80000000u))) ^ 0x80000000u;
  kmax = static_cast<uint32_t>(wave_max_int(static_cast<int>(kmax ^ 0x80000000u))) ^ 0x80000000u;
  if (threadIdx.x % kWave == 0) {
    s_k[threadIdx.x / kWave][0] = kmin;
    s_k[threadIdx.x / kWave][1] = kmax;
  }
  __syncthreads();
  for (int i = 0; i < kFilterWaves; ++i) {
    kmin = min(kmin, s_k[i][0]);
    kmax = max(kmax, s_k[i][1]);
  }
  const uint32_t hi = kmax + 1u;
  uint32_t cut = kmin;
  if (cut_k) cut = search<DT, VEC, false>(row, a.V, kmin, hi, 0u, static_cast<double>(k), 0.0f, 0.0f);
  if (cut_p) {
    // exponentials relative to the row max, as the chain's stream items form them
    const float m = key_value(full_key<DT>(kmax));
    const float sc = 1.4426950408889634f / T;
    const float msc = m * sc;
    double z[1] = {0.0};
    for_row<DT, VEC>(row, a.V, [&](float x) {
      if (search_key<DT>(x) >= cut) z[0] += static_cast<double>(__builtin_amdgcn_exp2f(__builtin_fmaf(x, sc, -msc)));
    });
    block_sum<double, 1>(z, s_z);
    cut = search<DT, VEC, true>(row, a.V, cut, hi, cut, static_cast<double>(p) * z[0], sc, msc);
  }
  if (threadIdx.x == 0) a.thr[static_cast<size_t>(b) * R + r] = full_key<DT>(cut) + 1u;
}

}  // namespace

int launch_filter_rows(const void* target, const void* draft, const float* temperature, const int32_t* top_k,
                       const float* top_p, int B, int gamma, int V, int dtype, uint32_t* thr, hipStream_t stream) {
  FilterArgs a{target, gamma > 0 ? draft : nullptr, temperature, top_k, top_p, B, gamma, V, thr};
  const long long n = static_cast<long long>(B) * (2 * gamma + 1);
  if (n == 0 || (!top_k && !top_p)) return SV_OK;
  if (n > 0x7fffffffLL) return SV_ERR_SHAPE;
  const dim3 grid(static_cast<unsigned>(n));
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) {
    if (vec) launch(SV_K_FILTER_ROWS, filter_rows<0, true>, grid, dim3(kFilterThreads), 0, stream, a);
    else launch(SV_K_FILTER_ROWS, filter_rows<0, false>, grid, dim3(kFilterThreads), 0, stream, a);
  } else {
    if (vec) launch(SV_K_FILTER_ROWS, filter_rows<1, true>, grid, dim3(kFilterThreads), 0, stream, a);
    else launch(SV_K_FILTER_ROWS, filter_rows<1, false>, grid, dim3(kFilterThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv
