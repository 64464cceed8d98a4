// Token-tree verification (CMU 15-779 lecture 17 notes: section 4.3 depth-first
// linearisation, section 4.4 VerifyGreedy, section 4.5 naive sampling).  See
// include/specverify.h for the contract.
//
// Path descent: only the rows of visited nodes are read (at most max_depth+1
// per request).  One step per depth level, two launches per step:
//   tree_node_pass   one workgroup per (request, chunk) of the current node's
//                    row: argmax (greedy) or the chunk max and the fp64 sum of
//                    exp((x - max) / T) (sampling);
//   tree_choose      one workgroup per request: merges the chunk partials,
//                    picks the token (argmax, or the inverse-CDF draw with
//                    u[b][node] scanned in fp64 inside the crossing chunk),
//                    looks for a child carrying it and either descends or
//                    emits the token and stops.
// A request that has stopped costs one early-exiting workgroup per launch.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

struct TreeState {
  int32_t node;    // current node
  int32_t len;     // accepted nodes so far
  int32_t active;  // 1 while descending
  int32_t pad;
};

struct NodePartial {
  float m;       // chunk max
  int32_t arg;   // lowest index of the max (greedy)
  double s;      // sum exp((x - m) / T) over the chunk in fp64 (sampling)
};

struct TreeArgs {
  const void* logits;
  const int32_t* tokens;
  const int32_t* parents;
  const float* uniforms;
  const float* temperature;
  int B, N, V, max_depth, nchunk;
  int32_t* out_tokens;
  int32_t* out_path;
  int32_t* out_n;
  TreeState* state;
  NodePartial* partials;  // [B][nchunk]
};

__device__ inline bool tree_temp_ok(float t) { return isfinite(t) && (t == 0.0f || t >= 1.17549435e-38f); }

template <int DT>
__device__ inline const void* node_row(const TreeArgs& a, int b, int node) {
  constexpr size_t es = DT == 0 ? 2 : 4;
  return static_cast<const char*>(a.logits) +
         (static_cast<size_t>(b) * a.N + node) * static_cast<size_t>(a.V) * es;
}

// validate every request and initialise outputs and state
__global__ __launch_bounds__(kThreads) void tree_init(TreeArgs a) {
  extern __shared__ int32_t s_par[];  // N entries
  const int b = blockIdx.x;
  const int L1 = a.max_depth + 1;
  for (int i = threadIdx.x; i < L1; i += kThreads) {
    a.out_tokens[static_cast<size_t>(b) * L1 + i] = -1;
    a.out_path[static_cast<size_t>(b) * L1 + i] = -1;
  }
  const int32_t* par = a.parents + static_cast<size_t>(b) * a.N;
  const int32_t* tok = a.tokens + static_cast<size_t>(b) * a.N;
  for (int i = threadIdx.x; i < a.N; i += kThreads) s_par[i] = par[i];
  __syncthreads();
  const float T = a.temperature[b];
  int bad = !tree_temp_ok(T);
  const bool sampling = !bad && T > 0.0f;
  for (int i = threadIdx.x; i < a.N; i += kThreads) {
    if (i == 0) {
      bad |= (s_par[0] != -1);
    } else {
      const int p = s_par[i];
      bad |= (p < 0 || p >= i);
      const int32_t t = tok[i];
      bad |= (t < 0 || t >= a.V);
      // depth by walking up; more than max_depth steps means too deep
      if (p >= 0 && p < i) {
        int n = i, d = 0;
        while (n > 0 && d <= a.max_depth) {
          const int q = s_par[n];
          if (q < 0 || q >= n) { d = a.max_depth + 1; break; }
          n = q;
          ++d;
        }
        bad |= (d > a.max_depth);
      }
    }
    if (sampling) {
      const float u = a.uniforms[static_cast<size_t>(b) * a.N + i];
      bad |= !(u >= 0.0f && u < 1.0f);
    }
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    a.state[b] = TreeState{0, 0, bad ? 0 : 1, 0};
    a.out_n[b] = -1;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_node_pass(TreeArgs a) {
  const int b = blockIdx.x / a.nchunk;
  const int c = blockIdx.x % a.nchunk;
  const TreeState st = a.state[b];
  if (!st.active) return;
  const float T = a.temperature[b];
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  Slice<DT, VEC> s;
  s.load(node_row<DT>(a, b, st.node), c0, c1);
  NodePartial out{};
  if (T == 0.0f) {
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
    __shared__ float s_m;
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < s.kItems; ++j)
#pragma unroll
      for (int e = 0; e < s.kPer; ++e) m = fmaxf(m, s.x[j][e]);
    m = wave_max(m);
    __shared__ float s_wm[kWaves];
    if ((threadIdx.x % kWave) == 0) s_wm[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float mm = s_wm[0];
      for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, s_wm[w]);
      s_m = mm;
    }
    __syncthreads();
    m = s_m;
    const double inv_t = 1.0 / static_cast<double>(T);
    double acc[1] = {0.0};
    if (m != -INFINITY) {
#pragma unroll
      for (int j = 0; j < s.kItems; ++j)
#pragma unroll
        for (int e = 0; e < s.kPer; ++e) acc[0] += exp(static_cast<double>(s.x[j][e] - m) * inv_t);
    }
    block_sum_doubles<1>(acc);
    out.m = m;
    out.s = acc[0];
  }
  if (threadIdx.x == 0) a.partials[static_cast<size_t>(b) * a.nchunk + c] = out;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_choose(TreeArgs a) {
  __shared__ int s_chunk, s_hit, s_last, s_child, s_token;
  __shared__ float s_m;
  __shared__ double s_before, s_target;
  const int b = blockIdx.x;
  const TreeState st = a.state[b];
  if (!st.active) return;
  const float T = a.temperature[b];
  const NodePartial* p = a.partials + static_cast<size_t>(b) * a.nchunk;
  const bool greedy = T == 0.0f;
  if (threadIdx.x == 0) {
    s_hit = 0x7fffffff;
    s_last = -1;
    s_child = 0x7fffffff;
    if (greedy) {
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int c = 0; c < a.nchunk; ++c) best = argmax_combine(best, ArgMax{p[c].m, p[c].arg});
      s_token = best.i;
    } else {
      const double inv_t = 1.0 / static_cast<double>(T);
      float m = -INFINITY;
      for (int c = 0; c < a.nchunk; ++c) m = fmaxf(m, p[c].m);
      double S = 0.0;
      for (int c = 0; c < a.nchunk; ++c)
        if (p[c].m != -INFINITY) S += p[c].s * exp(static_cast<double>(p[c].m - m) * inv_t);
      const double target = static_cast<double>(a.uniforms[static_cast<size_t>(b) * a.N + st.node]) * S;
      double run = 0.0, before = 0.0;
      int hit = -1, last = -1;
      for (int c = 0; c < a.nchunk; ++c) {
        const double wc = (p[c].m != -INFINITY) ? p[c].s * exp(static_cast<double>(p[c].m - m) * inv_t) : 0.0;
        if (wc > 0.0) last = c;
        if (hit < 0 && run + wc > target) { hit = c; before = run; }
        run += wc;
      }
      if (hit < 0) {
        hit = last < 0 ? 0 : last;
        before = 0.0;
        for (int c = 0; c < hit; ++c)
          if (p[c].m != -INFINITY) before += p[c].s * exp(static_cast<double>(p[c].m - m) * inv_t);
      }
      s_m = m;
      s_chunk = hit;
      s_before = before;
      s_target = target;
    }
  }
  __syncthreads();
  if (!greedy) {
    const double inv_t = 1.0 / static_cast<double>(T);
    constexpr int kPerThread = kChunk / kThreads;
    const int c0 = s_chunk * kChunk;
    const int c1 = min(a.V, c0 + kChunk);
    const int k0 = c0 + static_cast<int>(threadIdx.x) * kPerThread;
    const void* row = node_row<DT>(a, b, st.node);
    double w[kPerThread];
    double mine = 0.0;
    int last_pos = -1;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int k = k0 + i;
      const double wk = (k < c1) ? exp(static_cast<double>(Elem<DT>::at(row, k) - s_m) * inv_t) : 0.0;
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
    hit = wave_min(hit);
    last_pos = wave_max_int(last_pos);
    if ((threadIdx.x % kWave) == 0) {
      atomicMin(&s_hit, hit);
      atomicMax(&s_last, last_pos);
    }
    __syncthreads();
    if (threadIdx.x == 0) s_token = (s_hit != 0x7fffffff) ? s_hit : s_last;
    __syncthreads();
  }
  const int c_tok = s_token;
  const int32_t* par = a.parents + static_cast<size_t>(b) * a.N;
  const int32_t* tok = a.tokens + static_cast<size_t>(b) * a.N;
  for (int j = st.node + 1 + threadIdx.x; j < a.N; j += kThreads)
    if (par[j] == st.node && tok[j] == c_tok) atomicMin(&s_child, j);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int L1 = a.max_depth + 1;
    const int child = s_child;
    if (child != 0x7fffffff) {
      a.out_tokens[static_cast<size_t>(b) * L1 + st.len] = c_tok;
      a.out_path[static_cast<size_t>(b) * L1 + st.len] = child;
      a.state[b] = TreeState{child, st.len + 1, 1, 0};
    } else {
      a.out_tokens[static_cast<size_t>(b) * L1 + st.len] = c_tok;
      a.out_n[b] = st.len;
      a.state[b] = TreeState{st.node, st.len, 0, 0};
    }
  }
}

struct TreeLayout {
  size_t state, partials, total;
};

static TreeLayout tree_layout(int B, int V) {
  TreeLayout L{};
  L.state = 0;
  L.partials = align_up(static_cast<size_t>(B) * sizeof(TreeState));
  L.total = align_up(L.partials + static_cast<size_t>(B) * num_chunks(V) * sizeof(NodePartial));
  return L;
}

template <int DT, bool VEC>
static int launch_tree(const TreeArgs& a, hipStream_t stream) {
  const long long n = static_cast<long long>(a.B) * a.nchunk;
  if (n > 0x7fffffffLL) return SV_ERR_SHAPE;
  launch(SV_K_TREE_INIT, tree_init, dim3(a.B), dim3(kThreads), a.N * sizeof(int32_t), stream, a);
  for (int step = 0; step <= a.max_depth; ++step) {
    launch(SV_K_TREE_NODE_PASS, tree_node_pass<DT, VEC>, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream, a);
    launch(SV_K_TREE_CHOOSE, tree_choose<DT>, dim3(a.B), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_tree_workspace_bytes(int B, int N, int V, int dtype) {
  (void)dtype;
  (void)N;
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB) return 0;
  return tree_layout(B, V).total;
}

extern "C" int spec_verify_tree(const void* target_logits, const int32_t* node_tokens,
                                const int32_t* parents, const float* uniforms,
                                const float* temperature, int B, int N, int V, int max_depth,
                                int dtype, int32_t* out_tokens, int32_t* out_path_nodes,
                                int32_t* out_num_accepted, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || max_depth < 0 ||
      max_depth > SV_MAX_TREE_DEPTH)
    return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!target_logits || !node_tokens || !parents || !uniforms || !temperature || !out_tokens ||
      !out_path_nodes || !out_num_accepted || !workspace)
    return SV_ERR_NULL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, es)) return SV_ERR_ALIGN;
  const TreeLayout L = tree_layout(B, V);
  if (workspace_bytes < L.total || !aligned(workspace, 256)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  TreeArgs a{};
  a.logits = target_logits;
  a.tokens = node_tokens;
  a.parents = parents;
  a.uniforms = uniforms;
  a.temperature = temperature;
  a.B = B;
  a.N = N;
  a.V = V;
  a.max_depth = max_depth;
  a.nchunk = num_chunks(V);
  a.out_tokens = out_tokens;
  a.out_path = out_path_nodes;
  a.out_n = out_num_accepted;
  a.state = reinterpret_cast<TreeState*>(ws + L.state);
  a.partials = reinterpret_cast<NodePartial*>(ws + L.partials);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16);
  if (dtype == SV_BF16) return vec ? launch_tree<0, true>(a, stream) : launch_tree<0, false>(a, stream);
  return vec ? launch_tree<1, true>(a, stream) : launch_tree<1, false>(a, stream);
}
