// Token-tree verification (CMU 15-779 lecture 17 notes: section 4.3 depth-first
// linearisation, section 4.4 VerifyGreedy, section 4.5 naive sampling).  See
// include/specverify.h for the contract.
//
// Path descent: only the rows of visited nodes are read (at most max_depth+1
// per request).
//
// One launch, `tree_verify`, of one-wave workgroups that loop over the depth
// levels: per request a choose workgroup and one stream workgroup per
// 2048-logit chunk of a row.  The choose workgroup validates the request and
// publishes the root as its level-0 node.  At each level every stream
// workgroup reduces its chunk of that level's node row -- the chunk max and
// argmax (greedy), or the chunk max and the fp64 sums of exp((x - max) / T)
// of each lane's logits (sampling) -- and the choose workgroup merges them,
// picks the token (argmax, or the inverse-CDF draw narrowed chunk -> lane ->
// logit), looks for the child that carries it and publishes that child as the
// next level's node, or stops the request.  A chunk word is tagged with its
// level, so one buffer serves every level without clearing; once the request
// stops, each stream workgroup returns its chunk's words to zero and the last
// workgroup of the request its control words.  The grid is B * (nchunk + 1)
// workgroups whatever the depth.
//
// Shapes whose grid or chunk count is too large for one launch use the
// multi-launch form: one step per depth level, two launches per step:
//   tree_node_pass   one workgroup per (request, chunk) of the current node's
//                    row: argmax (greedy) or the chunk max and the fp64 sum of
//                    exp((x - max) / T) (sampling);
//   tree_choose      one workgroup per request: merges the chunk partials,
//                    picks the token (argmax, or the inverse-CDF draw with
//                    u[b][node] scanned in fp64 inside the crossing chunk),
//                    looks for a child carrying it and either descends or
//                    emits the token and stops.
// A request that has stopped costs one early-exiting workgroup per launch.
#include <stdlib.h>

#include <algorithm>

#include "sv_device.hpp"
#include "sv_host.hpp"
#include "sv_tree_common.hpp"

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
  int last;               // set for the last tree_choose launch: it returns the workspace to zero
};


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

// One chunk's partial of a node row: the max and lowest-index argmax
// (greedy, T == 0) or the max and the fp64 sum of exp((x - max) / T).
template <int DT, bool VEC>
__device__ NodePartial chunk_partial(const Slice<DT, VEC>& s, int c0, int c1, float T) {
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
  return out;
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
  const NodePartial out = chunk_partial(s, c0, c1, T);
  if (threadIdx.x == 0) a.partials[static_cast<size_t>(b) * a.nchunk + c] = out;
}

// The request's node partials back to zero (the last step, once they are read).
__device__ inline void tree_clear_partials(const TreeArgs& a, int b) {
  NodePartial* p = a.partials + static_cast<size_t>(b) * a.nchunk;
  for (int c = threadIdx.x; c < a.nchunk; c += kThreads) p[c] = NodePartial{};
}

// The choice at request b's node st.node from that node's chunk partials p:
// the token (argmax, or the inverse-CDF draw narrowed to a chunk and scanned
// there in fp64 with u[b][node]), and the child carrying it.  Writes the
// request's outputs for this level and returns its next state (inactive once
// it stops).  With `clear`, p is zeroed once read.  Called by every thread of
// the workgroup.
template <int DT>
__device__ TreeState choose_at(const TreeArgs& a, int b, const TreeState st, NodePartial* p, bool clear) {
  __shared__ int s_chunk, s_hit, s_last, s_child, s_token;
  __shared__ float s_m;
  __shared__ double s_before, s_target;
  const float T = a.temperature[b];
  const bool greedy = T == 0.0f;
  __syncthreads();  // a previous choice's readers of the shared words are done
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
  if (clear)  // only thread 0 read them, before the barrier
    for (int c = threadIdx.x; c < a.nchunk; c += kThreads) p[c] = NodePartial{};
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
  const int L1 = a.max_depth + 1;
  const int child = s_child;
  if (threadIdx.x == 0) {
    a.out_tokens[static_cast<size_t>(b) * L1 + st.len] = c_tok;
    if (child != 0x7fffffff) a.out_path[static_cast<size_t>(b) * L1 + st.len] = child;
    else a.out_n[b] = st.len;
  }
  return child != 0x7fffffff ? TreeState{child, st.len + 1, 1, 0} : TreeState{st.node, st.len, 0, 0};
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_choose(TreeArgs a) {
  const int b = blockIdx.x;
  const TreeState st = a.state[b];
  NodePartial* p = a.partials + static_cast<size_t>(b) * a.nchunk;
  if (!st.active) {
    // every thread has read active == 0, so zeroing the state splits no one
    if (a.last) {
      tree_clear_partials(a, b);
      if (threadIdx.x == 0) a.state[b] = TreeState{};
    }
    return;
  }
  const TreeState next = choose_at<DT>(a, b, st, p, a.last);
  if (threadIdx.x == 0) a.state[b] = a.last ? TreeState{} : next;
}

// ---------------------------------------------------------------------------
// all-nodes statistics (a test control: the design that reduces every node's
// row up front, measured against path descent)
// ---------------------------------------------------------------------------
// tree_all_pass: one workgroup per (request, node, chunk), the chunk partials
// of every node of every valid request (all B * N rows read); tree_all_descend:
// one workgroup per request, the choices level by level from those partials
// (the draw's crossing chunk read again), then its partials and state back to
// zero.  Partials: [B][N][nchunk].
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void tree_all_pass(TreeArgs a) {
  const int c = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.nchunk));
  const long long bn = blockIdx.x / static_cast<unsigned>(a.nchunk);
  const int b = static_cast<int>(bn / a.N);
  const int node = static_cast<int>(bn - static_cast<long long>(b) * a.N);
  if (!a.state[b].active) return;
  const float T = a.temperature[b];
  const int c0 = c * kChunk;
  const int c1 = min(a.V, c0 + kChunk);
  Slice<DT, VEC> s;
  s.load(node_row<DT>(a, b, node), c0, c1);
  const NodePartial out = chunk_partial(s, c0, c1, T);
  if (threadIdx.x == 0) a.partials[static_cast<size_t>(bn) * a.nchunk + c] = out;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void tree_all_descend(TreeArgs a) {
  const int b = blockIdx.x;
  TreeState st = a.state[b];
  NodePartial* p = a.partials + static_cast<size_t>(b) * a.N * a.nchunk;
  while (st.active) st = choose_at<DT>(a, b, st, p + static_cast<size_t>(st.node) * a.nchunk, false);
  __syncthreads();
  for (long long i = threadIdx.x; i < static_cast<long long>(a.N) * a.nchunk; i += kThreads) p[i] = NodePartial{};
  if (threadIdx.x == 0) a.state[b] = TreeState{};
}

// ---------------------------------------------------------------------------
// single launch
// ---------------------------------------------------------------------------
constexpr int kCtlNode = 0, kCtlStop = 1, kCtlExit = 2;

struct TreeFused {
  const void* logits;
  const int32_t* tokens;
  const int32_t* parents;
  const float* uniforms;
  const float* temperature;
  int B, N, V, max_depth, nchunk;  // nchunk: chunks of kTreeChunk logits
  int32_t* out_tokens;
  int32_t* out_path;
  int32_t* out_n;
  uint64_t* ctl;     // [B][kCtlStride]: node word, stop word and exit count of each request
  uint64_t* chunks;  // [B][nchunk]: level-tagged chunk max (and argmax)
  double* totals;    // [B][nchunk]: fp64 exp-sum of the chunk relative to its max (sampling)
  double* lanes;     // [B][nchunk][kWave]: the same per lane (sampling)
  uint32_t spin;     // poll bound of every wait (kTreeSpinLimit unless a test lowers it)
};

__device__ inline int levels_of(const TreeFused& a) { return a.max_depth + 1; }

template <int DT>
__device__ inline const void* fused_row(const TreeFused& a, int b, int node) {
  return static_cast<const char*>(a.logits) +
         (static_cast<size_t>(b) * a.N + node) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
}

// Control words of request b: the node word (marked, the level above bit 32,
// the node below it), the stop word (marked once the request has stopped)
// and the count of the request's workgroups that are done with both.
__device__ inline uint64_t* tree_ctl(const TreeFused& a, int b) { return a.ctl + static_cast<size_t>(b) * kCtlStride; }
__device__ inline uint64_t node_word(int level, int node) {
  return kTreeMark | (static_cast<uint64_t>(level) << 32) | static_cast<uint32_t>(node);
}

// Waits until request b's node word is that of level d (returns the node) or
// the request has stopped (-1); -2 if the wait gave up.
__device__ int tree_wait_node(const TreeFused& a, int b, int d) {
  const uint64_t* cw = tree_ctl(a, b);
  const uint64_t want = node_word(d, 0) >> 32;
  for (uint32_t spin = 0; spin < a.spin; ++spin) {
    const uint64_t nv = load_coherent(cw + kCtlNode);
    const uint64_t sv = load_coherent(cw + kCtlStop);
    if ((nv >> 32) == want) return static_cast<int>(static_cast<uint32_t>(nv));
    if (sv & kTreeMark) return -1;
    __builtin_amdgcn_s_sleep(2);
  }
  return -2;
}

// A workgroup of request b is done with the request; the last of its
// nchunk + 1 workgroups returns the control words to zero.
__device__ inline void tree_exit(const TreeFused& a, int b) {
  if (threadIdx.x != 0) return;
  uint64_t* cw = tree_ctl(a, b);
  if (arrive(reinterpret_cast<uint32_t*>(cw + kCtlExit)) == static_cast<uint32_t>(a.nchunk)) {
    store_coherent(cw + kCtlNode, 0ull);
    store_coherent(cw + kCtlStop, 0ull);
    store_coherent(cw + kCtlExit, 0ull);
  }
}

// Validation (as tree_init), by the choose workgroup before level 0: a valid
// request gets the root as its level-0 node, an invalid one its -1 outputs
// and the stop.  Every output word of a request is written by its choose
// workgroup alone, so no two XCDs' caches ever hold the same output bytes.
__device__ bool tree_validate(const TreeFused& a, int b) {
  __shared__ int32_t s_par[SV_MAX_TREE_NODES];
  const int lane = threadIdx.x;
  const int L1 = levels_of(a);
  const int32_t* par = a.parents + static_cast<size_t>(b) * a.N;
  const int32_t* tok = a.tokens + static_cast<size_t>(b) * a.N;
  for (int i = lane; i < a.N; i += kWave) s_par[i] = par[i];
  __syncthreads();
  const float T = a.temperature[b];
  int bad = !tree_temp_ok(T);
  const bool sampling = !bad && T > 0.0f;
  for (int i = lane; i < a.N; i += kWave) {
    if (i == 0) {
      bad |= (s_par[0] != -1);
    } else {
      const int p = s_par[i];
      bad |= (p < 0 || p >= i);
      const int32_t t = tok[i];
      bad |= (t < 0 || t >= a.V);
      if (p >= 0 && p < i) {
        int n = i, depth = 0;
        while (n > 0 && depth <= a.max_depth) {
          const int q = s_par[n];
          if (q < 0 || q >= n) { depth = a.max_depth + 1; break; }
          n = q;
          ++depth;
        }
        bad |= (depth > a.max_depth);
      }
    }
    if (sampling) {
      const float u = a.uniforms[static_cast<size_t>(b) * a.N + i];
      bad |= !(u >= 0.0f && u < 1.0f);
    }
  }
  const bool any_bad = __any(bad);
  if (any_bad) {
    for (int i = lane; i < L1; i += kWave) {
      a.out_tokens[static_cast<size_t>(b) * L1 + i] = -1;
      a.out_path[static_cast<size_t>(b) * L1 + i] = -1;
    }
    if (lane == 0) {
      a.out_n[b] = -1;
      store_coherent(tree_ctl(a, b) + kCtlStop, kTreeMark);
    }
  } else if (lane == 0) {
    store_coherent(tree_ctl(a, b) + kCtlNode, node_word(0, 0));
  }
  return !any_bad;
}

// Chunk c of the row of node `node`, the level-d node of request b.
template <int DT, bool VEC>
__device__ void tree_stream_chunk(const TreeFused& a, int b, int d, int c, int node, float T) {
  using Raw = LaneRun<DT, VEC>;
  const int c0 = c * kTreeChunk;
  const int c1 = min(a.V, c0 + kTreeChunk);
  Raw raw;
  raw.load(fused_row<DT>(a, b, node), c0, c1);
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
    for (int e = 0; e < Raw::kPer; ++e) m = fmaxf(m, raw.at(j, e));
  m = wave_max(m);
  const size_t slot = static_cast<size_t>(b) * a.nchunk + c;
  if (T == 0.0f) {
    int idx = 0x7fffffff;
#pragma unroll
    for (int j = Raw::kItems - 1; j >= 0; --j)
#pragma unroll
      for (int e = Raw::kPer - 1; e >= 0; --e) {
        const int k = Raw::index(c0, j, e);
        if (k < c1 && raw.at(j, e) == m) idx = k;
      }
    idx = wave_min(idx);
    if (threadIdx.x == 0) store_coherent(a.chunks + slot, tree_chunk_word(d, m, idx));
    return;
  }
  // sampling: fp64 sums of exp((x - m) / T) per lane and over the chunk
  const double l2t = kLog2e / static_cast<double>(T);
  const double ml2t = static_cast<double>(m) * l2t;
  double sl = 0.0;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
      for (int e = 0; e < Raw::kPer; ++e)
        sl += exp2_neg(__builtin_fma(static_cast<double>(raw.at(j, e)), l2t, -ml2t));
  }
  store_coherent(reinterpret_cast<uint64_t*>(a.lanes) + slot * kWave + threadIdx.x, tag_sum(sl, d));
  const double tot = wave_sum(sl);
  if (threadIdx.x == 0) {
    store_coherent(reinterpret_cast<uint64_t*>(a.totals) + slot, tag_sum(tot, d));
    store_coherent(a.chunks + slot, tree_chunk_word(d, m, 0));
  }
}

// The choice at level d of request b, whose node there is `node`: returns
// the child it descends to (published as the next level's node), or -1 once
// the request has stopped (the stop published).
template <int DT, bool VEC>
__device__ int tree_choose_level(const TreeFused& a, int b, int d, int node, float T) {
  constexpr int kLaneElems = LaneRun<DT, VEC>::kRun;  // logits per lane of a chunk
  const int lane = threadIdx.x;
  const bool greedy = T == 0.0f;
  const float u = greedy ? 0.0f : a.uniforms[static_cast<size_t>(b) * a.N + node];
  // the first kWave nodes' parents and tokens, loaded while the chunks finish
  const int32_t* par = a.parents + static_cast<size_t>(b) * a.N;
  const int32_t* tk = a.tokens + static_cast<size_t>(b) * a.N;
  const int32_t my_par = lane < a.N ? par[lane] : -1;
  const int32_t my_tok = lane < a.N ? tk[lane] : -1;
  // every chunk word of this level (lane l holds chunks l, l + kWave, ...)
  uint64_t w[kTreeChunkCache];
  bool lost = false;
  for (uint32_t spin = 0;; ++spin) {
    bool all = true;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q) {
      const int c = q * kWave + lane;
      w[q] = c < a.nchunk ? load_coherent(a.chunks + static_cast<size_t>(b) * a.nchunk + c) : 0ull;
      all = all && (c >= a.nchunk || chunk_at_level(w[q], d));
    }
    if (__all(all)) break;
    if (spin >= a.spin) { lost = true; break; }
    __builtin_amdgcn_s_sleep(2);
  }
  int token;
  if (greedy) {
    ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q)
      if (q * kWave + lane < a.nchunk)
        best = argmax_combine(best, ArgMax{__uint_as_float(static_cast<uint32_t>(w[q])),
                                           static_cast<int>((w[q] >> 32) & 0xffffffu)});
    token = wave_argmax(best).i;
  } else {
    const double l2t = kLog2e / static_cast<double>(T);
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q)
      if (q * kWave + lane < a.nchunk) m = fmaxf(m, __uint_as_float(static_cast<uint32_t>(w[q])));
    m = wave_max(m);
    // the chunk totals of this level (each arrives with or soon after its word)
    const uint64_t* tp = reinterpret_cast<const uint64_t*>(a.totals) + static_cast<size_t>(b) * a.nchunk;
    uint64_t tw[kTreeChunkCache];
    for (uint32_t spin = 0;; ++spin) {
      bool all = true;
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q) {
        const int c = q * kWave + lane;
        tw[q] = c < a.nchunk ? load_coherent(tp + c) : 0ull;
        all &= (c >= a.nchunk || sum_at_level(tw[q], d));
      }
      if (__all(all)) break;
      if (spin >= a.spin) { lost = true; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    double wc[kTreeChunkCache];
    double Z = 0.0;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q) {
      const int c = q * kWave + lane;
      const float mc = __uint_as_float(static_cast<uint32_t>(w[q]));
      wc[q] = (c < a.nchunk && mc != -INFINITY)
                  ? sum_value(tw[q]) * exp2_neg((static_cast<double>(mc) - static_cast<double>(m)) * l2t)
                  : 0.0;
      Z += wc[q];
    }
    Z = wave_sum(Z);
    const double target = static_cast<double>(u) * Z;
    // crossing chunk (the last positive one if rounding leaves u * Z on top)
    int chunk = -1, last_chunk = -1;
    double before = 0.0, carry = 0.0;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q) {
      if (chunk < 0 && q * kWave < a.nchunk) {
        const double inc = wave_inclusive_sum(wc[q]);
        const double bef = carry + lane_move<kDppWaveShr1>(inc);
        const uint64_t pos = __ballot(wc[q] > 0.0);
        if (pos) last_chunk = q * kWave + 63 - static_cast<int>(__builtin_clzll(pos));
        const uint64_t hit = __ballot(bef + wc[q] > target && q * kWave + lane < a.nchunk);
        if (hit) {
          const int l = static_cast<int>(__builtin_ctzll(hit));
          chunk = q * kWave + l;
          before = read_lane(bef, l);
        }
        carry += read_lane(inc, kWave - 1);
      }
    }
    if (chunk < 0) {
      chunk = last_chunk < 0 ? 0 : last_chunk;
      double bs = 0.0;
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q)
        if (q * kWave + lane < chunk) bs += wc[q];
      before = wave_sum(bs);
    }
    // crossing lane of that chunk: its per-lane sums, rescaled to the row max
    const uint64_t cw = load_coherent(a.chunks + static_cast<size_t>(b) * a.nchunk + chunk);
    const float mcs = __uint_as_float(static_cast<uint32_t>(cw));
    const double scale = mcs != -INFINITY ? exp2_neg((static_cast<double>(mcs) - static_cast<double>(m)) * l2t) : 0.0;
    const uint64_t* lp = reinterpret_cast<const uint64_t*>(a.lanes) + (static_cast<size_t>(b) * a.nchunk + chunk) * kWave;
    uint64_t lw = 0;
    for (uint32_t spin = 0;; ++spin) {
      lw = load_coherent(lp + lane);
      if (__all(sum_at_level(lw, d))) break;
      if (spin >= a.spin) { lost = true; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    const double wl = sum_value(lw) * scale;
    int cl = -1;
    {
      const double inc = wave_inclusive_sum(wl);
      const double bef = before + lane_move<kDppWaveShr1>(inc);
      const uint64_t hit = __ballot(bef + wl > target);
      if (hit) {
        cl = static_cast<int>(__builtin_ctzll(hit));
        before = read_lane(bef, cl);
      } else {
        const uint64_t pos = __ballot(wl > 0.0);
        cl = pos ? 63 - static_cast<int>(__builtin_clzll(pos)) : 0;
        double bs = lane < cl ? wl : 0.0;
        before = before + wave_sum(bs);
      }
    }
    // the logits of that lane (lane i takes the i-th of them, in index order)
    const int c0 = chunk * kTreeChunk;
    const int c1 = min(a.V, c0 + kTreeChunk);
    const int k = c0 + cl * kLaneElems + lane;
    const bool have = lane < kLaneElems && k < c1;
    const void* row = fused_row<DT>(a, b, node);
    const double x = have ? static_cast<double>(Elem<DT>::at(row, k)) : 0.0;
    const double wk = have ? exp2_neg(__builtin_fma(x, l2t, -static_cast<double>(m) * l2t)) : 0.0;
    const double inc = wave_inclusive_sum(wk);
    const uint64_t hit = __ballot(wk > 0.0 && before + inc > target);
    const uint64_t pos = __ballot(wk > 0.0);
    const int li = hit ? static_cast<int>(__builtin_ctzll(hit)) : (pos ? 63 - static_cast<int>(__builtin_clzll(pos)) : 0);
    token = read_lane(k, li);
  }
  // the lowest-index child of the node that carries the token
  int child = (lane > node && lane < a.N && my_par == node && my_tok == token) ? lane : 0x7fffffff;
  for (int j = kWave + lane; j < a.N; j += kWave)
    if (j > node && par[j] == node && tk[j] == token) child = min(child, j);
  child = wave_min(child);
  const int L1 = levels_of(a);
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * L1;
  int32_t* op = a.out_path + static_cast<size_t>(b) * L1;
  if (lane == 0) ot[d] = lost ? -1 : token;
  if (!lost && child != 0x7fffffff && d + 1 < L1) {
    if (lane == 0) {
      op[d] = child;
      store_coherent(tree_ctl(a, b) + kCtlNode, node_word(d + 1, child));
    }
    return child;
  }
  // the stop: this level's path slot and every later slot are padding
  for (int i = d + lane; i < L1; i += kWave) {
    if (i > d) ot[i] = -1;
    op[i] = -1;
  }
  if (lane == 0) {
    a.out_n[b] = lost ? SV_GAVE_UP : d;
    store_coherent(tree_ctl(a, b) + kCtlStop, kTreeMark);
  }
  return -1;
}

// Stream workgroup of chunk c of request b: chunk c of each level's node row
// until the request stops (the stop follows the last level's choice, whose
// reads are then complete); then the chunk's words return to zero.
template <int DT, bool VEC>
__device__ void tree_stream_loop(const TreeFused& a, int b, int c) {
  const float T = a.temperature[b];
  for (int d = 0;; ++d) {
    const int node = tree_wait_node(a, b, d);
    if (node < 0) break;
    tree_stream_chunk<DT, VEC>(a, b, d, c, node, T);
  }
  const size_t slot = static_cast<size_t>(b) * a.nchunk + c;
  if (threadIdx.x == 0) {
    store_coherent(a.chunks + slot, 0ull);
    store_coherent_f64(a.totals + slot, 0.0);
  }
  store_coherent_f64(a.lanes + slot * kWave + threadIdx.x, 0.0);
  tree_exit(a, b);
}

// Choose workgroup of request b: validation, then the choice at each level.
template <int DT, bool VEC>
__device__ void tree_choose_loop(const TreeFused& a, int b) {
  if (tree_validate(a, b)) {
    const float T = a.temperature[b];
    int node = 0;
    for (int d = 0; node >= 0; ++d) node = tree_choose_level<DT, VEC>(a, b, d, node, T);
  }
  tree_exit(a, b);
}

// Blocks: per request b its choose workgroup, then its nchunk stream
// workgroups; each loops over the depth levels until the request stops.  A
// workgroup waits only for workgroups of its own request, whose blocks are
// contiguous.  Blocks are dispatched in order on each XCD and a request never
// waits for a later one, so the lowest unfinished request always gets all of
// its nchunk + 1 <= 257 workgroups resident: every wait ends.
template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void tree_verify(TreeFused a) {
  const uint32_t per_b = static_cast<uint32_t>(a.nchunk) + 1u;
  const uint32_t b = blockIdx.x / per_b;
  const uint32_t j = blockIdx.x - b * per_b;
  if (j == 0) tree_choose_loop<DT, VEC>(a, static_cast<int>(b));
  else tree_stream_loop<DT, VEC>(a, static_cast<int>(b), static_cast<int>(j - 1u));
}

struct TreeLayout {
  size_t state, partials, total;                       // multi-launch form
  size_t a_total;                                      // all-nodes form (partials [B][N][nchunk])
  size_t f_ctl, f_chunks, f_totals, f_lanes;  // single launch (same buffer)
  size_t f_total;
};

static int tree_fused_chunks(int V) { return (V + kTreeChunk - 1) / kTreeChunk; }

static TreeLayout tree_layout(int B, int V, int N = 1) {
  TreeLayout L{};
  L.state = 0;
  L.partials = align_up(static_cast<size_t>(B) * sizeof(TreeState));
  L.total = align_up(L.partials + static_cast<size_t>(B) * num_chunks(V) * sizeof(NodePartial));
  L.a_total = align_up(L.partials + static_cast<size_t>(B) * N * num_chunks(V) * sizeof(NodePartial));
  const size_t nc = static_cast<size_t>(tree_fused_chunks(V));
  size_t off = 0;
  L.f_ctl = off;    off = align_up(off + static_cast<size_t>(B) * kCtlStride * sizeof(uint64_t));
  L.f_chunks = off; off = align_up(off + static_cast<size_t>(B) * nc * sizeof(uint64_t));
  L.f_totals = off; off = align_up(off + static_cast<size_t>(B) * nc * sizeof(double));
  L.f_lanes = off;  off = align_up(off + static_cast<size_t>(B) * nc * kWave * sizeof(double));
  L.f_total = off;
  return L;
}

// The single launch serves shapes with at most kTreeMaxChunks chunks and a
// grid within kTreeMaxGrid blocks (and no test hook asking otherwise).
constexpr long long kTreeMaxGrid = 1 << 20;
static bool tree_fused_fits(int B, int V) {
  if (test_hook(SV_HOOK_TREE_SPLIT) != 0 || test_hook(SV_HOOK_TREE_ALL_NODES) != 0) return false;
  const long long nc = tree_fused_chunks(V);
  return nc <= kTreeMaxChunks && static_cast<long long>(B) * (nc + 1) <= kTreeMaxGrid;
}

template <int DT, bool VEC>
static int launch_tree(TreeArgs a, hipStream_t stream) {
  const long long n = static_cast<long long>(a.B) * a.nchunk;
  if (n > 0x7fffffffLL) return SV_ERR_SHAPE;
  a.last = 0;
  launch(SV_K_TREE_INIT, tree_init, dim3(a.B), dim3(kThreads), a.N * sizeof(int32_t), stream, a);
  if (test_hook(SV_HOOK_TREE_ALL_NODES) != 0) {
    const long long na = n * a.N;
    if (na > 0x7fffffffLL) return SV_ERR_SHAPE;
    launch(SV_K_TREE_NODE_PASS, tree_all_pass<DT, VEC>, dim3(static_cast<unsigned>(na)), dim3(kThreads), 0, stream, a);
    launch(SV_K_TREE_CHOOSE, tree_all_descend<DT>, dim3(a.B), dim3(kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
  }
  for (int step = 0; step <= a.max_depth; ++step) {
    launch(SV_K_TREE_NODE_PASS, tree_node_pass<DT, VEC>, dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream, a);
    a.last = step == a.max_depth;
    launch(SV_K_TREE_CHOOSE, tree_choose<DT>, dim3(a.B), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv

using namespace sv;

extern "C" size_t sv_tree_workspace_bytes(int B, int N, int V, int dtype) {
  (void)dtype;
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB) return 0;
  const TreeLayout L = tree_layout(B, V, N);
  if (test_hook(SV_HOOK_TREE_ALL_NODES) != 0) return L.a_total;
  // either form may run (it depends on max_depth, given at call time)
  return tree_fused_chunks(V) <= kTreeMaxChunks ? std::max(L.total, L.f_total) : L.total;
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
  const TreeLayout L = tree_layout(B, V, N);
  const bool fused = tree_fused_fits(B, V);
  const size_t need = fused ? L.f_total : (test_hook(SV_HOOK_TREE_ALL_NODES) != 0 ? L.a_total : L.total);
  if (workspace_bytes < need || !aligned(workspace, 256)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16);
  if (fused) {
    TreeFused f{};
    f.logits = target_logits;
    f.tokens = node_tokens;
    f.parents = parents;
    f.uniforms = uniforms;
    f.temperature = temperature;
    f.B = B;
    f.N = N;
    f.V = V;
    f.max_depth = max_depth;
    f.nchunk = tree_fused_chunks(V);
    f.out_tokens = out_tokens;
    f.out_path = out_path_nodes;
    f.out_n = out_num_accepted;
    f.ctl = reinterpret_cast<uint64_t*>(ws + L.f_ctl);
    f.chunks = reinterpret_cast<uint64_t*>(ws + L.f_chunks);
    f.totals = reinterpret_cast<double*>(ws + L.f_totals);
    f.lanes = reinterpret_cast<double*>(ws + L.f_lanes);
    f.spin = spin_limit(kTreeSpinLimit);
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(B) * (f.nchunk + 1)));
    if (dtype == SV_BF16) {
      if (vec) launch(SV_K_TREE_VERIFY, tree_verify<0, true>, grid, dim3(kWave), 0, stream, f);
      else launch(SV_K_TREE_VERIFY, tree_verify<0, false>, grid, dim3(kWave), 0, stream, f);
    } else {
      if (vec) launch(SV_K_TREE_VERIFY, tree_verify<1, true>, grid, dim3(kWave), 0, stream, f);
      else launch(SV_K_TREE_VERIFY, tree_verify<1, false>, grid, dim3(kWave), 0, stream, f);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
  }
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
  if (dtype == SV_BF16) return vec ? launch_tree<0, true>(a, stream) : launch_tree<0, false>(a, stream);
  return vec ? launch_tree<1, true>(a, stream) : launch_tree<1, false>(a, stream);
}
