// Tree attention mask and depth positions for tree-parallel decoding
// (CMU 15-779 lecture 17 notes, section 4.3: a depth-first linearised token
// tree is verified in one forward pass under a topology-aware causal mask, a
// node seeing only itself and its ancestors, with position ids given by
// depth; exercise 5 works one tree through).
//
// One workgroup per request, one thread per node (N <= 1024).  The parent
// array sits in LDS; each thread walks from its node up to the root -- at most
// max_depth + 1 steps, since deeper trees are rejected on the way -- and sets
// one bit per node it passes in a row of W 64-bit words held in registers.
// The walk needs no ordering between threads, so the only synchronisation is
// the two validity votes; each thread stores its own row.  At token-tree
// sizes the kernel is bound by launch latency and the walk's dependent LDS
// reads; the row stores are its only sizeable traffic.
#include <hip/hip_runtime.h>

#include "sv_host.hpp"

namespace sv {
namespace {

constexpr int kMaskThreads = SV_MAX_TREE_NODES;

struct MaskArgs {
  const int32_t* parents;
  int N, max_depth, words;
  uint64_t* out_mask;
  int32_t* out_depth;
  int32_t* out_tree_depth;
};

// Row word w of node i's row gets bit (a & 63) when node a lies in word w.
template <int W>
__device__ inline void set_bit(uint64_t (&row)[W], int a) {
  const uint64_t bit = 1ull << (a & 63);
  const int w = a >> 6;
#pragma unroll
  for (int k = 0; k < W; ++k) row[k] |= (k == w) ? bit : 0ull;
}

template <int W>
__global__ __launch_bounds__(kMaskThreads) void tree_mask(MaskArgs a) {
  __shared__ int s_par[SV_MAX_TREE_NODES];
  __shared__ int s_bad, s_deep, s_maxd;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const bool mine = i < a.N;
  const int32_t* par = a.parents + static_cast<size_t>(b) * a.N;
  if (i == 0) {
    s_bad = 0;
    s_deep = 0;
    s_maxd = 0;
  }
  int p = -1;
  if (mine) {
    p = par[i];
    s_par[i] = p;
  }
  __syncthreads();
  // the root has no parent; every other node's parent comes before it
  if (mine && (i == 0 ? p != -1 : (p < 0 || p >= i))) s_bad = 1;
  __syncthreads();
  const bool bad = s_bad != 0;
  uint64_t row[W];
#pragma unroll
  for (int k = 0; k < W; ++k) row[k] = 0ull;
  int depth = -1;
  if (mine && !bad) {
    // the walk ends at the root (parents strictly decrease) or one node past
    // max_depth, whichever comes first
    int n = i;
    while (n >= 0) {
      if (++depth > a.max_depth) break;
      set_bit<W>(row, n);
      n = s_par[n];
    }
    if (n >= 0) s_deep = 1;
    else atomicMax(&s_maxd, depth);
  }
  __syncthreads();
  const bool valid = !bad && s_deep == 0;
  if (!mine) return;
  uint64_t* dst = a.out_mask + (static_cast<size_t>(b) * a.N + i) * a.words;
#pragma unroll
  for (int k = 0; k < W; ++k)
    if (k < a.words) dst[k] = valid ? row[k] : 0ull;
  a.out_depth[static_cast<size_t>(b) * a.N + i] = valid ? depth : -1;
  if (i == 0 && a.out_tree_depth) a.out_tree_depth[b] = valid ? s_maxd : -1;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" int spec_tree_mask(const int32_t* parents, int B, int N, int max_depth,
                              uint64_t* out_mask, int32_t* out_depth, int32_t* out_tree_depth,
                              void* hip_stream) {
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || max_depth < 0 || max_depth > SV_MAX_TREE_DEPTH)
    return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!parents || !out_mask || !out_depth) return SV_ERR_NULL;
  if (!aligned(out_mask, sizeof(uint64_t))) return SV_ERR_ALIGN;
  MaskArgs a{};
  a.parents = parents;
  a.N = N;
  a.max_depth = max_depth;
  a.words = (N + 63) / 64;
  a.out_mask = out_mask;
  a.out_depth = out_depth;
  a.out_tree_depth = out_tree_depth;
  const dim3 grid(static_cast<unsigned>(B));
  const dim3 block(static_cast<unsigned>((N + 63) / 64 * 64));
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (a.words <= 1) launch(SV_K_TREE_MASK, tree_mask<1>, grid, block, 0, stream, a);
  else if (a.words <= 2) launch(SV_K_TREE_MASK, tree_mask<2>, grid, block, 0, stream, a);
  else if (a.words <= 4) launch(SV_K_TREE_MASK, tree_mask<4>, grid, block, 0, stream, a);
  else if (a.words <= 8) launch(SV_K_TREE_MASK, tree_mask<8>, grid, block, 0, stream, a);
  else launch(SV_K_TREE_MASK, tree_mask<16>, grid, block, 0, stream, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
