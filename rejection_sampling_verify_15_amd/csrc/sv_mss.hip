// Token-tree verification by multi-step speculative sampling (CMU 15-779
// lecture 17 notes, section 4.5: VerifyStochastic, the children of a node
// drawn without replacement from its draft distribution; section 4.4
// VerifyGreedy for T == 0).  See include/specverify.h for the contract.
//
// At node n let P = softmax(target_n / T) and Q = softmax(draft_n / T).  The
// children x_1, x_2, ... are tested in index order; child j against the
// residual r_j and against q_j, which is Q without the tokens tested before,
// renormalised by S_j = 1 - sum_{i<j} Q(x_i).  After j rejections the
// residual (unnormalised) is max(0, P - A_j Q) on every token not yet tested
// and stays at F_i = max(0, P(x_i) - A_i Q(x_i)) on each tested x_i, where
// A_j = A_{j-1} + N_j / S_j and N_j is the residual's total.  One scalar so
// carries the whole residual: a rejection costs one pass over the vocabulary
// (the sum of max(0, P - A Q)), and a test needs only the two logits of the
// child's token.
//
// One launch of one-wave workgroups, laid out as the naive-sampling tree
// kernel: per request a choose workgroup and one stream workgroup per
// 2048-logit chunk.  The choose workgroup publishes passes (a sequence number,
// the kind and the node; for a residual pass the scalars M_t, M_d, Z_t, Z_d, A
// first); every stream workgroup answers each pass for its chunk and keeps
// the chunk of both rows in registers across the passes of one node:
//   stats pass     target chunk max and argmax, fp64 lane sums of
//                  exp((x - m) / T) and their total; with the draft, its chunk
//                  max and sum (sampling nodes that have children)
//   residual pass  fp64 lane sums of max(0, P - A Q) and their total, P from
//                  the stats pass's exponentials kept in registers
// Every pass rewrites every result slot under its own tag (sequence number
// mod 127), so a slot holds this pass's value or the previous pass's, whose
// tags differ.  The choose workgroup then decides: argmax descent; or the
// children's tests in order, each rejection followed by a residual pass; the
// final draw from the residual (or from P) narrowed chunk -> lane -> logit in
// fp64.
#include <hip/hip_runtime.h>

#include "sv_device.hpp"
#include "sv_host.hpp"
#include "sv_tree_common.hpp"

namespace sv {
namespace {

// control words of a request
constexpr int kMssPass = 0, kMssStop = 1, kMssExit = 2;
constexpr int kPrmMt = 3, kPrmMd = 4, kPrmZt = 5, kPrmZd = 6, kPrmA = 7;
// pass kinds
constexpr int kPassStats = 0, kPassStatsDraft = 1, kPassResidual = 2;
// result slot words of a chunk
constexpr int kSlotWords = 8;
constexpr int kSlotT = 0, kSlotD = 1, kSlotTotP = 2, kSlotTotD = 3, kSlotTotR = 4;
// children of one node (a node's tested children are held one per lane of
// the choose workgroup)
constexpr int kMssMaxChildren = kWave;
// logits per stream workgroup (32 per lane; halving it doubles the
// workgroups, and fewer requests then fit at once)
constexpr int kMssChunk = kTreeChunk;

struct MssArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* parents;
  const float* acc_u;
  const float* draw_u;
  const float* temperature;
  int B, N, V, max_depth, nchunk;
  int32_t* out_tokens;
  int32_t* out_path;
  int32_t* out_n;
  uint64_t* ctl;    // [B][kCtlStride]
  uint64_t* slots;  // [B][nchunk][kSlotWords]
  uint64_t* lanes;  // [B][nchunk][2][kWave]: lane sums of P (stats), of the residual
  uint32_t spin;    // poll bound of every wait (kTreeSpinLimit unless a test lowers it)
};

__device__ inline uint64_t* mss_ctl(const MssArgs& a, int b) { return a.ctl + static_cast<size_t>(b) * kCtlStride; }
__device__ inline uint64_t* mss_slot(const MssArgs& a, int b, int c) {
  return a.slots + (static_cast<size_t>(b) * a.nchunk + c) * kSlotWords;
}
__device__ inline uint64_t* mss_lanes(const MssArgs& a, int b, int c, int which) {
  return a.lanes + ((static_cast<size_t>(b) * a.nchunk + c) * 2 + which) * kWave;
}
template <int DT>
__device__ inline const void* mss_row(const void* base, const MssArgs& a, int b, int node) {
  return static_cast<const char*>(base) +
         (static_cast<size_t>(b) * a.N + node) * static_cast<size_t>(a.V) * Elem<DT>::kBytes;
}

__device__ inline int pass_tag(uint32_t s) { return static_cast<int>(s % 127u); }
__device__ inline uint64_t pass_word(uint32_t s, int kind, int node) {
  return kTreeMark | (static_cast<uint64_t>(s) << 34) | (static_cast<uint64_t>(kind) << 32) |
         static_cast<uint32_t>(node);
}

// Scalars of a residual pass.  P(x) = e_t(x) * rzt and Q(x) = e_d(x) * rzd with
// e = 2^((x - M) * log2(e) / T); the residual weight of an untested token is
// max(0, P - A Q).  Both sides evaluate it through mss_weight.
struct MssParams {
  double l2t, mtl, mdl, rzt, rzd, A;
};
__device__ inline double mss_p(double t, const MssParams& q) { return exp2_neg(__builtin_fma(t, q.l2t, -q.mtl)) * q.rzt; }
__device__ inline double mss_q(double d, const MssParams& q) { return exp2_neg(__builtin_fma(d, q.l2t, -q.mdl)) * q.rzd; }
__device__ inline double mss_weight(double P, double Q, double A) { return fmax(0.0, __builtin_fma(-A, Q, P)); }
__device__ inline MssParams mss_params(float T, float Mt, float Md, double Zt, double Zd, double A) {
  MssParams q;
  q.l2t = kLog2e / static_cast<double>(T);
  q.mtl = static_cast<double>(Mt) * q.l2t;
  q.mdl = static_cast<double>(Md) * q.l2t;
  q.rzt = 1.0 / Zt;
  q.rzd = 1.0 / Zd;
  q.A = A;
  return q;
}

// The scalars of a residual pass travel tagged with the pass (the maxima as
// chunk-style words, Z_t, Z_d and A as tagged doubles), so the pass word needs
// no wait for their stores.  A tagged double loses its low 7 mantissa bits;
// the choose workgroup uses the same truncated values (trunc7) throughout.
struct MssScalars {
  float Mt, Md;
  double Zt, Zd, A;
};
__device__ inline double trunc7(double v) { return sum_value(tag_sum(v, 0)); }

__device__ bool mss_wait_scalars(const MssArgs& a, int b, uint32_t s, MssScalars& sc) {
  const uint64_t* cw = mss_ctl(a, b);
  const int tag = pass_tag(s);
  for (uint32_t spin = 0; spin < a.spin; ++spin) {
    const uint64_t wmt = load_coherent(cw + kPrmMt);
    const uint64_t wmd = load_coherent(cw + kPrmMd);
    const uint64_t wzt = load_coherent(cw + kPrmZt);
    const uint64_t wzd = load_coherent(cw + kPrmZd);
    const uint64_t wa = load_coherent(cw + kPrmA);
    if (chunk_at_level(wmt, tag) && chunk_at_level(wmd, tag) && sum_at_level(wzt, tag) &&
        sum_at_level(wzd, tag) && sum_at_level(wa, tag)) {
      sc.Mt = __uint_as_float(static_cast<uint32_t>(wmt));
      sc.Md = __uint_as_float(static_cast<uint32_t>(wmd));
      sc.Zt = sum_value(wzt);
      sc.Zd = sum_value(wzd);
      sc.A = sum_value(wa);
      return true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Waits for pass s of request b: its pass word, or 0 once the request has
// stopped (or the wait gave up).
__device__ uint64_t mss_wait_pass(const MssArgs& a, int b, uint32_t s) {
  const uint64_t* cw = mss_ctl(a, b);
  for (uint32_t spin = 0; spin < a.spin; ++spin) {
    const uint64_t pv = load_coherent(cw + kMssPass);
    if ((pv & kTreeMark) && ((pv >> 34) & 0x1fffffffull) == s) return pv;
    if (load_coherent(cw + kMssStop) & kTreeMark) return 0;
    __builtin_amdgcn_s_sleep(2);
  }
  return 0;
}

// A workgroup of request b is done; the last of its nchunk + 1 workgroups
// returns the control words to zero.
__device__ inline void mss_exit(const MssArgs& a, int b) {
  if (threadIdx.x != 0) return;
  uint64_t* cw = mss_ctl(a, b);
  if (arrive(reinterpret_cast<uint32_t*>(cw + kMssExit)) == static_cast<uint32_t>(a.nchunk)) {
    for (int i = 0; i < kCtlStride; ++i) store_coherent(cw + i, 0ull);
  }
}

// ---------------------------------------------------------------------------
// stream workgroups
// ---------------------------------------------------------------------------
template <int DT, bool VEC>
__device__ void mss_stream_loop(const MssArgs& a, int b, int c) {
  using Raw = LaneRun<DT, VEC, kMssChunk>;
  const float T = a.temperature[b];
  const bool greedy = T == 0.0f;
  const double l2t = greedy ? 0.0 : kLog2e / static_cast<double>(T);
  const int c0 = c * kMssChunk;
  const int c1 = min(a.V, c0 + kMssChunk);
  const int lane = threadIdx.x;
  uint64_t* slot = mss_slot(a, b, c);
  uint64_t* lp_out = mss_lanes(a, b, c, 0);
  uint64_t* lr_out = mss_lanes(a, b, c, 1);
  // The node's chunk of both rows and its stats, stored again under every
  // later pass's tag.  The target's fp64 exponentials (relative to the chunk
  // max) are kept rounded to fp32, so a residual pass computes only the
  // draft's; the rounding (relative 6e-8 per logit, unbiased) reaches the
  // residual's sums alone -- the tests' normalisers and the chunk and lane
  // narrowing of a draw, whose logit scan recomputes fp64 weights.
  float mt = -INFINITY, md = -INFINITY;
  int arg = 0;
  double lp = 0.0, tot_p = 0.0, tot_d = 0.0;
  Raw rt, rd;
  float et[Raw::kItems * Raw::kPer];
  for (uint32_t s = 0;; ++s) {
    const uint64_t pw = mss_wait_pass(a, b, s);
    if (pw == 0) break;
    const int kind = static_cast<int>((pw >> 32) & 3u);
    const int node = static_cast<int>(static_cast<uint32_t>(pw));
    const int tag = pass_tag(s);
    double lr = 0.0, tot_r = 0.0;
    if (kind != kPassResidual) {
      rt.load(mss_row<DT>(a.target, a, b, node), c0, c1);
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
        for (int e = 0; e < Raw::kPer; ++e) m = fmaxf(m, rt.at(j, e));
      mt = wave_max(m);
      arg = 0;
      lp = tot_p = tot_d = 0.0;
      md = -INFINITY;
      if (greedy) {
        int idx = 0x7fffffff;
#pragma unroll
        for (int j = Raw::kItems - 1; j >= 0; --j)
#pragma unroll
          for (int e = Raw::kPer - 1; e >= 0; --e) {
            const int k = Raw::index(c0, j, e);
            if (k < c1 && rt.at(j, e) == mt) idx = k;
          }
        arg = wave_min(idx);
      } else if (mt == -INFINITY) {
#pragma unroll
        for (int i = 0; i < Raw::kItems * Raw::kPer; ++i) et[i] = 0.0f;
      } else {
        const double ml = static_cast<double>(mt) * l2t;
#pragma unroll
        for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
          for (int e = 0; e < Raw::kPer; ++e)
          {
            const double x = exp2_neg(__builtin_fma(static_cast<double>(rt.at(j, e)), l2t, -ml));
            et[j * Raw::kPer + e] = static_cast<float>(x);
            lp += x;
          }
        tot_p = wave_sum(lp);
      }
      if (kind == kPassStatsDraft) {
        rd.load(mss_row<DT>(a.draft, a, b, node), c0, c1);
        float m2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
          for (int e = 0; e < Raw::kPer; ++e) m2 = fmaxf(m2, rd.at(j, e));
        md = wave_max(m2);
        if (md != -INFINITY) {
          const double ml = static_cast<double>(md) * l2t;
          double sd = 0.0;
#pragma unroll
          for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
            for (int e = 0; e < Raw::kPer; ++e)
              sd += exp2_neg(__builtin_fma(static_cast<double>(rd.at(j, e)), l2t, -ml));
          tot_d = wave_sum(sd);
        }
      }
    } else {
      // residual pass: the scalars carry this pass's tag
      MssScalars sc;
      if (!mss_wait_scalars(a, b, s, sc)) break;
      const MssParams q = mss_params(T, sc.Mt, sc.Md, sc.Zt, sc.Zd, sc.A);
      // P from the stats pass's exponentials, rescaled to the row
      const double fp = mt != -INFINITY
                            ? exp2_neg((static_cast<double>(mt) - static_cast<double>(sc.Mt)) * l2t) / sc.Zt : 0.0;
#pragma unroll
      for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
        for (int e = 0; e < Raw::kPer; ++e)
          lr += mss_weight(static_cast<double>(et[j * Raw::kPer + e]) * fp,
                           mss_q(static_cast<double>(rd.at(j, e)), q), sc.A);
      tot_r = wave_sum(lr);
    }
    store_coherent(lp_out + lane, tag_sum(lp, tag));
    store_coherent(lr_out + lane, tag_sum(lr, tag));
    if (lane == 0) {
      store_coherent(slot + kSlotTotP, tag_sum(tot_p, tag));
      store_coherent(slot + kSlotTotD, tag_sum(tot_d, tag));
      store_coherent(slot + kSlotTotR, tag_sum(tot_r, tag));
      store_coherent(slot + kSlotD, tree_chunk_word(tag, md, 0));
      store_coherent(slot + kSlotT, tree_chunk_word(tag, mt, arg));
    }
  }
  store_coherent(lp_out + lane, 0ull);
  store_coherent(lr_out + lane, 0ull);
  if (lane < kSlotWords) store_coherent(slot + lane, 0ull);
  mss_exit(a, b);
}

// ---------------------------------------------------------------------------
// choose workgroup
// ---------------------------------------------------------------------------
// Polls word `which` of every chunk slot (lane l holds chunks l, l + kWave, ...)
// until all carry pass s's tag; `sum` selects the tagged-double format.
__device__ inline bool mss_poll_slots(const MssArgs& a, int b, int which, uint32_t s, bool sum,
                                      uint64_t (&w)[kTreeChunkCache]) {
  const int tag = pass_tag(s);
  for (uint32_t spin = 0;; ++spin) {
    bool all = true;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q) {
      const int c = q * kWave + static_cast<int>(threadIdx.x);
      w[q] = c < a.nchunk ? load_coherent(mss_slot(a, b, c) + which) : 0ull;
      all = all && (c >= a.nchunk || (sum ? sum_at_level(w[q], tag) : chunk_at_level(w[q], tag)));
    }
    if (__all(all)) return true;
    if (spin >= a.spin) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Polls the kWave lane sums `which` of chunk c until they carry pass s's tag.
__device__ inline bool mss_poll_lanes(const MssArgs& a, int b, int c, int which, uint32_t s, uint64_t& w) {
  const uint64_t* lp = mss_lanes(a, b, c, which);
  const int tag = pass_tag(s);
  for (uint32_t spin = 0;; ++spin) {
    w = load_coherent(lp + threadIdx.x);
    if (__all(sum_at_level(w, tag))) return true;
    if (spin >= a.spin) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// The crossing among kTreeChunkCache * kWave weights held lane-strided (lane l
// holds entries l, l + kWave, ...; n of them): the entry in which the running
// sum first exceeds `target`, or the last positive one if rounding leaves the
// target on top.  Returns the entry and the sum before it.
__device__ inline int mss_cross_chunks(const double (&wc)[kTreeChunkCache], int n, double target, double& before) {
  const int lane = threadIdx.x;
  int hit_at = -1, last = -1;
  double carry = 0.0;
  before = 0.0;
#pragma unroll
  for (int q = 0; q < kTreeChunkCache; ++q) {
    if (hit_at < 0 && q * kWave < n) {
      const double inc = wave_inclusive_sum(wc[q]);
      const double bef = carry + lane_move<kDppWaveShr1>(inc);
      const uint64_t pos = __ballot(wc[q] > 0.0);
      if (pos) last = q * kWave + 63 - static_cast<int>(__builtin_clzll(pos));
      const uint64_t hit = __ballot(bef + wc[q] > target && q * kWave + lane < n);
      if (hit) {
        const int l = static_cast<int>(__builtin_ctzll(hit));
        hit_at = q * kWave + l;
        before = read_lane(bef, l);
      }
      carry += read_lane(inc, kWave - 1);
    }
  }
  if (hit_at < 0) {
    hit_at = last < 0 ? 0 : last;
    double bs = 0.0;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q)
      if (q * kWave + lane < hit_at) bs += wc[q];
    before = wave_sum(bs);
  }
  return hit_at;
}

// The crossing lane of one chunk from its per-lane weights wl (this lane's).
__device__ inline int mss_cross_lane(double wl, double target, double& before) {
  const int lane = threadIdx.x;
  const double inc = wave_inclusive_sum(wl);
  const double bef = before + lane_move<kDppWaveShr1>(inc);
  const uint64_t hit = __ballot(bef + wl > target);
  if (hit) {
    const int cl = static_cast<int>(__builtin_ctzll(hit));
    before = read_lane(bef, cl);
    return cl;
  }
  const uint64_t pos = __ballot(wl > 0.0);
  const int cl = pos ? 63 - static_cast<int>(__builtin_clzll(pos)) : 0;
  before += wave_sum(lane < cl ? wl : 0.0);
  return cl;
}

// The crossing logit among the kRun logits of one lane's run (lane i holds the
// i-th of them, weight wk, index k).
__device__ inline int mss_cross_logit(double wk, int k, double before, double target) {
  const double inc = wave_inclusive_sum(wk);
  const uint64_t hit = __ballot(wk > 0.0 && before + inc > target);
  const uint64_t pos = __ballot(wk > 0.0);
  const int li = hit ? static_cast<int>(__builtin_ctzll(hit)) : (pos ? 63 - static_cast<int>(__builtin_clzll(pos)) : 0);
  return read_lane(k, li);
}

// Tested children of the current node, one per lane (lane r: the r-th tested):
// token, P and Q of the token, and its residual F, frozen once tested.
struct Tested {
  int tok;
  double P, Q, F;
  int count;
};

// The request's tree in LDS, filled by the choose workgroup's validation and
// read at every level: parents, node tokens and children counts.
struct MssTree {
  int32_t par[SV_MAX_TREE_NODES];
  int32_t tok[SV_MAX_TREE_NODES];
  int32_t kids[SV_MAX_TREE_NODES];
};

// Validation by the choose workgroup (as the naive-sampling tree kernel, plus
// both uniform arrays for sampling requests and the children limit).  An
// invalid request gets its -1 outputs and the stop.
__device__ bool mss_validate(const MssArgs& a, int b, MssTree& t) {
  const int lane = threadIdx.x;
  const int L1 = a.max_depth + 1;
  const int32_t* par = a.parents + static_cast<size_t>(b) * a.N;
  const int32_t* tok = a.tokens + static_cast<size_t>(b) * a.N;
  for (int i = lane; i < a.N; i += kWave) {
    t.par[i] = par[i];
    t.tok[i] = tok[i];
    t.kids[i] = 0;
  }
  __syncthreads();
  for (int i = lane + 1; i < a.N; i += kWave) {
    const int p = t.par[i];
    if (p >= 0 && p < i) atomicAdd(&t.kids[p], 1);
  }
  __syncthreads();
  const float T = a.temperature[b];
  int bad = !tree_temp_ok(T);
  const bool sampling = !bad && T > 0.0f;
  for (int i = lane; i < a.N; i += kWave) {
    bad |= (t.kids[i] > kMssMaxChildren);
    if (i == 0) {
      bad |= (t.par[0] != -1);
    } else {
      const int p = t.par[i];
      bad |= (p < 0 || p >= i);
      bad |= (t.tok[i] < 0 || t.tok[i] >= a.V);
      if (p >= 0 && p < i) {
        int n = i, depth = 0;
        while (n > 0 && depth <= a.max_depth) {
          const int q = t.par[n];
          if (q < 0 || q >= n) { depth = a.max_depth + 1; break; }
          n = q;
          ++depth;
        }
        bad |= (depth > a.max_depth);
      }
    }
    if (sampling) {
      const float ud = a.draw_u[static_cast<size_t>(b) * a.N + i];
      bad |= !(ud >= 0.0f && ud < 1.0f);
      if (i > 0) {
        const float ua = a.acc_u[static_cast<size_t>(b) * a.N + i];
        bad |= !(ua >= 0.0f && ua < 1.0f);
      }
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
      store_coherent(mss_ctl(a, b) + kMssStop, kTreeMark);
    }
  }
  return !any_bad;
}

// The children of `node` in index order, one per lane (at most kWave after
// validation): lane i gets the i-th child's id and token; returns the count.
__device__ inline int mss_children(const MssArgs& a, const MssTree& t, int node, int& id, int& tk) {
  const int lane = threadIdx.x;
  int count = 0;
  id = -1;
  tk = -1;
  for (int base = node + 1; base < a.N && count < t.kids[node]; base += kWave) {
    const int j = base + lane;
    const bool kid = j < a.N && t.par[j] == node;
    const uint64_t m = __ballot(kid);
    const int slot = count + __popcll(m & ((1ull << lane) - 1ull));
    // lane `slot` takes child j: route through LDS-free lane moves
    for (uint64_t r = m; r; r &= r - 1) {
      const int l = static_cast<int>(__builtin_ctzll(r));
      const int at = read_lane(slot, l);
      const int jj = base + l;
      if (lane == at) {
        id = jj;
        tk = t.tok[jj];
      }
    }
    count += __popcll(m);
  }
  return count;
}

// Publishes pass s; a residual pass carries its scalars, tagged with s.
__device__ inline void mss_publish(const MssArgs& a, int b, uint32_t s, int kind, int node, float Mt = 0.0f,
                                   float Md = 0.0f, double Zt = 0.0, double Zd = 0.0, double A = 0.0) {
  if (threadIdx.x != 0) return;
  uint64_t* cw = mss_ctl(a, b);
  if (kind == kPassResidual) {
    const int tag = pass_tag(s);
    store_coherent(cw + kPrmMt, tree_chunk_word(tag, Mt, 0));
    store_coherent(cw + kPrmMd, tree_chunk_word(tag, Md, 0));
    store_coherent(cw + kPrmZt, tag_sum(Zt, tag));
    store_coherent(cw + kPrmZd, tag_sum(Zd, tag));
    store_coherent(cw + kPrmA, tag_sum(A, tag));
  }
  store_coherent(cw + kMssPass, pass_word(s, kind, node));
}

// Outputs of a request that stops at level d with `token` (or is lost).
__device__ inline void mss_stop(const MssArgs& a, int b, int d, int token, bool lost) {
  const int L1 = a.max_depth + 1;
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * L1;
  int32_t* op = a.out_path + static_cast<size_t>(b) * L1;
  for (int i = threadIdx.x; i < L1; i += kWave) {
    if (lost) {
      ot[i] = -1;
      op[i] = -1;
    } else {
      if (i == d) ot[i] = token;
      else if (i > d) ot[i] = -1;
      if (i >= d) op[i] = -1;
    }
  }
  if (threadIdx.x == 0) {
    a.out_n[b] = lost ? SV_GAVE_UP : d;
    store_coherent(mss_ctl(a, b) + kMssStop, kTreeMark);
  }
}

// The choose workgroup of request b: validation, then each level's decision.
template <int DT, bool VEC>
__device__ void mss_choose_loop(const MssArgs& a, int b, MssTree& tree) {
  constexpr int kRun = LaneRun<DT, VEC, kMssChunk>::kRun;
  if (!mss_validate(a, b, tree)) return;
  const int lane = threadIdx.x;
  const float T = a.temperature[b];
  const bool greedy = T == 0.0f;
  const double l2t = greedy ? 0.0 : kLog2e / static_cast<double>(T);
  const int L1 = a.max_depth + 1;
  int32_t* ot = a.out_tokens + static_cast<size_t>(b) * L1;
  int32_t* op = a.out_path + static_cast<size_t>(b) * L1;
  uint32_t s = 0;
  int node = 0;
  mss_publish(a, b, s, (!greedy && tree.kids[0] > 0) ? kPassStatsDraft : kPassStats, node);
  for (int d = 0;; ++d) {
    // the node's children, one per lane, and (sampling) their two logits and
    // accept uniforms, loaded while the stats pass runs
    int kid = -1, ktok = -1;
    const int nk = mss_children(a, tree, node, kid, ktok);
    float tv = 0.0f, dv = 0.0f, uv = 0.0f;
    if (!greedy && lane < nk) {
      tv = Elem<DT>::at(mss_row<DT>(a.target, a, b, node), ktok);
      dv = Elem<DT>::at(mss_row<DT>(a.draft, a, b, node), ktok);
      uv = a.acc_u[static_cast<size_t>(b) * a.N + kid];
    }
    uint64_t wt[kTreeChunkCache];
    if (!mss_poll_slots(a, b, kSlotT, s, false, wt)) { mss_stop(a, b, d, -1, true); return; }
    if (greedy) {
      ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q)
        if (q * kWave + lane < a.nchunk)
          best = argmax_combine(best, ArgMax{__uint_as_float(static_cast<uint32_t>(wt[q])),
                                             static_cast<int>((wt[q] >> 32) & 0xffffffu)});
      const int token = wave_argmax(best).i;
      const uint64_t hit = __ballot(lane < nk && ktok == token);
      if (!hit || d + 1 >= L1) { mss_stop(a, b, d, token, false); return; }
      const int child = read_lane(kid, static_cast<int>(__builtin_ctzll(hit)));
      if (lane == 0) { ot[d] = token; op[d] = child; }
      node = child;
      ++s;
      mss_publish(a, b, s, kPassStats, node);
      continue;
    }
    uint64_t wp[kTreeChunkCache];
    if (!mss_poll_slots(a, b, kSlotTotP, s, true, wp)) { mss_stop(a, b, d, -1, true); return; }
    // P's normaliser: the chunk sums rescaled to the row max
    float Mt = -INFINITY;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q)
      if (q * kWave + lane < a.nchunk) Mt = fmaxf(Mt, __uint_as_float(static_cast<uint32_t>(wt[q])));
    Mt = wave_max(Mt);
    double pc[kTreeChunkCache];  // P's chunk weights relative to the row max
    double Zt = 0.0;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q) {
      const float mc = __uint_as_float(static_cast<uint32_t>(wt[q]));
      pc[q] = (q * kWave + lane < a.nchunk && mc != -INFINITY)
                  ? sum_value(wp[q]) * exp2_neg((static_cast<double>(mc) - static_cast<double>(Mt)) * l2t)
                  : 0.0;
      Zt += pc[q];
    }
    Zt = trunc7(wave_sum(Zt));
    int token = -1, child = -1;
    bool lost = false;
    // the final draw takes its weights from P (the stats pass) or from the
    // residual of the last residual pass
    bool from_residual = false;
    double A = 0.0;
    Tested tx{-1, 0.0, 0.0, 0.0, 0};
    float Md = -INFINITY;
    double Zd = 1.0;
    if (nk > 0) {
      uint64_t wd[kTreeChunkCache], wdt[kTreeChunkCache];
      if (!mss_poll_slots(a, b, kSlotD, s, false, wd) || !mss_poll_slots(a, b, kSlotTotD, s, true, wdt)) {
        mss_stop(a, b, d, -1, true);
        return;
      }
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q)
        if (q * kWave + lane < a.nchunk) Md = fmaxf(Md, __uint_as_float(static_cast<uint32_t>(wd[q])));
      Md = wave_max(Md);
      Zd = 0.0;
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q) {
        const float mc = __uint_as_float(static_cast<uint32_t>(wd[q]));
        Zd += (q * kWave + lane < a.nchunk && mc != -INFINITY)
                  ? sum_value(wdt[q]) * exp2_neg((static_cast<double>(mc) - static_cast<double>(Md)) * l2t)
                  : 0.0;
      }
      Zd = trunc7(wave_sum(Zd));
      const MssParams prm0 = mss_params(T, Mt, Md, Zt, Zd, 0.0);
      // lane i: P and Q at the i-th child's token
      const double Pk = lane < nk ? mss_p(static_cast<double>(tv), prm0) : 0.0;
      const double Qk = lane < nk ? mss_q(static_cast<double>(dv), prm0) : 0.0;
      double Nn = 1.0, S = 1.0;
      for (int i = 0; i < nk; ++i) {
        const int t = read_lane(ktok, i);
        // a token tested already at this node is skipped
        if (__any(lane < tx.count && tx.tok == t)) continue;
        const double P = read_lane(Pk, i);
        const double Q = read_lane(Qk, i);
        const double r = mss_weight(P, Q, A) / Nn;
        const double qj = Q / S;
        const double tau = qj <= r ? 1.0 : r / qj;
        if (static_cast<double>(read_lane(uv, i)) <= tau) {
          child = read_lane(kid, i);
          token = t;
          break;
        }
        // rejected: the residual moves to A + N / S, the token is frozen
        const double A2 = trunc7(A + Nn / S);
        if (lane == tx.count) {
          tx.tok = t;
          tx.P = P;
          tx.Q = Q;
          tx.F = mss_weight(P, Q, A2);
        }
        ++tx.count;
        A = A2;
        S -= Q;
        ++s;
        mss_publish(a, b, s, kPassResidual, node, Mt, Md, Zt, Zd, A);
        uint64_t wr[kTreeChunkCache];
        if (!mss_poll_slots(a, b, kSlotTotR, s, true, wr)) { lost = true; break; }
        double G = 0.0;
#pragma unroll
        for (int q = 0; q < kTreeChunkCache; ++q)
          if (q * kWave + lane < a.nchunk) G += sum_value(wr[q]);
        const double fix = lane < tx.count ? tx.F - mss_weight(tx.P, tx.Q, A) : 0.0;
        Nn = wave_sum(G + fix);
        if (!(Nn > 0.0)) { from_residual = false; break; }  // empty residual: draw from P
        from_residual = true;
        if (!(S > 0.0)) break;  // no draft mass left: no later child can have been drawn
      }
    }
    if (lost) { mss_stop(a, b, d, -1, true); return; }
    if (child >= 0) {
      if (d + 1 >= L1) { mss_stop(a, b, d, token, false); return; }  // unreachable after validation
      if (lane == 0) { ot[d] = token; op[d] = child; }
      node = child;
      ++s;
      mss_publish(a, b, s, tree.kids[node] > 0 ? kPassStatsDraft : kPassStats, node);
      continue;
    }
    // the final draw: chunk -> lane -> logit
    const float ud = a.draw_u[static_cast<size_t>(b) * a.N + node];
    const void* trow = mss_row<DT>(a.target, a, b, node);
    double wc[kTreeChunkCache];
    const MssParams prm = mss_params(T, Mt, Md, Zt, Zd, A);
    if (from_residual) {
      uint64_t wr[kTreeChunkCache];
      if (!mss_poll_slots(a, b, kSlotTotR, s, true, wr)) { mss_stop(a, b, d, -1, true); return; }
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q) wc[q] = q * kWave + lane < a.nchunk ? sum_value(wr[q]) : 0.0;
      // the tested tokens hold their frozen residual, not max(0, P - A Q)
      for (int r = 0; r < tx.count; ++r) {
        const int xt = read_lane(tx.tok, r);
        const double delta = read_lane(lane == r ? tx.F - mss_weight(tx.P, tx.Q, A) : 0.0, r);
        const int cc = xt / kMssChunk;
#pragma unroll
        for (int q = 0; q < kTreeChunkCache; ++q)
          if (q * kWave + lane == cc) wc[q] += delta;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kTreeChunkCache; ++q) wc[q] = pc[q];
    }
    double W = 0.0;
#pragma unroll
    for (int q = 0; q < kTreeChunkCache; ++q) W += wc[q];
    W = wave_sum(W);
    const double target = static_cast<double>(ud) * W;
    double before = 0.0;
    const int chunk = mss_cross_chunks(wc, a.nchunk, target, before);
    const int c0 = chunk * kMssChunk;
    const int c1 = min(a.V, c0 + kMssChunk);
    uint64_t lw = 0;
    if (!mss_poll_lanes(a, b, chunk, from_residual ? 1 : 0, s, lw)) { mss_stop(a, b, d, -1, true); return; }
    double wl = sum_value(lw);
    if (from_residual) {
      for (int r = 0; r < tx.count; ++r) {
        const int xt = read_lane(tx.tok, r);
        const double delta = read_lane(lane == r ? tx.F - mss_weight(tx.P, tx.Q, A) : 0.0, r);
        if (xt >= c0 && xt < c1 && (xt - c0) / kRun == lane) wl += delta;
      }
    } else {
      const uint64_t cw = load_coherent(mss_slot(a, b, chunk) + kSlotT);
      const float mcs = __uint_as_float(static_cast<uint32_t>(cw));
      wl *= mcs != -INFINITY ? exp2_neg((static_cast<double>(mcs) - static_cast<double>(Mt)) * l2t) : 0.0;
    }
    const int cl = mss_cross_lane(wl, target, before);
    const int k = c0 + cl * kRun + lane;
    const bool have = lane < kRun && k < c1;
    double wk = 0.0;
    if (have) {
      const double pt = static_cast<double>(Elem<DT>::at(trow, k));
      if (from_residual) {
        const double qd = static_cast<double>(Elem<DT>::at(mss_row<DT>(a.draft, a, b, node), k));
        wk = mss_weight(mss_p(pt, prm), mss_q(qd, prm), A);
      } else {
        wk = exp2_neg(__builtin_fma(pt, l2t, -static_cast<double>(Mt) * l2t));
      }
    }
    if (from_residual) {
      for (int r = 0; r < tx.count; ++r) {
        const int xt = read_lane(tx.tok, r);
        const double F = read_lane(tx.F, r);
        if (have && k == xt) wk = F;
      }
    }
    mss_stop(a, b, d, mss_cross_logit(wk, k, before, target), false);
    return;
  }
}

// Blocks: per request b its choose workgroup, then its nchunk stream
// workgroups.  A workgroup waits only for workgroups of its own request,
// whose blocks are contiguous and dispatched in order, and a request never
// waits for a later one: every wait ends (as for the naive-sampling kernel).
template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void tree_mss(MssArgs a) {
  const uint32_t per_b = static_cast<uint32_t>(a.nchunk) + 1u;
  const uint32_t b = blockIdx.x / per_b;
  const uint32_t j = blockIdx.x - b * per_b;
  if (j == 0) {
    __shared__ MssTree tree;
    mss_choose_loop<DT, VEC>(a, static_cast<int>(b), tree);
    mss_exit(a, static_cast<int>(b));
  } else {
    mss_stream_loop<DT, VEC>(a, static_cast<int>(b), static_cast<int>(j - 1u));
  }
}

struct MssLayout {
  size_t ctl, slots, lanes, total;
};

int mss_chunks(int V) { return (V + kMssChunk - 1) / kMssChunk; }

MssLayout mss_layout(int B, int V) {
  const size_t nc = static_cast<size_t>(mss_chunks(V));
  MssLayout L{};
  L.ctl = 0;
  L.slots = align_up(L.ctl + static_cast<size_t>(B) * kCtlStride * sizeof(uint64_t));
  L.lanes = align_up(L.slots + static_cast<size_t>(B) * nc * kSlotWords * sizeof(uint64_t));
  L.total = align_up(L.lanes + static_cast<size_t>(B) * nc * 2 * kWave * sizeof(uint64_t));
  return L;
}

constexpr long long kMssMaxGrid = 1 << 20;
bool mss_fits(int B, int V) {
  return mss_chunks(V) <= kTreeMaxChunks && static_cast<long long>(B) * (mss_chunks(V) + 1) <= kMssMaxGrid;
}

}  // namespace
}  // namespace sv

using namespace sv;

extern "C" size_t sv_tree_mss_workspace_bytes(int B, int N, int V, int dtype) {
  if (dtype != SV_BF16 && dtype != SV_F32) return 0;
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || !mss_fits(B, V)) return 0;
  return mss_layout(B, V).total;
}

extern "C" int spec_verify_tree_mss(const void* target_logits, const void* draft_logits,
                                    const int32_t* node_tokens, const int32_t* parents,
                                    const float* accept_uniforms, const float* draw_uniforms,
                                    const float* temperature, int B, int N, int V, int max_depth,
                                    int dtype, int32_t* out_tokens, int32_t* out_path_nodes,
                                    int32_t* out_num_accepted, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > SV_MAX_VOCAB || max_depth < 0 ||
      max_depth > SV_MAX_TREE_DEPTH || !mss_fits(B, V))
    return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!target_logits || !draft_logits || !node_tokens || !parents || !accept_uniforms || !draw_uniforms ||
      !temperature || !out_tokens || !out_path_nodes || !out_num_accepted || !workspace)
    return SV_ERR_NULL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || !aligned(draft_logits, es)) return SV_ERR_ALIGN;
  const MssLayout L = mss_layout(B, V);
  if (workspace_bytes < L.total || !aligned(workspace, 256)) return SV_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  MssArgs a{};
  a.target = target_logits;
  a.draft = draft_logits;
  a.tokens = node_tokens;
  a.parents = parents;
  a.acc_u = accept_uniforms;
  a.draw_u = draw_uniforms;
  a.temperature = temperature;
  a.B = B;
  a.N = N;
  a.V = V;
  a.max_depth = max_depth;
  a.nchunk = mss_chunks(V);
  a.out_tokens = out_tokens;
  a.out_path = out_path_nodes;
  a.out_n = out_num_accepted;
  a.ctl = reinterpret_cast<uint64_t*>(ws + L.ctl);
  a.slots = reinterpret_cast<uint64_t*>(ws + L.slots);
  a.lanes = reinterpret_cast<uint64_t*>(ws + L.lanes);
  a.spin = spin_limit(kTreeSpinLimit);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && aligned(draft_logits, 16);
  const dim3 grid(static_cast<unsigned>(static_cast<long long>(B) * (a.nchunk + 1)));
  if (dtype == SV_BF16) {
    if (vec) launch(SV_K_TREE_MSS, tree_mss<0, true>, grid, dim3(kWave), 0, stream, a);
    else launch(SV_K_TREE_MSS, tree_mss<0, false>, grid, dim3(kWave), 0, stream, a);
  } else {
    if (vec) launch(SV_K_TREE_MSS, tree_mss<1, true>, grid, dim3(kWave), 0, stream, a);
    else launch(SV_K_TREE_MSS, tree_mss<1, false>, grid, dim3(kWave), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
