// Chain verification: the acceptance stage of one speculative-decoding round
// for a batch of requests (Leviathan et al.'s Algorithm 1 as restated in the
// close-reading notes 02, section 4, and CMU 15-779 lecture 17 notes, sections
// 2.2-2.4).  See include/specverify.h for the contract.
//
// One launch of one-wave workgroups on the caller's stream (chain_verify),
// whose blocks fall into three parts:
//
//  1. stream items  one per (request, row, chunk of kRowChunk logits),
//                   request-major: the chunk max and, for a sampling row, the
//                   fp32 sum of exp2((x - max) * log2e / T); for a greedy row
//                   the argmax (lowest index).  Every result is one
//                   self-marked 64-bit word, so stream items never wait for
//                   anything.  Draft rows of greedy requests are not read.
//  2. decide items  one per request: waits until every word of its request
//                   carries its mark, merges the chunks in fp64, reads the
//                   logits of the draft tokens from the input rows, runs the
//                   gamma-step test (u <= tau, tau = 1 if q <= p else p / q;
//                   greedy: argmax equality), writes the accepted tokens and
//                   the count, and publishes a sampling request's final draw.
//  3. draw units    per drawing request, one per span of the draw's rows:
//                   fp64 sums of exp((x - max) / T) over the span (all, and
//                   where p > q), handed back as one self-marked record.  The
//                   decide item, which waits for the records, draws the token
//                   -- the smallest k with C_k > u * W (for large batches the
//                   last unit of the request to count itself in draws).
//
// Workgroups are dispatched in block order and every wait is for lower blocks
// (but for a decide item's wait for its units, bounded below), so each wait
// ends.  The decide items and units are dispatched while the last stream items
// are still in flight: early requests are decided and drawn under the
// streaming of later ones.  Very large shapes run the same three parts as
// three launches (chain_stream, chain_decide, chain_units) with capped grids
// whose workgroups stride over the items; there the last unit of a request to
// count itself in draws.  Whoever consumes a workspace word last returns it to
// zero.
//
// Precision: the accept test needs p(x)/q(x) to ~1e-6 and uses the fp32 chunk
// sums merged in fp64; the final draw uses fp64 exponentials and fp64
// normalisers summed by the units, so the inverse CDF matches an fp64
// reference except where u lies within a few ulps of a CDF step.
#include <stdlib.h>

#include <algorithm>
#include <mutex>

#include <atomic>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// workspace records
// ---------------------------------------------------------------------------
// One (row, chunk) result in one 64-bit word: the chunk max's float bits in
// the low half; above them the exp-sum's float bits (sampling) or the argmax
// (greedy), with bit 63 set as the mark -- neither value uses that bit (sums
// are >= 0, indices < 2^31).  A zero word is "not yet written".
constexpr uint64_t kMark = 1ull << 63;

__device__ inline uint64_t pack_partial(float m, int32_t v) {
  return kMark | (static_cast<uint64_t>(static_cast<uint32_t>(v)) << 32) | __float_as_uint(m);
}
__device__ inline float partial_max(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }
__device__ inline int32_t partial_value(uint64_t w) { return static_cast<int32_t>((w >> 32) & 0x7fffffffu); }
__device__ inline bool marked(uint64_t w) { return (w & kMark) != 0; }

// Per (request, draw unit), fp64: sums over the unit of the target (t) and
// draft (d) exponentials, over all tokens and over the tokens with p > q.
// Each field is stored negated: the sums are >= 0, so a stored field has its
// sign bit set (-0.0 included) and a zero word is "not yet written".
enum : int { kUnitAllT = 0, kUnitAllD = 1, kUnitPosT = 2, kUnitPosD = 3, kUnitFields = 4 };
struct UnitRec {
  double f[kUnitFields];
};

// A sampling request's final draw, decided by its decide item and drawn by
// its units.
struct Pending {
  int32_t valid;  // kPendingDraw or kPendingNone once published
  int32_t n;      // accepted drafts; the draw fills out_tokens[b][n]
  int32_t mode;   // kModeResidual / kModeBonus
  float u;        // u[b][gamma]
  float t;        // temperature
  float mt, md;   // maxima of the draw's target row and of draft row n
  uint32_t thr_t, thr_d;  // their filter thresholds (stored keys; 0: none)
  int32_t pad;
  double zt, zd;  // their fp64-merged pass-1 normalisers
};

// A drawing request's Pending record travels to its units as kWireWords
// 64-bit words, each holding one 32-bit word of the record and, above it, the
// record's `valid` value.  The decider stores all words at once with
// device-coherent stores, in no particular order; a unit takes the record once
// every word it reads carries a nonzero mark.
constexpr int kWireWords = sizeof(Pending) / 4;
struct PendingWire {
  uint64_t w[kWireWords];
};

static_assert(sizeof(UnitRec) % 8 == 0 && sizeof(Pending) % 8 == 0, "records are cleared in 64-bit words");
static_assert(kWireWords <= kWave, "one wire word per lane");

enum : int32_t { kModeResidual = 1, kModeBonus = 2 };
enum : int32_t { kPendingDraw = 1, kPendingNone = 2 };  // Pending::valid once published

constexpr int kCounterStride = 32;  // uint32 words per request: one 128-byte line
constexpr int kUnitCounter = 0;     // draw units of the request that have counted in

// The block layout of a call with a sampling hint (batches of up to
// SV_HINT_MAX_BATCH requests): the requests the caller expects to sample
// first, then the unit pool, then the others.  nS < 0: no plan.
struct ChainPlan {
  int32_t nS;                          // requests hinted to sample: order[0, nS)
  int32_t pool;                        // unit-pool workgroups after them
  uint8_t order[SV_HINT_MAX_BATCH];    // request of each segment
};

struct ChainArgs {
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const float* uniforms;
  const float* temperature;
  int B, gamma, V, nchunk, nunit;
  long long nstream;  // stream items: B * (2 * gamma + 1) * nchunk
  int per_req;        // stream items of one request: (2 * gamma + 1) * nchunk
  int32_t* out_tokens;
  int32_t* out_n;
  uint64_t* partials;    // [B][2*gamma+1][nchunk] marked (row, chunk) words
  PendingWire* pending;  // [B]
  UnitRec* units;        // [B][nunit]
  uint32_t* counters;    // [B][kCounterStride]
  const int32_t* gammas; // [B] draft length of each request (ragged calls), or NULL: all gamma
  float* out_tau;        // [B][gamma] tau of each test taken, -1 elsewhere; or NULL
  uint32_t spin;         // poll bound of every wait (kSpinLimit unless a test lowers it)
  const uint32_t* thr;   // [B][2*gamma+1] filter thresholds of a filtered call (key + 1, 0: none), or NULL
  const RowStat* stats;  // [B][2*gamma+1] maximum and kept mass of every row with a cut, or NULL
  const int32_t* top_k;  // [B] of a filtered call, or NULL
  const float* top_p;    // [B] of a filtered call, or NULL
  ChainPlan plan;        // block layout of a hinted call
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
  return exp2_neg((static_cast<double>(x) - static_cast<double>(m)) * l2t);
}

// The same for a whole row: ml2t = m * l2t once per row, then one fused
// multiply-add per logit.  Rounding ml2t shifts every exponent of the row by
// the same amount, which the row's own normaliser cancels.
__device__ inline double exp_row(float x, double ml2t, double l2t) {
  return exp2_neg(__builtin_fma(static_cast<double>(x), l2t, -ml2t));
}

// Whether any lane of the wave holds a logit above -inf in either value: a
// -inf logit (masked, or below a filter's cut) weighs exactly 0, so where no
// lane holds another the exponentials are skipped with no change to any sum.
__device__ inline bool any_finite(float x, float y) {
  return __ballot(x != -INFINITY || y != -INFINITY) != 0ull;
}

// Request classes: 0 samples with its draft rows or has gamma == 0 (it has a
// final draw), 1 is greedy or cannot sample (target rows only), 2 has an
// invalid temperature.
__device__ inline int request_class(const ChainArgs& a, float T) {
  if (!temp_ok(T)) return 2;
  if (T > 0.0f && (a.draft != nullptr || a.gamma == 0)) return 0;
  return 1;
}

// Draft length of request b: gamma, or in a ragged call its own length (-1
// when that lies outside [0, gamma]).  The arrays keep gamma's padded layout.
__device__ inline int req_gamma(const ChainArgs& a, int b) {
  if (!a.gammas) return a.gamma;
  const int g = a.gammas[b];
  return (g >= 0 && g <= a.gamma) ? g : -1;
}

// Rows of a request of length g that are read: target rows 0..g, plus draft
// rows 0..g-1 when sampling (none for an invalid length).
__device__ inline int needed_rows(const ChainArgs& a, float T, int g) {
  if (g < 0) return 0;
  return (T > 0.0f && a.draft != nullptr) ? 2 * g + 1 : g + 1;
}

// Partial row of the lr-th needed row of a request of length g: target rows
// sit at 0..gamma, draft rows at gamma+1..2*gamma.
__device__ inline int phys_row(const ChainArgs& a, int g, int lr) { return lr <= g ? lr : a.gamma + 1 + (lr - g - 1); }

// Whether row k (partial-row numbering) of a request of length g is read.
__device__ inline bool row_in_round(const ChainArgs& a, int g, int k) {
  return g >= 0 && (k <= a.gamma ? k <= g : k - a.gamma - 1 < g);
}

// Upper bound on the polls of a waiting workgroup (seconds at the least);
// every wait is for workgroups dispatched before the waiting one, so the bound
// only guards against a broken dispatch order.  A wait that gives up makes
// its request report SV_GAVE_UP.
constexpr uint32_t kSpinLimit = 1u << 22;

// Lane t < kWireWords stores word t of the record.
__device__ inline void publish_pending(PendingWire* wire, const Pending& d) {
  const int t = threadIdx.x;
  if (t < kWireWords) {
    struct Dwords { uint32_t v[kWireWords]; };
    const Dwords src = __builtin_bit_cast(Dwords, d);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < kWireWords; ++i)
      if (t == i) v = src.v[i];  // constant indices keep the record in registers
    const uint64_t mark = static_cast<uint64_t>(static_cast<uint32_t>(d.valid)) << 32;
    store_coherent(&wire->w[t], mark | v);
  }
}

// Waits until the decision of request b is published (lane t polls word t)
// and returns it to every lane; valid = 0 means the wait gave up.
__device__ Pending wait_pending(const ChainArgs& a, int b) {
  const int lane = threadIdx.x;
  const PendingWire* wire = a.pending + b;
  uint64_t w = 0;
  bool whole = false;
  for (uint32_t spin = 0; spin < a.spin; ++spin) {
    if (lane < kWireWords) w = load_coherent(&wire->w[lane]);
    const uint64_t got = __ballot(lane < kWireWords && (w >> 32) != 0);
    if (got == (1ull << kWireWords) - 1ull) {
      whole = true;
      break;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  struct Dwords { uint32_t v[kWireWords]; };
  Dwords got{};
#pragma unroll
  for (int i = 0; i < kWireWords; ++i) got.v[i] = static_cast<uint32_t>(read_lane(static_cast<int>(w), i));
  Pending d = __builtin_bit_cast(Pending, got);
  if (!whole) d.valid = 0;
  return d;
}

__device__ void write_invalid(const ChainArgs& a, int b) {
  const int G = a.gamma;
  for (int i = threadIdx.x; i <= G; i += kWave) a.out_tokens[static_cast<size_t>(b) * (G + 1) + i] = -1;
  if (threadIdx.x == 0) a.out_n[b] = -1;
}

// ---------------------------------------------------------------------------
// part 1: streaming row statistics
// ---------------------------------------------------------------------------
// Row chunk of one stream item, and so of one row partial.
constexpr int kRowChunk = 4096;
__host__ __device__ inline int row_chunks(int V) { return (V + kRowChunk - 1) / kRowChunk; }

template <int DT, bool VEC, int NT>
struct StreamItem {
  using Raw = RawSlice<DT, VEC, kRowChunk / (NT * (VEC ? Elem<DT>::kVec : 1)), NT>;
  Raw raw;
  float t;  // temperature of the request
};

// Item order: request-major, rows (target 0..gamma, then draft), then chunks.
struct RowItem {
  int b, k, c;
};
__device__ inline RowItem decode_item(const ChainArgs& a, long long item) {
  const int per_req = (2 * a.gamma + 1) * a.nchunk;
  const int rem = static_cast<int>(item % per_req);
  return RowItem{static_cast<int>(item / per_req), rem / a.nchunk, rem % a.nchunk};
}

template <int DT, bool VEC, int NT>
__device__ inline void stream_issue(const ChainArgs& a, const RowItem& r, StreamItem<DT, VEC, NT>& it) {
  const int G = a.gamma;
  const int b = r.b, k = r.k, c = r.c;
  const int pos = k <= G ? k : k - G - 1;
  const void* row = (k <= G) ? row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + k, a.V)
                             : row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + pos, a.V);
  const int c0 = c * kRowChunk;
  it.raw.load(row, c0, min(a.V, c0 + kRowChunk));
  it.t = a.temperature[b];
}

// NT == kWave: one wave per workgroup, reductions within the wave only;
// otherwise the waves combine through LDS.
template <int DT, bool VEC, int NT>
__device__ inline void stream_reduce(const ChainArgs& a, const RowItem& r, const StreamItem<DT, VEC, NT>& it) {
  using Raw = typename StreamItem<DT, VEC, NT>::Raw;
  constexpr int kNW = NT / kWave;
  __shared__ float s_a[kNW];
  __shared__ int s_i[kNW];
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const int b = r.b, k = r.k, c = r.c;
  const int c0 = c * kRowChunk;
  const int c1 = min(a.V, c0 + kRowChunk);
  const bool sampling = it.t > 0.0f;
  auto val = [&](int j, int e) -> float { return it.raw.at(j, e); };
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
    for (int e = 0; e < Raw::kPer; ++e) m = fmaxf(m, val(j, e));
  const int w = threadIdx.x / kWave;
  const bool lane0 = (threadIdx.x % kWave) == 0;
  float out_m;
  int32_t out_v;
  if (!sampling) {
    // chunk max first; only the lanes holding it look for its lowest index
    const float wm = wave_max(m);
    float bm = wm;
    if constexpr (kNW > 1) {
      if (lane0) s_a[w] = wm;
      lds_barrier();
      bm = s_a[0];
#pragma unroll
      for (int i = 1; i < kNW; ++i) bm = fmaxf(bm, s_a[i]);
    }
    int idx = 0x7fffffff;
    if (m == bm) {
#pragma unroll
      for (int j = Raw::kItems - 1; j >= 0; --j)
#pragma unroll
        for (int e = Raw::kPer - 1; e >= 0; --e) {
          const int kk = Raw::index(c0, j, e);
          if (kk < c1 && it.raw.at(j, e) == bm) idx = kk;
        }
    }
    int bi = wave_min(idx);
    if constexpr (kNW > 1) {
      lds_barrier();  // s_a has been read
      if (lane0) s_i[w] = bi;
      lds_barrier();
      bi = s_i[0];
#pragma unroll
      for (int i = 1; i < kNW; ++i) bi = min(bi, s_i[i]);
    }
    out_m = bm;
    out_v = bi;
  } else {
    const float sc = 1.4426950408889634f / it.t;
    float z = 0.0f;
    if (m != -INFINITY) {
      const float msc = m * sc;
#pragma unroll
      for (int j = 0; j < Raw::kItems; ++j)
#pragma unroll
        for (int e = 0; e < Raw::kPer; ++e) z += __builtin_amdgcn_exp2f(__builtin_fmaf(val(j, e), sc, -msc));
    }
    MaxSum rs = wave_maxsum(MaxSum{m, z}, sc);
    if constexpr (kNW > 1) {
      if (lane0) {
        s_a[w] = rs.m;
        s_i[w] = __float_as_int(rs.z);
      }
      lds_barrier();
      rs = MaxSum{s_a[0], __int_as_float(s_i[0])};
#pragma unroll
      for (int i = 1; i < kNW; ++i) rs = maxsum_combine(rs, MaxSum{s_a[i], __int_as_float(s_i[i])}, sc);
    }
    out_m = rs.m;
    out_v = __float_as_int(rs.z);
  }
  if (threadIdx.x == 0)
    store_coherent(&a.partials[(static_cast<size_t>(b) * R + k) * a.nchunk + c], pack_partial(out_m, out_v));
  if constexpr (kNW > 1) lds_barrier();  // s_a / s_i are reused by the next item
}

// Words of a RawSlice past `c1` (loaded from a clamped address) become -inf.
// Vector groups lie wholly inside or outside the row (V is a multiple of the
// vector width on that path).
template <int DT, bool VEC, typename Raw>
__device__ inline void pad_tail(Raw& raw, int c0, int c1) {
  if (c1 - c0 != Raw::kSpan) {
    constexpr uint32_t kNegInf = DT == 0 ? (VEC ? 0xff80ff80u : 0xff80u) : 0xff800000u;
#pragma unroll
    for (int j = 0; j < Raw::kItems; ++j)
      if (Raw::index(c0, j, 0) >= c1) {
#pragma unroll
        for (int q = 0; q < (VEC ? 4 : 1); ++q) raw.w[j][q] = kNegInf;
      }
  }
}

template <int DT, bool VEC, int NT>
__device__ inline void stream_reduce_any(const ChainArgs& a, const RowItem& r, StreamItem<DT, VEC, NT>& it) {
  if (a.thr && it.t > 0.0f) {  // a filtered call: the row's cut applies to the sampling rows
    const uint32_t stored = a.thr[static_cast<size_t>(r.b) * (2 * a.gamma + 1) + r.k];
    if (stored) it.raw.mask_below(stored_threshold(stored));
  }
  const int c0 = r.c * kRowChunk;
  pad_tail<DT, VEC>(it.raw, c0, min(a.V, c0 + kRowChunk));
  stream_reduce<DT, VEC, NT>(a, r, it);
}

// One stream item in a one-wave workgroup (no prefetch, no barriers).
template <int DT, bool VEC>
__device__ inline void stream_once(const ChainArgs& a, const RowItem& r) {
  StreamItem<DT, VEC, kWave> x;
  if (a.gammas && !row_in_round(a, req_gamma(a, r.b), r.k)) return;  // past the request's length
  if (a.stats) {
    // A row the cut search has seen is not read again: its maximum and kept
    // mass stand in for the chunk results (the first chunk carries them, the
    // others are empty).  Its decide item clears the cut only once this
    // item's word is in, so the cut read here is still the search's.
    const size_t ri = static_cast<size_t>(r.b) * (2 * a.gamma + 1) + r.k;
    if (a.thr[ri] != 0u) {
      if (threadIdx.x == 0) {
        uint64_t w = pack_partial(-INFINITY, 0);
        if (r.c == 0) {
          const RowStat st = a.stats[ri];
          w = pack_partial(st.m, __float_as_int(static_cast<float>(st.z)));
        }
        store_coherent(&a.partials[ri * a.nchunk + r.c], w);
      }
      return;
    }
  }
  if (r.k <= a.gamma) {
    stream_issue<DT, VEC, kWave>(a, r, x);  // target rows: the loads do not wait for the temperature
    if (!temp_ok(x.t)) return;
  } else {
    const float T = a.temperature[r.b];
    if (!(temp_ok(T) && T > 0.0f && a.draft != nullptr)) return;
    stream_issue<DT, VEC, kWave>(a, r, x);
  }
  stream_reduce_any<DT, VEC, kWave>(a, r, x);
}

// ---------------------------------------------------------------------------
// part 2: the decision of request b (one wave)
// ---------------------------------------------------------------------------
// Lane s takes slot s = row * gpr + group: a group of consecutive chunks of a
// row, polled kPoll words at a time until all carry their mark, then merged in
// fp64 (the group's max first, then every chunk sum rescaled to it, the
// exponentials independent of each other).  One lane per row combines the
// groups the same way.  The drafts are then tested in order; tokens [0, n]
// (all but a sampling request's slot n) and the count are written, a drawing
// request's outcome is published to its units, and the request's partials
// return to zero.
constexpr int kPoll = 8;
constexpr int kMaxRows = 2 * SV_MAX_GAMMA + 1;
constexpr int kMaxSlots = 2 * kWave;  // nrows * gpr <= max(kWave, kMaxRows)
static_assert(kMaxRows <= kMaxSlots, "slots cover the rows");

// Polls words [c0, min(c0 + kPoll, ce)) of p until all are marked (reads
// beyond ce repeat word ce - 1); false if the wait gave up after `limit` polls.
__device__ inline bool poll_words(const uint64_t* p, int c0, int ce, uint64_t (&w)[kPoll], uint32_t limit) {
  for (uint32_t spin = 0; spin < limit; ++spin) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < kPoll; ++i) {
      w[i] = load_coherent(p + min(c0 + i, ce - 1));
      all = all && marked(w[i]);
    }
    if (all) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

template <int DT, bool VEC, int SPAN, bool kSkip = false>
__device__ bool draw_token(const ChainArgs& a, int b, const Pending& d, bool zero_wire);

// With kDraws (the single launch), the decide item of a drawing request then
// waits for its units' records (of SPAN logits each) and draws the token
// itself.  The count of a drawing request is written by whoever draws (this
// item, or with counted units the last unit), once the draw has its records:
// so SV_GAVE_UP from any wait of the request reaches it through one writer.
template <int DT, bool VEC, int SPAN, bool kDraws, bool kSkip = false>
__device__ void decide_request(const ChainArgs& a, int b) {
  __shared__ float s_gm[kMaxSlots];
  __shared__ double s_gz[kMaxSlots];
  __shared__ int32_t s_garg[kMaxSlots];
  __shared__ float s_m[kMaxRows];
  __shared__ double s_z[kMaxRows];
  __shared__ int32_t s_arg[kMaxRows];
  const int lane = threadIdx.x;
  const int G = a.gamma;
  const int R = 2 * G + 1;
  const float T = a.temperature[b];
  if (request_class(a, T) == 2) {  // nothing was streamed
    write_invalid(a, b);
    if (a.out_tau)
      for (int i = lane; i < G; i += kWave) a.out_tau[static_cast<size_t>(b) * G + i] = -1.0f;
    return;
  }
  const bool sampling = T > 0.0f;
  const double l2t = sampling ? kLog2e / static_cast<double>(T) : 0.0;
  // the request's own length (a ragged call); rows are numbered logically:
  // target rows 0..Gb, then draft rows 0..Gb-1
  const int Gb = req_gamma(a, b);
  const int nrows = needed_rows(a, T, Gb);
  const int gpr = nrows > 0 ? max(1, min(a.nchunk, kWave / nrows)) : 1;  // groups per row
  const int gs = (a.nchunk + gpr - 1) / gpr;              // chunks per group
  const int nslots = nrows * gpr;
  int bad = Gb < 0;
  int lost = 0;  // a wait of this item gave up
  int32_t x = -1;
  float u = 0.0f;
  if (lane < Gb) {
    x = a.tokens[static_cast<size_t>(b) * G + lane];
    bad |= (x < 0 || x >= a.V);
  }
  if (sampling && lane <= Gb) {
    u = a.uniforms[static_cast<size_t>(b) * (G + 1) + lane];
    bad |= !(u >= 0.0f && u < 1.0f);
  }
  if (sampling && Gb > 0 && a.draft == nullptr) bad = 1;
  if (sampling && a.top_k && a.top_k[b] < 1) bad = 1;
  if (sampling && a.top_p) {
    const float pp = a.top_p[b];
    if (!(pp > 0.0f && pp <= 1.0f)) bad = 1;
  }
  // a filtered call: the cut of target row i (lane i <= Gb) and draft row i (lane i < Gb)
  uint32_t thr_t = 0, thr_d = 0;
  if (sampling && a.thr) {
    if (lane <= Gb) thr_t = a.thr[static_cast<size_t>(b) * R + lane];
    if (lane < Gb) thr_d = a.thr[static_cast<size_t>(b) * R + G + 1 + lane];
  }
  // the logits of the draft tokens in target row i and draft row i (-inf
  // below a cut)
  float xt = 0.0f, xd = 0.0f;
  if (sampling && lane < Gb && x >= 0 && x < a.V) {
    xt = Elem<DT>::at(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + lane, a.V), x);
    if (a.draft != nullptr) xd = Elem<DT>::at(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + lane, a.V), x);
    if (xt < stored_threshold(thr_t)) xt = -INFINITY;
    if (xd < stored_threshold(thr_d)) xd = -INFINITY;
  }
  // every partial of the needed rows, whatever the verdict: they are all
  // written, and returned to zero below
  const uint64_t* pb = a.partials + static_cast<size_t>(b) * R * a.nchunk;
  for (int s = lane; s < nslots; s += kWave) {
    const int r = s / gpr;
    const int g = s % gpr;
    const uint64_t* p = pb + static_cast<size_t>(phys_row(a, Gb, r)) * a.nchunk;
    const int cb = g * gs;
    const int ce = min(a.nchunk, cb + gs);
    float m = -INFINITY;
    double z = 0.0;
    ArgMax best{-INFINITY, 0x7fffffff};
    for (int c0 = cb; c0 < ce; c0 += kPoll) {
      uint64_t w[kPoll];
      if (!poll_words(p, c0, ce, w, a.spin)) {
        bad = 1;
        lost = 1;
      }
      if (!sampling) {
#pragma unroll
        for (int i = 0; i < kPoll; ++i)
          if (c0 + i < ce) best = argmax_combine(best, ArgMax{partial_max(w[i]), partial_value(w[i])});
      } else {
        float m8 = m;
#pragma unroll
        for (int i = 0; i < kPoll; ++i)
          if (c0 + i < ce) m8 = fmaxf(m8, partial_max(w[i]));
        if (m8 != -INFINITY) {
          double z8 = (m != -INFINITY) ? z * exp_scaled(m, m8, l2t) : 0.0;
#pragma unroll
          for (int i = 0; i < kPoll; ++i) {
            const float wm = partial_max(w[i]);
            if (c0 + i < ce && wm != -INFINITY)
              z8 += static_cast<double>(__int_as_float(partial_value(w[i]))) * exp_scaled(wm, m8, l2t);
          }
          m = m8;
          z = z8;
        }
      }
    }
    if (sampling) {
      s_gm[s] = m;
      s_gz[s] = z;
    } else {
      s_gm[s] = best.v;
      s_garg[s] = best.i;
    }
  }
  __syncthreads();
  // combine the groups of each row
  for (int r = lane; r < nrows; r += kWave) {
    if (!sampling) {
      ArgMax best{-INFINITY, 0x7fffffff};
      for (int g = 0; g < gpr; ++g) best = argmax_combine(best, ArgMax{s_gm[r * gpr + g], s_garg[r * gpr + g]});
      s_m[r] = best.v;
      s_arg[r] = best.i;
    } else {
      float m = -INFINITY;
      for (int g = 0; g < gpr; ++g) m = fmaxf(m, s_gm[r * gpr + g]);
      double z = 0.0;
      for (int g = 0; g < gpr; ++g) {
        const float gm = s_gm[r * gpr + g];
        if (gm != -INFINITY) z += s_gz[r * gpr + g] * exp_scaled(gm, m, l2t);
      }
      s_m[r] = m;
      s_z[r] = z;
    }
  }
  __syncthreads();
  const bool any_bad = __any(bad);
  const bool any_lost = __any(lost);
  int n = -1;
  double tau = -1.0;
  if (!any_bad) {
    int ok = 1;
    if (lane < Gb) {
      if (!sampling) {
        ok = (x == s_arg[lane]);
        tau = ok ? 1.0 : 0.0;
      } else {
        const double p = exp_scaled(xt, s_m[lane], l2t) / s_z[lane];
        const double q = exp_scaled(xd, s_m[Gb + 1 + lane], l2t) / s_z[Gb + 1 + lane];
        tau = (q <= p) ? 1.0 : p / q;
        ok = (static_cast<double>(u) <= tau);
      }
    }
    const uint64_t fail = __ballot(lane < Gb && !ok);
    n = fail ? static_cast<int>(__builtin_ctzll(fail)) : Gb;
  }
  // the tests taken: positions 0..n (the first rejection included)
  if (a.out_tau)
    for (int i = lane; i < G; i += kWave)
      a.out_tau[static_cast<size_t>(b) * G + i] = (i == lane && i <= n && i < Gb) ? static_cast<float>(tau) : -1.0f;
  // a request with draw units hears the outcome in every case: the draw, or
  // that there is none
  Pending d{};
  const bool drawing = request_class(a, T) == 0;
  if (drawing) {
    if (any_bad) {
      d.valid = kPendingNone;
      d.n = any_lost ? SV_GAVE_UP : -1;  // the count the drawer writes
    } else {
      d.valid = kPendingDraw;
      d.n = n;  // the row of the draw: the rejected position, or Gb for the bonus
      d.mode = n < Gb ? kModeResidual : kModeBonus;
      d.u = read_lane(u, Gb);
      d.t = T;
      d.mt = s_m[n];
      d.zt = s_z[n];
      d.thr_t = static_cast<uint32_t>(read_lane(static_cast<int>(thr_t), n));
      if (n < Gb) {
        d.md = s_m[Gb + 1 + n];
        d.zd = s_z[Gb + 1 + n];
        d.thr_d = static_cast<uint32_t>(read_lane(static_cast<int>(thr_d), n));
      }
    }
    publish_pending(a.pending + b, d);
  }
  // outputs: tokens [0, n), greedy: the argmax at slot n, the rest -1; slot n
  // of a sampling request is filled by its draw
  if (lane <= G) {
    int32_t v = -1;
    bool write = true;
    if (!any_bad) {
      if (lane < n) v = x;
      else if (lane == n) {
        if (sampling) write = false;
        else v = s_arg[n];
      }
    }
    if (write) a.out_tokens[static_cast<size_t>(b) * (G + 1) + lane] = v;
  }
  if (lane == 0 && !drawing) a.out_n[b] = any_lost ? SV_GAVE_UP : n;
  // the workspace words of this request back to zero (the cuts travel in
  // the decision, so no one reads them after this item)
  uint64_t* pz = a.partials + static_cast<size_t>(b) * R * a.nchunk;
  for (int i = lane; i < nrows * a.nchunk; i += kWave) {
    const int r = i / a.nchunk;
    store_coherent(pz + static_cast<size_t>(phys_row(a, Gb, r)) * a.nchunk + (i - r * a.nchunk), 0ull);
  }
  if (a.thr)
    for (int i = lane; i < R; i += kWave) const_cast<uint32_t*>(a.thr)[static_cast<size_t>(b) * R + i] = 0u;
  if (a.stats)
    for (int i = lane; i < R; i += kWave) const_cast<RowStat*>(a.stats)[static_cast<size_t>(b) * R + i] = RowStat{};
  if (kDraws && drawing) {
    // the draw runs beside other requests' units: let this wave issue first
    __builtin_amdgcn_s_setprio(3);
    const bool whole = draw_token<DT, VEC, SPAN, kSkip>(a, b, d, true);
    __builtin_amdgcn_s_setprio(0);
    if (lane == 0) a.out_n[b] = whole ? d.n : SV_GAVE_UP;
  }
}

// ---------------------------------------------------------------------------
// part 3: draw units, and the draw by the last unit of each request
// ---------------------------------------------------------------------------
// A draw unit covers SPAN logits: 512 (one 16-byte group per lane for bf16,
// two for fp32, eight single logits on the scalar path) or 1024.  Small units
// spread a draw over many SIMDs, which a lone request's latency wants; but
// each unit also costs its round trips and a wave slot, and from a couple of
// thousand 512-logit units on, 1024 measured faster (2048 was slower again).
constexpr int kUnitSpanSmall = 512;
constexpr int kUnitSpanLarge = 1024;
constexpr long long kSmallSpanUnits = 2048;  // B * ceil(V / 512) up to which units span 512
template <int DT, bool VEC, int SPAN>
struct Unit {
  static constexpr int kItems = SPAN / (kWave * (VEC ? Elem<DT>::kVec : 1));
  using Raw = RawSlice<DT, VEC, kItems, kWave>;
  static constexpr int kSpan = Raw::kSpan;
  static_assert(kSpan == SPAN, "one span for every path");
};

__device__ inline bool field_marked(double v) { return __double_as_longlong(v) < 0; }
__device__ inline double unit_field(const UnitRec* r, int f) { return -load_coherent_f64(&r->f[f]); }

// Weight of a unit in the final draw (rzt, rzd: reciprocal normalisers).
__device__ inline double unit_weight(double pos_t, double pos_d, double all_t, bool residual, double rzt, double rzd) {
  return residual ? (pos_t * rzt - pos_d * rzd) : all_t;
}

// The draw of request b from its unit records: fp64 normalisers, the weight W
// of the draw (residual mass, or the target normaliser for a bonus draw), the
// unit where the running weight first exceeds u * W, then an fp64 wave scan
// of that unit's logits for the token.  With up to kDrawCache * kWave units
// the records are read once and kept in registers (lane l holds units l,
// l + kWave, ...); otherwise they are read again for each pass.
constexpr int kDrawCache = 5;

// Waits until every record of request b carries its mark (every unit has read
// the decision and handed its sums back); with `cached`, lane l returns the
// values of records l, l + kWave, ... in f, each field read until it arrives.
// False if the wait gave up.
__device__ bool wait_records(const ChainArgs& a, int b, bool cached, double (&f)[kDrawCache][kUnitFields]) {
  const UnitRec* ur = a.units + static_cast<size_t>(b) * a.nunit;
  const int lane = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kDrawCache; ++q)
#pragma unroll
    for (int k = 0; k < kUnitFields; ++k) f[q][k] = (q * kWave + lane < a.nunit) ? 0.0 : -0.0;
  bool whole = false;
  for (uint32_t spin = 0; spin < a.spin; ++spin) {
    bool all = true;
    if (cached) {
#pragma unroll
      for (int q = 0; q < kDrawCache; ++q)
#pragma unroll
        for (int k = 0; k < kUnitFields; ++k) {
          if (!field_marked(f[q][k])) f[q][k] = load_coherent_f64(&ur[q * kWave + lane].f[k]);
          all &= field_marked(f[q][k]);
        }
    } else {
      for (int i = lane; i < a.nunit; i += kWave)
#pragma unroll
        for (int k = 0; k < kUnitFields; ++k) all &= field_marked(load_coherent_f64(&ur[i].f[k]));
    }
    if (__all(all)) {
      whole = true;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
#pragma unroll
  for (int q = 0; q < kDrawCache; ++q)
#pragma unroll
    for (int k = 0; k < kUnitFields; ++k) f[q][k] = -f[q][k];
  return whole;
}

// Also returns the request's records (and, with `zero_wire`, its decision
// wire, which every unit has read once its record is in) to zero; a request
// without a draw only has that done.  False if the wait for the records gave
// up or a unit gave up waiting for the decision (its record then holds +inf
// sums, which no real record can: every exponential is at most 1); the
// token slot is then left alone.
// kSkip: the calls whose rows carry cuts skip the exponentials where a whole
// wave holds only cut logits (the unfiltered kernels carry no such test).
template <int DT, bool VEC, int SPAN, bool kSkip>
__device__ bool draw_token(const ChainArgs& a, int b, const Pending& d, bool zero_wire) {
  using U = Unit<DT, VEC, SPAN>;
  using Raw = typename U::Raw;
  const int G = a.gamma;
  const int lane = threadIdx.x;
  const UnitRec* ur = a.units + static_cast<size_t>(b) * a.nunit;
  const bool cached = a.nunit <= kDrawCache * kWave;
  uint64_t* wz = reinterpret_cast<uint64_t*>(a.units + static_cast<size_t>(b) * a.nunit);
  const int nw = a.nunit * static_cast<int>(sizeof(UnitRec) / 8);
  // 1) the totals: fp64 normalisers of the draw's rows, and the residual mass
  double f[kDrawCache][kUnitFields];
  if (!wait_records(a, b, cached, f)) return false;
  if (zero_wire && lane < kWireWords) store_coherent(&a.pending[b].w[lane], 0ull);
  if (d.valid != kPendingDraw) {
    for (int i = lane; i < nw; i += kWave) store_coherent(wz + i, 0ull);
    return true;
  }
  double tot[kUnitFields] = {0.0, 0.0, 0.0, 0.0};
  if (cached) {
#pragma unroll
    for (int q = 0; q < kDrawCache; ++q)
#pragma unroll
      for (int k = 0; k < kUnitFields; ++k) tot[k] += f[q][k];
    // the records are in registers: return them to zero now, so that the
    // stores drain while the draw goes on
    for (int i = lane; i < nw; i += kWave) store_coherent(wz + i, 0ull);
  } else {
    for (int i = lane; i < a.nunit; i += kWave)
#pragma unroll
      for (int k = 0; k < kUnitFields; ++k) tot[k] += unit_field(ur + i, k);
  }
#pragma unroll
  for (int k = 0; k < kUnitFields; ++k) tot[k] = wave_sum(tot[k]);
  if (tot[kUnitAllT] == INFINITY) {  // a unit gave up
    if (!cached)
      for (int i = lane; i < nw; i += kWave) store_coherent(wz + i, 0ull);
    return false;
  }
  // p = e_t / zt and q = e_d / zd are formed with the reciprocals throughout
  const double rzt = 1.0 / tot[kUnitAllT], rzd = 1.0 / tot[kUnitAllD];
  // an empty residual (p and q equal up to rounding) draws from p of that
  // position instead
  const bool residual = d.mode == kModeResidual && (tot[kUnitPosT] * rzt - tot[kUnitPosD] * rzd > 0.0);
  auto weight_of = [&](int i) -> double {
    return unit_weight(unit_field(ur + i, kUnitPosT), unit_field(ur + i, kUnitPosD), unit_field(ur + i, kUnitAllT),
                       residual, rzt, rzd);
  };
  double wc[kDrawCache];
#pragma unroll
  for (int q = 0; q < kDrawCache; ++q) wc[q] = unit_weight(f[q][kUnitPosT], f[q][kUnitPosD], f[q][kUnitAllT], residual, rzt, rzd);
  double W = 0.0;
  if (cached) {
#pragma unroll
    for (int q = 0; q < kDrawCache; ++q) W += wc[q];
  } else {
    for (int i = lane; i < a.nunit; i += kWave) W += weight_of(i);
  }
  W = wave_sum(W);
  const double target = static_cast<double>(d.u) * W;
  // 2) crossing unit: wave scans of the unit weights in unit order
  int unit = -1, last_unit = -1;
  double before_unit = 0.0, carry = 0.0;
  auto scan_batch = [&](int base, double wu) -> bool {
    const int i = base + lane;
    const double inc = wave_inclusive_sum(wu);
    const double before = carry + lane_move<kDppWaveShr1>(inc);  // lane 0 receives 0
    const uint64_t pos = __ballot(i < a.nunit && wu > 0.0);
    if (pos) last_unit = base + 63 - static_cast<int>(__builtin_clzll(pos));
    const uint64_t hit = __ballot(i < a.nunit && before + wu > target);
    if (hit) {
      const int l = static_cast<int>(__builtin_ctzll(hit));
      unit = base + l;
      before_unit = read_lane(before, l);
      return true;
    }
    carry += read_lane(inc, kWave - 1);
    return false;
  };
  if (cached) {
#pragma unroll
    for (int q = 0; q < kDrawCache; ++q)
      if (q * kWave < a.nunit && scan_batch(q * kWave, wc[q])) break;
  } else {
    for (int base = 0; base < a.nunit; base += kWave)
      if (scan_batch(base, base + lane < a.nunit ? weight_of(base + lane) : 0.0)) break;
  }
  if (unit < 0) {  // rounding left u * W at the very top: take the last positive unit
    unit = last_unit < 0 ? 0 : last_unit;
    double bsum = 0.0;
    if (cached) {
#pragma unroll
      for (int q = 0; q < kDrawCache; ++q)
        if (q * kWave + lane < unit) bsum += wc[q];
    } else {
      for (int i = lane; i < unit; i += kWave) bsum += weight_of(i);
    }
    before_unit = wave_sum(bsum);
  }
  // 3) fp64 wave scans of the crossing unit, one per vector group (group j of
  //    all lanes precedes group j + 1); lane t owns kPer logits of each
  const int c0 = unit * U::kSpan;
  const int c1 = min(a.V, c0 + U::kSpan);
  const double l2t = kLog2e / static_cast<double>(d.t);
  const double mtl = static_cast<double>(d.mt) * l2t, mdl = static_cast<double>(d.md) * l2t;
  const int trow = d.n;  // the rejected position, or the request's length for the bonus
  Raw st, sd;
  st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow, a.V), c0, c1);
  if (residual) sd.load(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V), c0, c1);
  if (d.thr_t) st.mask_below(stored_threshold(d.thr_t));
  if (residual && d.thr_d) sd.mask_below(stored_threshold(d.thr_d));
  pad_tail<DT, VEC>(st, c0, c1);
  if (residual) pad_tail<DT, VEC>(sd, c0, c1);
  int hit = 0x7fffffff;
  int last_pos = -1;
  double run0 = before_unit;
  // group j sits in group 0 of the slices after j shifts
#pragma unroll 1
  for (int j = 0; j < Raw::kItems; ++j) {
    double wk[Raw::kPer];
    if (residual) {
#pragma unroll
      for (int e = 0; e < Raw::kPer; ++e)
        wk[e] = (!kSkip || any_finite(st.at(0, e), sd.at(0, e)))
                    ? fmax(0.0, exp_row(st.at(0, e), mtl, l2t) * rzt - exp_row(sd.at(0, e), mdl, l2t) * rzd)
                    : 0.0;
    } else {
#pragma unroll
      for (int e = 0; e < Raw::kPer; ++e)
        wk[e] = (!kSkip || any_finite(st.at(0, e), st.at(0, e))) ? exp_row(st.at(0, e), mtl, l2t) : 0.0;
    }
    st.shift();
    sd.shift();
    double own = 0.0;
#pragma unroll
    for (int e = 0; e < Raw::kPer; ++e) {
      own += wk[e];
      if (wk[e] > 0.0) last_pos = Raw::index(c0, j, e);
    }
    const double inc = wave_inclusive_sum(own);
    double run = run0 + lane_move<kDppWaveShr1>(inc);
    run0 += read_lane(inc, kWave - 1);
#pragma unroll
    for (int e = 0; e < Raw::kPer; ++e) {
      run += wk[e];
      if (hit == 0x7fffffff && wk[e] > 0.0 && run > target) hit = Raw::index(c0, j, e);
    }
  }
  hit = wave_min(hit);
  last_pos = wave_max_int(last_pos);
  if (lane == 0) a.out_tokens[static_cast<size_t>(b) * (G + 1) + d.n] = (hit != 0x7fffffff) ? hit : last_pos;
  if (!cached)
    for (int i = lane; i < nw; i += kWave) store_coherent(wz + i, 0ull);
  return true;
}

// The drawing requests (class 0) of a batch of at most kRankMaxBatch: lane l
// of mask k stands for request k * kWave + l.  The ranking reads only the
// temperatures, which no workgroup changes.
constexpr int kRankMaxBatch = 4 * kWave;
struct DrawingSet {
  uint64_t m[kRankMaxBatch / kWave];
  int count;
};

__device__ inline DrawingSet drawing_requests(const ChainArgs& a) {
  const int lane = threadIdx.x;
  DrawingSet s{};
  bool v[kRankMaxBatch / kWave];
#pragma unroll
  for (int k = 0; k < kRankMaxBatch / kWave; ++k) {
    const int i = k * kWave + lane;
    v[k] = i < a.B && request_class(a, a.temperature[i]) == 0;
  }
#pragma unroll
  for (int k = 0; k < kRankMaxBatch / kWave; ++k) {
    s.m[k] = __ballot(v[k]);
    s.count += __popcll(s.m[k]);
  }
  return s;
}

// The p-th drawing request (0-based, request order); p < s.count.
__device__ inline int nth_drawing(const DrawingSet& s, int p) {
  const int lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  int seen = 0;
#pragma unroll
  for (int k = 0; k < kRankMaxBatch / kWave; ++k) {
    const int c = __popcll(s.m[k]);
    if (p < seen + c) {
      const uint64_t at = __ballot(((s.m[k] >> lane) & 1ull) && __popcll(s.m[k] & below) == p - seen);
      return k * kWave + static_cast<int>(__builtin_ctzll(at));
    }
    seen += c;
  }
  return -1;
}

// Unit `unit` of request b (a class-0 request): waits for the decision, then
// hands back its share of the final draw as a marked record (zeros when there
// is no draw, +inf when the wait gave up).  With kCounted it also counts
// itself in, and the last unit of the request draws and writes the count.
template <int DT, bool VEC, int SPAN, bool kCounted, bool kSkip = false>
__device__ void unit_work(const ChainArgs& a, int b, int unit) {
  using U = Unit<DT, VEC, SPAN>;
  using Raw = typename U::Raw;
  const int G = a.gamma;
  const int lane = threadIdx.x;
  const Pending d = wait_pending(a, b);
  const bool draw = d.valid == kPendingDraw;
  UnitRec* rec = a.units + static_cast<size_t>(b) * a.nunit + unit;
  double pos_t = 0.0, pos_d = 0.0, all_t = 0.0, all_d = 0.0;
  if (draw) {
    const double l2t = kLog2e / static_cast<double>(d.t);
    const double mtl = static_cast<double>(d.mt) * l2t, mdl = static_cast<double>(d.md) * l2t;
    // p > q under the pass-1 normalisers: e_t * zd > e_d * zt, i.e. e_t > e_d * zt / zd
    const double ratio = d.zt / d.zd;
    const int c0 = unit * U::kSpan;
    const int c1 = min(a.V, c0 + U::kSpan);
    const bool residual = d.mode == kModeResidual;
    const int trow = d.n;  // the rejected position, or the request's length for the bonus
    Raw st, sd;
    st.load(row_ptr<DT>(a.target, static_cast<size_t>(b) * (G + 1) + trow, a.V), c0, c1);
    if (residual) sd.load(row_ptr<DT>(a.draft, static_cast<size_t>(b) * G + d.n, a.V), c0, c1);
    if (d.thr_t) st.mask_below(stored_threshold(d.thr_t));
    if (residual && d.thr_d) sd.mask_below(stored_threshold(d.thr_d));
    pad_tail<DT, VEC>(st, c0, c1);
    // one group at a time: group j sits in group 0 of the slices after j shifts
    if (residual) {
      pad_tail<DT, VEC>(sd, c0, c1);
#pragma unroll 1
      for (int j = 0; j < Raw::kItems; ++j) {
#pragma unroll
        for (int e = 0; e < Raw::kPer; ++e) {
          if (kSkip && !any_finite(st.at(0, e), sd.at(0, e))) continue;
          const double et = exp_row(st.at(0, e), mtl, l2t);
          const double ed = exp_row(sd.at(0, e), mdl, l2t);
          all_t += et;
          all_d += ed;
          if (et > ed * ratio) {
            pos_t += et;
            pos_d += ed;
          }
        }
        st.shift();
        sd.shift();
      }
    } else {
#pragma unroll 1
      for (int j = 0; j < Raw::kItems; ++j) {
#pragma unroll
        for (int e = 0; e < Raw::kPer; ++e)
          if (!kSkip || any_finite(st.at(0, e), st.at(0, e))) all_t += exp_row(st.at(0, e), mtl, l2t);
        st.shift();
      }
    }
    pos_t = wave_sum(pos_t);
    pos_d = wave_sum(pos_d);
    all_t = wave_sum(all_t);
    all_d = wave_sum(all_d);
  }
  // lane f hands over field f, negated (the mark)
  if (lane < kUnitFields) {
    const double v = d.valid == 0 ? INFINITY
                     : lane == kUnitAllT ? all_t : lane == kUnitAllD ? all_d : lane == kUnitPosT ? pos_t : pos_d;
    store_coherent_f64(&rec->f[lane], -v);
  }
  if constexpr (!kCounted) return;
  uint32_t old = 0;
  if (lane == 0) old = arrive(a.counters + static_cast<size_t>(b) * kCounterStride + kUnitCounter);
  const bool last = read_lane(static_cast<int>(old), 0) == a.nunit - 1;
  if (last) {
    // every unit of the request has read the decision and counted in: both
    // words return to zero before the draw, which returns the records
    if (lane < kWireWords) store_coherent(&a.pending[b].w[lane], 0ull);
    if (lane == 0) store_coherent(a.counters + static_cast<size_t>(b) * kCounterStride + kUnitCounter, 0u);
    // the last unit of a request draws while other units may still compute:
    // let its wave issue first on its SIMD
    __builtin_amdgcn_s_setprio(3);
    const bool whole = draw_token<DT, VEC, SPAN, kSkip>(a, b, d, false);
    __builtin_amdgcn_s_setprio(0);
    if (lane == 0) a.out_n[b] = (d.valid != 0 && whole) ? d.n : SV_GAVE_UP;
  }
}

// A pool of `count` workgroups (this one is number `w`) strides over the unit
// tasks (drawing request, unit) in request order, so greedy requests take no
// workgroups and each task waits only for its own request's decision.
// Task counts fit in 32 bits (B * nunit < 2^31 within the shape limits).
template <int DT, bool VEC, int SPAN, bool kCounted, bool kSkip = false>
__device__ void unit_pool(const ChainArgs& a, uint32_t w, uint32_t count) {
  const uint32_t nunit = static_cast<uint32_t>(a.nunit);
  if (a.B <= kRankMaxBatch) {
    const DrawingSet ds = drawing_requests(a);
    const uint32_t tasks = static_cast<uint32_t>(ds.count) * nunit;
    if (w >= tasks) return;
    for (uint32_t t = w; t < tasks; t += count) {
      const uint32_t p = t / nunit;
      unit_work<DT, VEC, SPAN, kCounted, kSkip>(a, nth_drawing(ds, static_cast<int>(p)),
                                                static_cast<int>(t - p * nunit));
    }
  } else {
    const uint32_t tasks = static_cast<uint32_t>(a.B) * nunit;
    if (w >= tasks) return;
    for (uint32_t t = w; t < tasks; t += count) {
      const uint32_t b = t / nunit;
      if (request_class(a, a.temperature[b]) == 0)
        unit_work<DT, VEC, SPAN, kCounted, kSkip>(a, static_cast<int>(b), static_cast<int>(t - b * nunit));
    }
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------
// Blocks come in one segment per request -- its stream items, then its
// decide item, which so waits about as long as its own request's loads take --
// followed by the unit pool.  Up to kDecideDrawsMax requests, a decide item
// then waits for its units' records and draws: the only wait for higher
// blocks, and one that always ends, since those few hundred waiting items at
// most leave most of every XCD's 600-odd wave slots to the units.  Larger
// batches count their units in and the last one draws.  Each workgroup keeps at most 96 VGPRs, so five
// waves share a SIMD (six would force the draw path to spill).
constexpr int kDecideDrawsMax = 256;
static_assert(SV_HINT_MAX_BATCH <= kDecideDrawsMax, "hinted calls have their decide items draw");

// What a block of chain_verify does: a stream item (request, row, chunk), a
// decide item, or pool workgroup w of `count`.  Each part is called from one
// place, so everything stays inlined into the kernel (a call would put the
// arguments in scratch memory).
struct BlockRole {
  enum : int { kNone = 0, kStream = 1, kDecide = 2, kPool = 3, kDraftTail = 4 } kind;
  RowItem item;
  uint32_t w, count;
};

// Chunks of a hinted-greedy request's draft row that one tail workgroup takes.
constexpr uint32_t kTailChunks = 4;

// Default layout: one segment per request (its stream items, then its decide
// item), then the unit pool.
__device__ inline BlockRole default_role(const ChainArgs& a, uint32_t blk) {
  const uint32_t seg = static_cast<uint32_t>(a.per_req) + 1u;
  const uint32_t nseg = static_cast<uint32_t>(a.B) * seg;
  BlockRole r{};
  if (blk < nseg) {
    const uint32_t b = blk / seg;
    const uint32_t rem = blk - b * seg;
    r.item.b = static_cast<int>(b);
    if (rem < static_cast<uint32_t>(a.per_req)) {
      const uint32_t k = rem / static_cast<uint32_t>(a.nchunk);
      r.kind = BlockRole::kStream;
      r.item.k = static_cast<int>(k);
      r.item.c = static_cast<int>(rem - k * static_cast<uint32_t>(a.nchunk));
    } else {
      r.kind = BlockRole::kDecide;
    }
    return r;
  }
  r.kind = BlockRole::kPool;
  r.w = blk - nseg;
  r.count = gridDim.x - nseg;
  return r;
}

// The layout of a hinted call: segments of the requests hinted to sample (all
// rows, then the decide item), the unit pool, the target-row segments of the
// other requests (target rows, then the decide item), and last those
// requests' draft rows, kTailChunks chunks per workgroup, which stream only if
// their request does sample after all.  So the greedy rows stream while the sampling requests are
// decided and drawn.  A wrong hint costs time only: the pool ranks the
// requests by their temperatures, and every request's rows are in the grid.
// The waits for higher blocks (pool and decide items of a request that
// samples against its hint) always end: the host keeps the pool and the
// decide items well below the wave slots of the device, so stream items,
// which never wait, always find slots.
__device__ inline BlockRole planned_role(const ChainArgs& a, uint32_t blk) {
  const uint32_t nc = static_cast<uint32_t>(a.nchunk);
  const uint32_t nS = static_cast<uint32_t>(a.plan.nS);
  const uint32_t nG = static_cast<uint32_t>(a.B) - nS;
  const uint32_t segS = static_cast<uint32_t>(a.per_req) + 1u;
  const uint32_t endS = nS * segS;
  const uint32_t pool = static_cast<uint32_t>(a.plan.pool);
  const uint32_t segT = static_cast<uint32_t>(a.gamma + 1) * nc;
  const uint32_t endG = endS + pool + nG * (segT + 1u);
  BlockRole r{};
  if (blk < endS) {
    const uint32_t s = blk / segS, rem = blk - s * segS;
    r.item.b = a.plan.order[s];
    if (rem < static_cast<uint32_t>(a.per_req)) {
      const uint32_t k = rem / nc;
      r.kind = BlockRole::kStream;
      r.item.k = static_cast<int>(k);
      r.item.c = static_cast<int>(rem - k * nc);
    } else {
      r.kind = BlockRole::kDecide;
    }
    return r;
  }
  if (blk < endS + pool) {
    r.kind = BlockRole::kPool;
    r.w = blk - endS;
    r.count = pool;
    return r;
  }
  if (blk < endG) {
    const uint32_t q = blk - endS - pool, g = q / (segT + 1u), rem = q - g * (segT + 1u);
    r.item.b = a.plan.order[nS + g];
    if (rem < segT) {
      const uint32_t k = rem / nc;
      r.kind = BlockRole::kStream;
      r.item.k = static_cast<int>(k);
      r.item.c = static_cast<int>(rem - k * nc);
    } else {
      r.kind = BlockRole::kDecide;
    }
    return r;
  }
  const uint32_t per_row = (nc + kTailChunks - 1) / kTailChunks;
  const uint32_t dr = static_cast<uint32_t>(a.gamma) * per_row;
  const uint32_t q = blk - endG, g = q / dr, rem = q - g * dr;
  if (g >= nG) return r;
  const uint32_t k = rem / per_row;
  r.kind = BlockRole::kDraftTail;
  r.item = RowItem{a.plan.order[nS + g], a.gamma + 1 + static_cast<int>(k),
                   static_cast<int>((rem - k * per_row) * kTailChunks)};
  return r;
}

// SKIP: a filtered call's form (see draw_token).
template <int DT, bool VEC, int SPAN, bool SKIP = false>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(5))) void chain_verify(ChainArgs a) {
  // 32-bit index arithmetic: this grid has at most kMaxGrid blocks
  const BlockRole r = a.plan.nS >= 0 ? planned_role(a, blockIdx.x) : default_role(a, blockIdx.x);
  const bool draws = a.B <= kDecideDrawsMax;
  if (r.kind == BlockRole::kStream) {
    stream_once<DT, VEC>(a, r.item);
  } else if (r.kind == BlockRole::kDraftTail) {
    const float T = a.temperature[r.item.b];
    if (!(temp_ok(T) && T > 0.0f)) return;  // greedy as hinted: no draft rows
    for (uint32_t j = 0; j < kTailChunks; ++j) {
      const RowItem it{r.item.b, r.item.k, r.item.c + static_cast<int>(j)};
      if (it.c < a.nchunk) stream_once<DT, VEC>(a, it);
    }
  } else if (r.kind == BlockRole::kDecide) {
    if (draws) decide_request<DT, VEC, SPAN, true, SKIP>(a, r.item.b);
    else decide_request<DT, VEC, SPAN, false, SKIP>(a, r.item.b);
  } else if (r.kind == BlockRole::kPool) {
    if (draws) unit_pool<DT, VEC, SPAN, false, SKIP>(a, r.w, r.count);
    else unit_pool<DT, VEC, SPAN, true, SKIP>(a, r.w, r.count);
  }
}

// Very large shapes: the three parts as three launches.  Persistent
// workgroups (as many as fit on the GPU) stride over the stream items in
// request-major order, keeping two items in flight: the loads of the next
// item are issued before the current one is reduced, and the reductions
// synchronise through LDS only, so the prefetch stays outstanding.  Rows that
// no decision needs (draft rows of greedy requests, requests with an invalid
// temperature) are skipped.
enum : uint32_t { kStreamTarget = 1u, kStreamDraft = 2u };

// Which rows of each request are streamed, 2 bits per request, kept in LDS.
struct StreamFlags {
  uint32_t w[SV_MAX_BATCH / 16];
  __device__ inline uint32_t get(int b) const { return (w[b >> 4] >> ((b & 15) * 2)) & 3u; }
};

__device__ inline bool stream_needed(const ChainArgs& a, const StreamFlags& fl, long long item) {
  const RowItem r = decode_item(a, item);
  const uint32_t f = fl.get(r.b);
  if (!(r.k <= a.gamma ? (f & kStreamTarget) != 0 : (f & kStreamDraft) != 0)) return false;
  return !a.gammas || row_in_round(a, req_gamma(a, r.b), r.k);
}

__device__ inline long long stream_next(const ChainArgs& a, const StreamFlags& fl, long long item) {
  while (item < a.nstream && !stream_needed(a, fl, item)) item += gridDim.x;
  return item;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void chain_stream(ChainArgs a) {
  __shared__ StreamFlags s_flags;
  for (int i = threadIdx.x; i < (a.B + 15) / 16; i += kThreads) {
    uint32_t word = 0;
    for (int q = 0; q < 16; ++q) {
      const int b = i * 16 + q;
      if (b >= a.B) break;
      const float T = a.temperature[b];
      uint32_t f = 0;
      if (temp_ok(T)) f = kStreamTarget | ((T > 0.0f && a.draft != nullptr) ? kStreamDraft : 0u);
      word |= f << (q * 2);
    }
    s_flags.w[i] = word;
  }
  __syncthreads();
  long long ia = stream_next(a, s_flags, blockIdx.x);
  if (ia >= a.nstream) return;
  StreamItem<DT, VEC, kThreads> x, y;
  stream_issue<DT, VEC, kThreads>(a, decode_item(a, ia), x);
  for (;;) {
    const long long ib = stream_next(a, s_flags, ia + gridDim.x);
    if (ib < a.nstream) stream_issue<DT, VEC, kThreads>(a, decode_item(a, ib), y);
    stream_reduce_any<DT, VEC, kThreads>(a, decode_item(a, ia), x);
    if (ib >= a.nstream) break;
    const long long ic = stream_next(a, s_flags, ib + gridDim.x);
    if (ic < a.nstream) stream_issue<DT, VEC, kThreads>(a, decode_item(a, ic), x);
    stream_reduce_any<DT, VEC, kThreads>(a, decode_item(a, ib), y);
    if (ic >= a.nstream) break;
    ia = ic;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void chain_decide(ChainArgs a) {
  for (int b = blockIdx.x; b < a.B; b += gridDim.x) {
    decide_request<DT, VEC, kUnitSpanLarge, false>(a, b);
    __syncthreads();  // LDS is reused by the next request
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kWave) void chain_units(ChainArgs a) {
  unit_pool<DT, VEC, kUnitSpanLarge, true>(a, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct ChainLayout {
  size_t partials, pending, units, counters, thr, stats, filt, total;
};

static int units_for(int V, int span) { return (V + span - 1) / span; }

// Sized for the largest draw-unit count (the smallest unit span).
// A filtered call adds the filter's search area.
static ChainLayout chain_layout(int B, int gamma, int V, bool filtered = false, int dtype = SV_BF16) {
  ChainLayout L{};
  const size_t nchunk = static_cast<size_t>(row_chunks(V));
  const size_t R = 2 * static_cast<size_t>(gamma) + 1;
  const size_t nunit = static_cast<size_t>(units_for(V, kUnitSpanSmall));
  size_t off = 0;
  L.partials = off; off = align_up(off + static_cast<size_t>(B) * R * nchunk * sizeof(uint64_t));
  L.pending = off;  off = align_up(off + static_cast<size_t>(B) * sizeof(PendingWire));
  L.units = off;    off = align_up(off + static_cast<size_t>(B) * nunit * sizeof(UnitRec));
  L.counters = off; off = align_up(off + static_cast<size_t>(B) * kCounterStride * sizeof(uint32_t));
  L.thr = off;      off = align_up(off + static_cast<size_t>(B) * R * sizeof(uint32_t));
  L.stats = off;    off = align_up(off + (filtered ? static_cast<size_t>(B) * R * sizeof(RowStat) : 0));
  L.filt = off;     off += filtered ? filter_workspace_bytes(B, gamma, V, dtype) : 0;
  L.total = off;
  return L;
}

// Largest grid of any launch; larger work runs in the three-launch form.
constexpr long long kMaxGrid = 1 << 20;
// Workgroups of the unit pool (at most; fewer when the batch has fewer tasks).
constexpr long long kUnitPool = 16384;

// Workgroups of chain_stream that fit on the current device at once.
template <int DT, bool VEC>
static long long stream_capacity() {
  static std::atomic<long long> cached[64];  // per device, filled on first use (any thread)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_stream<DT, VEC>, kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1)
      return 1024;
    cached[dev].store(static_cast<long long>(per_cu) * cus, std::memory_order_relaxed);
  }
  return cached[dev].load(std::memory_order_relaxed);
}

// Wave slots of chain_verify on the current device (one-wave workgroups).
template <int DT, bool VEC, int SPAN>
static long long verify_capacity() {
  static std::atomic<long long> cached[64];  // per device, filled on first use (any thread)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_verify<DT, VEC, SPAN>, kWave, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1)
      return 0;
    cached[dev].store(static_cast<long long>(per_cu) * cus, std::memory_order_relaxed);
  }
  return cached[dev].load(std::memory_order_relaxed);
}

// The hinted layout's grid (0: the call runs unplanned).  With every request
// hinted to sample, the pool is last, as in the default layout.  Otherwise it
// gets one workgroup per unit of the requests hinted to sample, at least one
// unit's worth (a request may sample against its hint), and at most what
// leaves an eighth of the device's wave slots, beyond the decide items, to the
// stream items after it.
template <int DT, bool VEC, int SPAN>
static long long planned_grid(ChainArgs& a) {
  const long long nS = a.plan.nS, nG = a.B - nS, nc = a.nchunk;
  if (nG == 0) {
    a.plan.pool = static_cast<int32_t>(std::min(static_cast<long long>(a.B) * a.nunit, kUnitPool));
  } else {
    const long long cap = verify_capacity<DT, VEC, SPAN>();
    const long long budget = cap - a.B - cap / 8;
    const long long want = std::max<long long>(nS * a.nunit, a.nunit);
    if (budget < a.nunit) return 0;
    a.plan.pool = static_cast<int32_t>(std::min(want, budget));
  }
  return nS * (a.per_req + 1) + a.plan.pool + nG * ((a.gamma + 1) * nc + 1) +
         nG * a.gamma * ((nc + kTailChunks - 1) / kTailChunks);
}

template <int DT, bool VEC>
static int launch_chain(ChainArgs a, hipStream_t stream) {
  a.nstream = static_cast<long long>(a.B) * (2 * a.gamma + 1) * a.nchunk;
  a.per_req = (2 * a.gamma + 1) * a.nchunk;
  const long long cap = test_hook(SV_HOOK_CHAIN_GRID_CAP);
  // the single launch, with 512- or 1024-logit draw units
  const bool small = static_cast<long long>(a.B) * units_for(a.V, kUnitSpanSmall) <= kSmallSpanUnits;
  a.nunit = units_for(a.V, small ? kUnitSpanSmall : kUnitSpanLarge);
  const long long pool = std::min(static_cast<long long>(a.B) * a.nunit, kUnitPool);
  const long long fused = a.nstream + a.B + pool;
  if (cap <= 0 && test_hook(SV_HOOK_CHAIN_SPLIT) == 0 && fused <= kMaxGrid) {
    long long n = fused;
    if (a.plan.nS >= 0) {
      const long long planned = small ? planned_grid<DT, VEC, kUnitSpanSmall>(a) : planned_grid<DT, VEC, kUnitSpanLarge>(a);
      if (planned > 0 && planned <= kMaxGrid) n = planned;
      else a.plan.nS = -1;
    }
    const dim3 grid(static_cast<unsigned>(n));
    if (a.thr) {  // rows with cuts: the form that skips the exponentials of cut logits
      if (small) launch(SV_K_CHAIN_VERIFY, chain_verify<DT, VEC, kUnitSpanSmall, true>, grid, dim3(kWave), 0, stream, a);
      else launch(SV_K_CHAIN_VERIFY, chain_verify<DT, VEC, kUnitSpanLarge, true>, grid, dim3(kWave), 0, stream, a);
    } else {
      if (small) launch(SV_K_CHAIN_VERIFY, chain_verify<DT, VEC, kUnitSpanSmall>, grid, dim3(kWave), 0, stream, a);
      else launch(SV_K_CHAIN_VERIFY, chain_verify<DT, VEC, kUnitSpanLarge>, grid, dim3(kWave), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
  }
  a.plan.nS = -1;
  // three launches, with 1024-logit draw units
  a.nunit = units_for(a.V, kUnitSpanLarge);
  const long long units = static_cast<long long>(a.B) * a.nunit;
  long long sg = stream_capacity<DT, VEC>();
  if (cap > 0 && cap < sg) sg = cap;
  const long long g = cap > 0 ? cap : kMaxGrid;
  launch(SV_K_CHAIN_STREAM, chain_stream<DT, VEC>, dim3(static_cast<unsigned>(std::min(a.nstream, sg))),
         dim3(kThreads), 0, stream, a);
  launch(SV_K_CHAIN_DECIDE, chain_decide<DT, VEC>, dim3(static_cast<unsigned>(std::min<long long>(a.B, g))),
         dim3(kWave), 0, stream, a);
  launch(SV_K_CHAIN_UNITS, chain_units<DT, VEC>, dim3(static_cast<unsigned>(std::min(units, g))), dim3(kWave), 0,
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

extern "C" size_t sv_chain_filtered_workspace_bytes(int B, int gamma, int V, int dtype) {
  if (B < 0 || B > SV_MAX_BATCH || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB ||
      (dtype != SV_BF16 && dtype != SV_F32))
    return 0;
  return chain_layout(B, gamma, V, true, dtype).total;
}

// Host-side checks of a chain call that need no device (the workspace is
// checked by chain_entry).
static int chain_check(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const float* uniforms, const float* temperature, int B, int gamma, int V, int dtype,
                       const int32_t* out_tokens, const int32_t* out_num_accepted) {
  if (dtype != SV_BF16 && dtype != SV_F32) return SV_ERR_DTYPE;
  if (B < 0 || B > SV_MAX_BATCH || gamma < 0 || gamma > SV_MAX_GAMMA || V < 1 || V > SV_MAX_VOCAB)
    return SV_ERR_SHAPE;
  if (B == 0) return SV_OK;
  if (!target_logits || !temperature || !uniforms || !out_tokens || !out_num_accepted) return SV_ERR_NULL;
  if (gamma > 0 && !draft_tokens) return SV_ERR_NULL;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(target_logits, es) || (draft_logits && !aligned(draft_logits, es))) return SV_ERR_ALIGN;
  return SV_OK;
}

static int chain_entry(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const float* uniforms, const float* temperature, const int32_t* gammas, int B, int gamma,
                       int V, int dtype, int32_t* out_tokens, int32_t* out_num_accepted, float* out_tau,
                       void* workspace, size_t workspace_bytes, void* hip_stream,
                       const uint8_t* sampling_hint = nullptr, const int32_t* top_k = nullptr,
                       const float* top_p = nullptr, bool filtered = false) {
  const int chk = chain_check(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, gamma, V, dtype,
                              out_tokens, out_num_accepted);
  if (chk != SV_OK || B == 0) return chk;
  if (!workspace) return SV_ERR_NULL;
  const ChainLayout L = chain_layout(B, gamma, V, filtered, dtype);
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
  a.nchunk = row_chunks(V);
  a.out_tokens = out_tokens;
  a.out_n = out_num_accepted;
  a.partials = reinterpret_cast<uint64_t*>(ws + L.partials);
  a.pending = reinterpret_cast<PendingWire*>(ws + L.pending);
  a.units = reinterpret_cast<UnitRec*>(ws + L.units);
  a.counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  a.gammas = gammas;
  a.out_tau = gamma > 0 ? out_tau : nullptr;
  a.spin = spin_limit(kSpinLimit);
  if (filtered) {
    a.thr = reinterpret_cast<uint32_t*>(ws + L.thr);
    // bf16 cut searches also leave each cut row's maximum and kept mass, so
    // the verification does not read those rows again
    if (dtype == SV_BF16 && (top_k || top_p)) a.stats = reinterpret_cast<RowStat*>(ws + L.stats);
    a.top_k = top_k;
    a.top_p = top_p;
  }
  a.plan.nS = -1;
  if (sampling_hint && B <= SV_HINT_MAX_BATCH) {
    int s = 0;
    for (int b = 0; b < B; ++b)
      if (sampling_hint[b]) a.plan.order[s++] = static_cast<uint8_t>(b);
    a.plan.nS = s;
    for (int b = 0; b < B; ++b)
      if (!sampling_hint[b]) a.plan.order[s++] = static_cast<uint8_t>(b);
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (filtered) {
    const int st = launch_filter_rows(target_logits, a.draft, temperature, top_k, top_p, B, gamma, V, dtype,
                                      const_cast<uint32_t*>(a.thr), const_cast<RowStat*>(a.stats), ws + L.filt,
                                      stream);
    if (st != SV_OK) return st;
  }
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target_logits, 16) && (!a.draft || aligned(a.draft, 16));
  if (dtype == SV_BF16) return vec ? launch_chain<0, true>(a, stream) : launch_chain<0, false>(a, stream);
  return vec ? launch_chain<1, true>(a, stream) : launch_chain<1, false>(a, stream);
}

extern "C" int spec_verify_chain(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 const float* temperature, int B, int gamma, int V, int dtype,
                                 int32_t* out_tokens, int32_t* out_num_accepted,
                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  return chain_entry(target_logits, draft_logits, draft_tokens, uniforms, temperature, nullptr, B, gamma, V,
                     dtype, out_tokens, out_num_accepted, nullptr, workspace, workspace_bytes, hip_stream);
}

extern "C" int spec_verify_chain_filtered(const void* target_logits, const void* draft_logits,
                                          const int32_t* draft_tokens, const float* uniforms,
                                          const float* temperature, const int32_t* top_k, const float* top_p,
                                          int B, int gamma, int V, int dtype, int32_t* out_tokens,
                                          int32_t* out_num_accepted, void* workspace, size_t workspace_bytes,
                                          void* hip_stream) {
  if (B > 0 && gamma > 0 && !draft_logits) return SV_ERR_NULL;
  return chain_entry(target_logits, draft_logits, draft_tokens, uniforms, temperature, nullptr, B, gamma, V,
                     dtype, out_tokens, out_num_accepted, nullptr, workspace, workspace_bytes, hip_stream, nullptr,
                     top_k, top_p, top_k != nullptr || top_p != nullptr);
}

extern "C" int spec_verify_chain_hinted(const void* target_logits, const void* draft_logits,
                                        const int32_t* draft_tokens, const float* uniforms,
                                        const float* temperature, const uint8_t* sampling_hint, int B, int gamma,
                                        int V, int dtype, int32_t* out_tokens, int32_t* out_num_accepted,
                                        void* workspace, size_t workspace_bytes, void* hip_stream) {
  return chain_entry(target_logits, draft_logits, draft_tokens, uniforms, temperature, nullptr, B, gamma, V,
                     dtype, out_tokens, out_num_accepted, nullptr, workspace, workspace_bytes, hip_stream,
                     sampling_hint);
}

extern "C" int spec_verify_chain_ragged(const void* target_logits, const void* draft_logits,
                                        const int32_t* draft_tokens, const float* uniforms,
                                        const float* temperature, const int32_t* gammas, int B, int gamma,
                                        int V, int dtype, int32_t* out_tokens, int32_t* out_num_accepted,
                                        float* out_accept_prob, void* workspace, size_t workspace_bytes,
                                        void* hip_stream) {
  if (B > 0 && gamma > 0 && !draft_logits) return SV_ERR_NULL;
  return chain_entry(target_logits, draft_logits, draft_tokens, uniforms, temperature, gammas, B, gamma, V,
                     dtype, out_tokens, out_num_accepted, out_accept_prob, workspace, workspace_bytes,
                     hip_stream);
}

// ---------------------------------------------------------------------------
// chain verification without a caller workspace
// ---------------------------------------------------------------------------
// The workspace of spec_verify_chain_noalloc: a static device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, so its device address on each GPU is taken once with
// hipGetSymbolAddress (with that GPU current) and only that address is used.
__device__ __align__(256) unsigned char scratch[SV_CHAIN_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The current device's copy of `scratch`, zero-filled by a fill kernel on
// `stream` the first time it is handed out (*fresh is then true; every call
// that completes leaves it zero again).
static int scratch_on_current_device(hipStream_t stream, void** out, bool* fresh) {
  *fresh = false;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SV_ERR_HIP;
    const int st = sv_workspace_clear(p, SV_CHAIN_SCRATCH_BYTES, stream);
    if (st != SV_OK) return st;
    g_scratch_ptr[dev] = p;
    *fresh = true;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}

extern "C" int spec_verify_chain_noalloc(const void* target_logits, const void* draft_logits,
                                         const int32_t* draft_tokens, const float* uniforms,
                                         const float* temperature, int B, int gamma, int V, int dtype,
                                         int32_t* out_tokens, int32_t* out_num_accepted, void* hip_stream) {
  const int chk = chain_check(target_logits, draft_logits, draft_tokens, uniforms, temperature, B, gamma, V, dtype,
                              out_tokens, out_num_accepted);
  if (chk != SV_OK) return chk;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  void* ws = nullptr;
  bool fresh = false;
  if (B == 0) {  // the reset: zero-fill this GPU's array
    const int st = scratch_on_current_device(stream, &ws, &fresh);
    if (st != SV_OK) return st;
    return fresh ? SV_OK : sv_workspace_clear(ws, SV_CHAIN_SCRATCH_BYTES, stream);
  }
  if (chain_layout(B, gamma, V).total > SV_CHAIN_SCRATCH_BYTES) return SV_ERR_SCRATCH;
  const int st = scratch_on_current_device(stream, &ws, &fresh);
  if (st != SV_OK) return st;
  return chain_entry(target_logits, draft_logits, draft_tokens, uniforms, temperature, nullptr, B, gamma, V, dtype,
                     out_tokens, out_num_accepted, nullptr, ws, SV_CHAIN_SCRATCH_BYTES, hip_stream);
}
