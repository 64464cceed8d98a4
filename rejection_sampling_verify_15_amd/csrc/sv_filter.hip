// Thresholds of the general consistent filter (top-k and/or top-p over the
// whole vocabulary, the same rule on the target and the draft rows: the
// close-reading notes 02, section 5.4).  Every row of a sampling request gets
// a cut t, stored as order_key(t) + 1 (0: nothing is cut); the chain kernel
// then treats every logit below t as -inf.  See include/specverify.h for the
// contract.
//
// Two searches, one launch per group of rows:
//  - bf16 logits (the exact-count kernel, filter_rows_bf16, below): a bf16
//    logit has one of 65536 values, so one read of the row counting every
//    value gives both cuts exactly, with fp64 masses per value;
//  - fp32 logits (filter_rows): radix selections over order-preserving
//    32-bit keys, one digit at a time (12, 12, then 8 bits).
// The cuts, over keys that order like the logits:
//  - top-k counts: the largest key kt with #{keys >= kt} >= min(k, V), the
//    k-th largest logit (every logit equal to it is kept);
//  - top-p masses over the keys >= kt: the largest key kp whose mass
//    mass(keys >= kp) reaches p * Z, Z the mass of all those keys.  Masses
//    are on the scale of the row maximum M (the largest logit weighs 1), so a
//    weight underflows only where the fp64 softmax's does.
//
// The fp32 radix search: the first digit, the one pass that reads the rows
// from HBM, is split over S workgroups of kSlice logits per row: each builds
// the histogram of its slice in LDS and adds its non-empty bins into the
// row's histogram in the workspace.  The row's last workgroup to arrive
// (nothing waits: the others simply end) reads the merged histogram back,
// clears it, and takes every further digit itself, one pass over the whole
// row per digit (from the caches), each a histogram in LDS of the elements
// whose higher digits match the prefix chosen so far and a block scan from
// the top for the next digit.  An element's top-p weight is
// 2^((x - M) * log2(e) / T), 2^f in fp32 times 2^n in fp64, summed in fp64.
// With top-p alone the split first pass does not know M yet: there each
// element adds its weight relative to the largest value of its bin, and the
// last workgroup rescales the bins once M is known; should the top bin be
// too wide for that (a temperature so small that its top weighs more than
// 2^900 on the scale of M), it takes digit 0 again on the scale of M.  With
// top-k the first pass takes counts only, and the top-p digits follow the
// top-k ones, each a pass of the last workgroup.  These masses have fp32
// precision per element, so an fp32 cut can differ from an fp64 reference
// only where p lies within about 1e-7 of the mass at the cut.
#include <atomic>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {
namespace {

constexpr int kFilterThreads = 512;
constexpr int kFilterWaves = kFilterThreads / kWave;
// Logits per workgroup of the first digit (a multiple of every vector width).
constexpr int kSlice = 65536;
// Rows searched together; larger batches go through the launches in groups of
// this many rows.
constexpr int kFilterSlots = 1024;
constexpr int kMaxBins = 1 << 12;
constexpr size_t kQueueBytes = 256;  // the search area starts with the bf16 item counters
// Largest log2 weight of the top bin's largest value on the scale of M for
// which the first launch's bin-relative weights are kept.
constexpr double kMaxTopLog2 = 900.0;

// What the workgroups of a row share in the workspace besides the histogram
// (all zero between calls).
struct FilterState {
  uint32_t arrivals;  // workgroups that have added their digit-0 bins
  uint32_t max_key;   // order key of the row maximum
  uint32_t pad[14];
};
static_assert(sizeof(FilterState) == 64, "state size");

struct FilterSlot {
  FilterState st;
  uint32_t cnt[kMaxBins];
  double mass[kMaxBins];
};

struct FilterArgs {
  const void* target;
  const void* draft;
  const float* temperature;
  const int32_t* top_k;  // [B] or NULL
  const float* top_p;    // [B] or NULL
  int B, gamma, V;
  int S;                 // slices per row
  int row0;              // first row of this group
  int group;             // rows in this group
  void* slots;           // per-row search areas of the group (FilterSlot, or the bf16 parts)
  uint32_t* queue;       // bf16 item counter and exit counter
  uint32_t* thr;         // [B][2 * gamma + 1]: key + 1, 0 = no cut
  RowStat* stats;        // [B][2 * gamma + 1]: maximum and kept mass of each cut row (bf16), or NULL
};

__device__ inline bool filter_temp_ok(float t) { return isfinite(t) && t >= 1.17549435e-38f; }

// Search key of a logit: bf16 keys differ only in their top 16 bits.
template <int DT>
__device__ inline uint32_t search_key(uint32_t key) {
  return DT == 0 ? (key >> 16) : key;
}
// The full key of a search key (for bf16: the low half of a bf16 value's key
// is 0 for a positive value and 0xffff for a negative one).
template <int DT>
__device__ inline uint32_t full_key(uint32_t k) {
  return DT == 0 ? ((k << 16) | ((k & 0x8000u) ? 0u : 0xffffu)) : k;
}

template <int DT> constexpr int kKeyBits = DT == 0 ? 16 : 32;
// Digit widths, top first: bf16 keys 12 + 4 bits, fp32 keys 12 + 12 + 8.  A
// wide first digit splits every binade into eight bins, so few lanes of a
// wave add to the same bin at once.
template <int DT> constexpr int kLevels = DT == 0 ? 2 : 3;
template <int DT>
__device__ inline int digit_bits(int level) {
  return DT == 0 ? (level == 0 ? 12 : 4) : (level < 2 ? 12 : 8);
}

// The largest search key whose top `bits` bits are `prefix`, and its value
// (the top bins' largest keys are +inf and NaN patterns: their value is taken
// as the largest finite float).
template <int DT>
__device__ inline float prefix_top_value(uint32_t prefix, int bits) {
  const int shift = kKeyBits<DT> - bits;
  const uint32_t k = shift > 0 ? ((prefix << shift) | ((1u << shift) - 1u)) : prefix;
  return fminf(key_value(full_key<DT>(k)), 3.40282347e38f);
}

// 2^t in fp64 for t <= 1100 (t < -1074 gives 0).
__device__ inline double exp2_any(double t) {
  if (t <= 0.0) return exp2_neg(t);
  const double n = __builtin_ceil(t);
  return __builtin_ldexp(exp2_neg(t - n), static_cast<int>(n));
}

// What a row needs: which cuts apply (none for a greedy or invalid request,
// for a draft row without draft logits, and for k >= V with p == 1).
struct RowJob {
  float T;
  double k, p;
  bool cut_k, cut_p;
};

__device__ inline bool row_job(const FilterArgs& a, int row, RowJob& j) {
  const int R = 2 * a.gamma + 1;
  const int b = row / R, r = row - b * R;
  j.T = a.temperature[b];
  if (!filter_temp_ok(j.T)) return false;
  if (r > a.gamma && a.draft == nullptr) return false;
  int k = a.V;
  if (a.top_k) {
    k = a.top_k[b];
    if (k < 1) return false;  // invalid request: the decide item reports it
    k = min(k, a.V);
  }
  float p = 1.0f;
  if (a.top_p) {
    p = a.top_p[b];
    if (!(p > 0.0f && p <= 1.0f)) return false;
  }
  j.k = static_cast<double>(k);
  j.p = static_cast<double>(p);
  j.cut_k = k < a.V;
  j.cut_p = p < 1.0f;
  return j.cut_k || j.cut_p;
}

template <int DT>
__device__ inline const void* row_ptr(const FilterArgs& a, int row) {
  const int R = 2 * a.gamma + 1;
  const int b = row / R, r = row - b * R;
  const size_t es = Elem<DT>::kBytes;
  return r <= a.gamma
      ? static_cast<const char*>(a.target) + (static_cast<size_t>(b) * (a.gamma + 1) + r) * a.V * es
      : static_cast<const char*>(a.draft) + (static_cast<size_t>(b) * a.gamma + (r - a.gamma - 1)) * a.V * es;
}

// Visits n elements of a row slice in batches: each thread issues the loads
// of kBatch vectors (or single elements) before it uses any of them, so a
// pass keeps kBatch * 16 bytes per thread in flight.
constexpr int kBatch = 8;
template <int DT, bool VEC, int NT = kFilterThreads, typename F>
__device__ inline void for_slice(const void* base, int n, F&& fn) {
  if constexpr (VEC) {
    constexpr int kv = Elem<DT>::kVec;
    const int nv = n / kv;
    for (int v0 = 0; v0 < nv; v0 += kBatch * NT) {
      uint4 w[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = v0 + j * NT + static_cast<int>(threadIdx.x);
        w[j] = Elem<DT>::raw(base, (i < nv ? i : 0) * kv);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (v0 + j * NT + static_cast<int>(threadIdx.x) >= nv) continue;
        float x[kv];
        Elem<DT>::unpack(w[j], x);
#pragma unroll
        for (int e = 0; e < kv; ++e) fn(x[e]);
      }
    }
  } else {
    constexpr int kScalar = 4 * kBatch;
    for (int i0 = 0; i0 < n; i0 += kScalar * NT) {
      float x[kScalar];
#pragma unroll
      for (int j = 0; j < kScalar; ++j) {
        const int i = i0 + j * NT + static_cast<int>(threadIdx.x);
        x[j] = Elem<DT>::at(base, i < n ? i : 0);
      }
#pragma unroll
      for (int j = 0; j < kScalar; ++j)
        if (i0 + j * NT + static_cast<int>(threadIdx.x) < n) fn(x[j]);
    }
  }
}

struct FilterHist {
  uint32_t cnt[kMaxBins];
  double mass[kMaxBins];
};

// Block-wide maximum of an order key.
__device__ inline uint32_t block_max_key(uint32_t k, int* s_red) {
  int v = wave_max_int(static_cast<int>(k ^ 0x80000000u));
  __syncthreads();  // earlier readers of s_red are done
  if (threadIdx.x % kWave == 0) s_red[threadIdx.x / kWave] = v;
  __syncthreads();
  v = s_red[0];
  for (int i = 1; i < kFilterWaves; ++i) v = max(v, s_red[i]);
  return static_cast<uint32_t>(v) ^ 0x80000000u;
}

// Block-wide sum (every thread gets it).
__device__ inline double block_total(double v, double (*s_w)[1]) {
  v = wave_sum(v);
  __syncthreads();
  if (threadIdx.x % kWave == 0) s_w[threadIdx.x / kWave][0] = v;
  __syncthreads();
  double t = s_w[0][0];
  for (int i = 1; i < kFilterWaves; ++i) t += s_w[i][0];
  return t;
}

// The slice's histogram of digit `level` over the elements with search key
// >= floor whose `above` higher bits equal `prefix`: counts per bin, and with
// kMass the weights, relative to the bin's largest value (kBinTop) or to the
// row maximum M.  Returns the thread's largest order key when kMax.
template <int DT, bool VEC, bool kMass, bool kBinTop, bool kMax>
__device__ uint32_t slice_hist(const void* base, int n, int width, int above, uint32_t prefix, uint32_t floor,
                               float M, double l2t, FilterHist& h) {
  constexpr int KB = kKeyBits<DT>;
  const int nb = 1 << width;
  for (int i = threadIdx.x; i < nb; i += kFilterThreads) {
    h.cnt[i] = 0u;
    if (kMass) h.mass[i] = 0.0;
  }
  __syncthreads();
  const int shift = KB - above - width;
  const float l2t_f = static_cast<float>(l2t);
  const double Md = static_cast<double>(M);
  uint32_t kmax = 0u;
  for_slice<DT, VEC>(base, n, [&](float x) {
    const uint32_t key = order_key(x);
    if (kMax) kmax = max(kmax, key);
    const uint32_t k = search_key<DT>(key);
    if (k < floor) return;
    if (above > 0 && (k >> (shift + width)) != prefix) return;
    const uint32_t bin = (k >> shift) & static_cast<uint32_t>(nb - 1);
    atomicAdd(&h.cnt[bin], 1u);
    if constexpr (kMass) {
      double w;
      if constexpr (kBinTop) {
        // x and its bin's top lie within an eighth of a binade, so x - top is
        // exact in fp32
        const float top = prefix_top_value<DT>(k >> shift, above + width);
        const float t = fminf(fmaxf((x - top) * l2t_f, -1100.0f), 0.0f);
        const float nn = __builtin_floorf(t);
        w = __builtin_ldexp(static_cast<double>(__builtin_amdgcn_exp2f(t - nn)), static_cast<int>(nn));
      } else {
        const double t = __builtin_fmin(__builtin_fmax((static_cast<double>(x) - Md) * l2t, -1100.0), 0.0);
        const double nn = __builtin_floor(t);
        w = __builtin_ldexp(static_cast<double>(__builtin_amdgcn_exp2f(static_cast<float>(t - nn))),
                            static_cast<int>(nn));
      }
      atomicAdd(&h.mass[bin], w);
    }
  });
  __syncthreads();
  return kmax;
}

// From the top bin down, the first bin b of the nb bins where above + v[b]
// reaches `want`, with above the sum of v over the bins higher than b; the
// lowest non-empty bin, with everything above it, when rounding leaves `want`
// above the total.  Block scan: thread t takes ceil(nb / threads) consecutive
// bins from the top.
__device__ void find_from_top(const double* v, const uint32_t* cnt, int nb, double want, uint32_t* s_pick,
                              double* s_above, double (*s_w)[1]) {
  __syncthreads();  // earlier readers of s_w are done
  const int t = threadIdx.x;
  const int per = (nb + kFilterThreads - 1) / kFilterThreads;
  double own = 0.0;
  for (int j = 0; j < per; ++j) {
    const int bin = nb - 1 - (t * per + j);
    if (bin >= 0) own += v[bin];
  }
  // exclusive prefix over threads (higher bins first)
  double inc = own;
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = __shfl_up(inc, d, kWave);
    if (static_cast<int>(threadIdx.x % kWave) >= d) inc += o;
  }
  const int w = t / kWave;
  if (t % kWave == kWave - 1) s_w[w][0] = inc;
  if (t == 0) *s_pick = 0xffffffffu;
  __syncthreads();
  double base = 0.0;
  for (int i = 0; i < w; ++i) base += s_w[i][0];
  const double before = base + inc - own;
  if (before < want && before + own >= want) {
    double acc = before;
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - (t * per + j);
      if (bin < 0) break;
      if (acc + v[bin] >= want) {
        *s_pick = static_cast<uint32_t>(bin);
        *s_above = acc;
        break;
      }
      acc += v[bin];
    }
  }
  __syncthreads();
  if (*s_pick == 0xffffffffu) {
    int lowest = nb;
    for (int j = 0; j < per; ++j) {
      const int bin = nb - 1 - (t * per + j);
      if (bin >= 0 && cnt[bin]) lowest = min(lowest, bin);
    }
    lowest = wave_min(lowest);
    __syncthreads();
    if (t % kWave == 0) s_w[w][0] = static_cast<double>(lowest);
    __syncthreads();
    int low = nb;
    for (int i = 0; i < kFilterWaves; ++i) low = min(low, static_cast<int>(s_w[i][0]));
    if (low >= nb) low = 0;
    double part = 0.0;
    for (int bin = low + 1 + t; bin < nb; bin += kFilterThreads) part += v[bin];
    const double total = block_total(part, s_w);
    if (t == 0) {
      *s_pick = static_cast<uint32_t>(low);
      *s_above = total;
    }
  }
  __syncthreads();
}

// One search of the finishing workgroup: the digits of one cut, top first.
// Digit 0 may come from the merged histogram already in s_h (have0); every
// other digit is a pass of this workgroup over the whole row.  kMass: top-p
// masses on the scale of M over the keys >= floor, else top-k counts.
// Returns the cut's search key.
template <int DT, bool VEC, bool kMass>
__device__ uint32_t search_digits(const void* row, int V, bool have0, double want, uint32_t floor, float M,
                                  double l2t, double p, FilterHist& h, uint32_t* s_pick, double* s_above,
                                  double (*s_w)[1]) {
  constexpr int L = kLevels<DT>;
  uint32_t prefix = 0u;
  int above = 0;
  for (int level = 0; level < L; ++level) {
    const int width = digit_bits<DT>(level);
    const int nb = 1 << width;
    if (level > 0 || !have0) slice_hist<DT, VEC, kMass, false, false>(row, V, width, above, prefix, floor, M, l2t, h);
    if (!kMass) {
      for (int bin = threadIdx.x; bin < nb; bin += kFilterThreads) h.mass[bin] = static_cast<double>(h.cnt[bin]);
      __syncthreads();
    } else if (level == 0) {
      double part = 0.0;
      for (int bin = threadIdx.x; bin < nb; bin += kFilterThreads) part += h.mass[bin];
      want = p * block_total(part, s_w);
    }
    find_from_top(h.mass, h.cnt, nb, want, s_pick, s_above, s_w);
    want -= *s_above;
    prefix = (prefix << width) | *s_pick;
    above += width;
    __syncthreads();  // s_pick and s_above are read
  }
  return prefix;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kFilterThreads) void filter_rows(FilterArgs a) {
  __shared__ FilterHist s_h;
  __shared__ uint32_t s_pick;
  __shared__ double s_above;
  __shared__ double s_w[kFilterWaves][1];
  __shared__ int s_red[kFilterWaves];
  __shared__ int s_last;
  __shared__ uint32_t s_max;
  const int local = static_cast<int>(blockIdx.x) / a.S;
  const int slice = static_cast<int>(blockIdx.x) - local * a.S;
  const int row_id = a.row0 + local;
  RowJob j;
  if (!row_job(a, row_id, j)) return;
  FilterSlot& sl = static_cast<FilterSlot*>(a.slots)[local];
  const double l2t = kLog2e / static_cast<double>(j.T);
  const void* row = row_ptr<DT>(a, row_id);
  constexpr int W0 = 12;  // digit 0 of either key width
  const int nb0 = 1 << W0;

  // digit 0 over this workgroup's slice: top-k counts, or (top-p alone) the
  // counts and the bin-relative weights; and the slice maximum
  const int s0 = slice * kSlice;
  const int n = min(kSlice, a.V - s0);
  const void* base = static_cast<const char*>(row) + static_cast<size_t>(s0) * Elem<DT>::kBytes;
  const bool mass0 = !j.cut_k;
  const uint32_t kmax = mass0 ? slice_hist<DT, VEC, true, true, true>(base, n, W0, 0, 0u, 0u, 0.0f, l2t, s_h)
                              : slice_hist<DT, VEC, false, false, true>(base, n, W0, 0, 0u, 0u, 0.0f, l2t, s_h);
  for (int bin = threadIdx.x; bin < nb0; bin += kFilterThreads) {
    const uint32_t c = s_h.cnt[bin];
    if (c) {
      __hip_atomic_fetch_add(&sl.cnt[bin], c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (mass0) __hip_atomic_fetch_add(&sl.mass[bin], s_h.mass[bin], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const uint32_t m = block_max_key(kmax, s_red);
  if (threadIdx.x == 0) __hip_atomic_fetch_max(&sl.st.max_key, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_memory();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive(&sl.st.arrivals) == static_cast<uint32_t>(a.S - 1);
  __syncthreads();
  if (!s_last) return;

  // the row's last workgroup: the merged histogram, cleared behind it (each
  // thread issues all its loads before it waits for any), and the maximum
  constexpr int kPer = kMaxBins / kFilterThreads;
  {
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) c[i] = load_coherent(&sl.cnt[i * kFilterThreads + threadIdx.x]);
    double mm[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      mm[i] = (mass0 && c[i]) ? load_coherent_f64(&sl.mass[i * kFilterThreads + threadIdx.x]) : 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int bin = i * kFilterThreads + static_cast<int>(threadIdx.x);
      s_h.cnt[bin] = c[i];
      s_h.mass[bin] = mm[i];
      if (c[i]) {
        store_coherent(&sl.cnt[bin], 0u);
        if (mass0) store_coherent_f64(&sl.mass[bin], 0.0);
      }
    }
  }
  if (threadIdx.x == 0) {
    s_max = load_coherent(&sl.st.max_key);  // every workgroup's maximum is in
    store_coherent(&sl.st.arrivals, 0u);
    store_coherent(&sl.st.max_key, 0u);
  }
  __syncthreads();
  const float M = key_value(s_max);

  uint32_t cut;
  if (j.cut_k) {
    const uint32_t floor_key = search_digits<DT, VEC, false>(row, a.V, true, j.k, 0u, M, l2t, j.p, s_h, &s_pick,
                                                             &s_above, s_w);
    cut = j.cut_p ? search_digits<DT, VEC, true>(row, a.V, false, 0.0, floor_key, M, l2t, j.p, s_h, &s_pick,
                                                 &s_above, s_w)
                  : floor_key;
  } else {
    // top-p alone: digit 0's weights put on the scale of M, unless the top
    // bin is too wide for that
    int hi = -1;
    for (int bin = threadIdx.x; bin < nb0; bin += kFilterThreads)
      if (s_h.cnt[bin]) hi = bin;
    hi = wave_max_int(hi);
    if (threadIdx.x % kWave == 0) s_red[threadIdx.x / kWave] = hi;
    __syncthreads();
    for (int i = 0; i < kFilterWaves; ++i) hi = max(hi, s_red[i]);
    hi = max(hi, 0);
    const double dtop =
        (static_cast<double>(prefix_top_value<DT>(static_cast<uint32_t>(hi), W0)) - static_cast<double>(M)) * l2t;
    const bool rescale = dtop <= kMaxTopLog2;
    if (rescale) {
      for (int bin = threadIdx.x; bin < nb0; bin += kFilterThreads) {
        if (!s_h.cnt[bin]) continue;
        const double d =
            (static_cast<double>(prefix_top_value<DT>(static_cast<uint32_t>(bin), W0)) - static_cast<double>(M)) *
            l2t;
        s_h.mass[bin] *= exp2_any(__builtin_fmin(__builtin_fmax(d, -1100.0), kMaxTopLog2));
      }
    }
    __syncthreads();
    cut = search_digits<DT, VEC, true>(row, a.V, rescale, 0.0, 0u, M, l2t, j.p, s_h, &s_pick, &s_above, s_w);
  }
  if (threadIdx.x == 0) a.thr[row_id] = full_key<DT>(cut) + 1u;
}


// ---------------------------------------------------------------------------
// bf16 rows: exact counts of every value, one read of each row
// ---------------------------------------------------------------------------
// A bf16 logit has one of 65536 values, so a row is fully described by how
// many times each value occurs.  A row is cut into S slices of kB16Slice
// logits; one persistent workgroup per CU takes the (row, slice) items in
// turn and counts the slice's values in LDS (16-bit counters, two to a word:
// a slice has fewer than 65536 logits).  It then writes the slice's part of
// the row, by binade (sign and exponent, the top 9 bits of a key: 128
// evenly spaced values each): for every non-empty binade a record (count,
// largest key present, fp64 mass relative to that key's value) and its 128
// counters.  The row's last item to arrive (nothing waits: the others go on
// to their next item) merges the S records of each binade, one binade per
// thread: the maximum M is the largest key of the row (each item adds its
// own with an atomic maximum), a value v weighs count(v) * 2^((v - M) *
// log2(e) / T) in fp64, and a binade's mass is the sum over the parts of
// the relative mass times the weight of the part's largest key.  Top-k and
// top-p are block scans from the top over the 512 binades, then one wave
// over the 128 values of the chosen binade (the only counters read back).
// The last item also clears what the items wrote.  No row is read twice.
constexpr int kB16Threads = 512;                 // two waves per SIMD: 256 VGPRs each, so a slice's loads
                                                 // stay in registers
constexpr int kB16Waves = kB16Threads / kWave;
constexpr int kB16Slice = 65528;                 // a multiple of 8 below 65536: one value's count fits 16 bits
constexpr int kB16Batch = (kB16Slice + 8 * kB16Threads - 1) / (8 * kB16Threads);  // 16-byte loads per thread
constexpr int kB16Binades = 512;                 // top 9 bits of a 16-bit key
constexpr int kB16PerBinade = 128;               // keys per binade
static_assert(kB16Binades == kB16Threads, "the finisher holds one binade per thread");
constexpr size_t kB16RecBytes = kB16Binades * 16;                 // records
constexpr size_t kB16CountBytes = size_t(1 << 16) * 2;            // 16-bit counters of every key
constexpr size_t kB16PartBytes = kB16RecBytes + kB16CountBytes;
constexpr size_t kB16Head = 256;  // arrival counter, then 1 + the row's largest key (atomic maximum)

__host__ __device__ inline size_t b16_slot_bytes(int S) { return kB16Head + static_cast<size_t>(S) * kB16PartBytes; }

// A binade of one part: ck = count | (largest key << 32), m = fp64 mass
// relative to the largest key's value.  All zero for an empty binade.
struct B16Rec {
  uint64_t ck;
  uint64_t m;
};
__device__ inline B16Rec* b16_recs(char* slot, int s) {
  return reinterpret_cast<B16Rec*>(slot + kB16Head + static_cast<size_t>(s) * kB16PartBytes);
}
// The counters of part s as 64-bit words (four 16-bit counters, lowest key
// first; binade b is words 32 b .. 32 b + 31).
__device__ inline uint64_t* b16_words(char* slot, int s) {
  return reinterpret_cast<uint64_t*>(slot + kB16Head + static_cast<size_t>(s) * kB16PartBytes + kB16RecBytes);
}
__device__ inline uint32_t* b16_row_max(char* slot) { return reinterpret_cast<uint32_t*>(slot) + 1; }

__device__ inline double b16_value(uint32_t k16) { return static_cast<double>(key_value(full_key<0>(k16))); }
// Weight of value v on the scale of M (v <= M); 0 for -inf and the inf / NaN
// patterns.
__device__ inline double b16_weight(double v, double M, double l2t) {
  return (__builtin_isfinite(v) && __builtin_isfinite(M)) ? exp2_neg(__builtin_fmin((v - M) * l2t, 0.0)) : 0.0;
}

// Weights of the 16 values of prefix `pre` (keys 16 pre .. 16 pre + 15)
// relative to value `ref`: the values of one binade are evenly spaced, so
// their weights form a geometric sequence, w(s - 1) = w(s) * q, taken from
// the prefix's highest value present (s_hi) down, every weight at most 1
// when ref is at least that value.  Two fp64 exponentials per prefix; the
// rest are products.  The prefixes of inf and NaN values weigh 0 (only -inf
// is a valid logit there).
struct B16Weights {
  double top, q;  // weight of value s_hi, ratio between neighbours
  int s_hi;       // highest sub-index with a count (-1: none)
};
__device__ inline B16Weights b16_weights(const uint32_t (&c)[16], int pre, double ref, double l2t) {
  int s_hi = -1;
#pragma unroll
  for (int sb = 0; sb < 16; ++sb)
    if (c[sb]) s_hi = sb;
  const double v15 = b16_value(static_cast<uint32_t>(16 * pre + 15));
  const double v14 = b16_value(static_cast<uint32_t>(16 * pre + 14));
  if (s_hi < 0 || !__builtin_isfinite(v15) || !__builtin_isfinite(v14)) return B16Weights{0.0, 0.0, s_hi};
  const double vh = b16_value(static_cast<uint32_t>(16 * pre + s_hi));
  return B16Weights{exp2_neg(__builtin_fmin((vh - ref) * l2t, 0.0)), exp2_neg((v14 - v15) * l2t), s_hi};
}
__device__ inline void b16_unpack(const uint32_t (&w)[8], uint32_t (&c)[16]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    c[2 * q] = w[q] & 0xffffu;
    c[2 * q + 1] = w[q] >> 16;
  }
}
// Mass of a prefix's values relative to ref.
__device__ inline double b16_mass(const uint32_t (&c)[16], int pre, double ref, double l2t) {
  const B16Weights w = b16_weights(c, pre, ref, l2t);
  double m = 0.0, x = w.top;
#pragma unroll
  for (int sb = 15; sb >= 0; --sb) {
    if (sb > w.s_hi) continue;
    if (c[sb]) m += static_cast<double>(c[sb]) * x;
    x *= w.q;
  }
  return m;
}

// Reduction over each group of eight lanes (8 g .. 8 g + 7), all of them
// active; every lane of the group receives the result.
template <typename T, typename Op>
__device__ inline T group8_reduce(T v, Op op) {
  v = op(v, lane_move<kDppQuadSwap1>(v));
  v = op(v, lane_move<kDppQuadSwap2>(v));
  return op(v, lane_move<kDppRowHalfMirror>(v));
}

// Binade b's 128 counters summed over the S parts into s_cnt (threads 0-31,
// one word of four counters each, eight parts' loads at a time); the
// caller synchronises.
__device__ inline void b16_load_binade(char* slot, int S, int b, uint32_t* s_cnt) {
  if (threadIdx.x >= kB16PerBinade / 4) return;
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  constexpr int kPB = 8;
  for (int s0 = 0; s0 < S; s0 += kPB) {
    uint64_t w[kPB];
#pragma unroll
    for (int u = 0; u < kPB; ++u)
      w[u] = s0 + u < S ? load_coherent(b16_words(slot, s0 + u) + 32 * b + threadIdx.x) : 0ull;
#pragma unroll
    for (int u = 0; u < kPB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += static_cast<uint32_t>(w[u] >> (16 * i)) & 0xffffu;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_cnt[4 * threadIdx.x + i] = c[i];
}

// One wave over binade b's values from the top (lane l holds keys
// 128 b + 127 - 2 l and the one below): the first key >= floor16 where acc
// plus the counts (or masses on the scale of M) of the keys from the top
// through it reaches `want`; when rounding leaves `want` above them all, the
// lowest such key present.  With want <= 0 (mass mode) it is the total of
// those keys' masses that is asked for: returned through *total.
__device__ inline uint32_t b16_walk(const uint32_t* s_cnt, int b, uint32_t floor16, double acc, double want,
                                    bool mass, double M, double l2t, double* total) {
  const int lane = threadIdx.x % kWave;
  const int ia = kB16PerBinade - 1 - 2 * lane, ib = ia - 1;
  const uint32_t ka = static_cast<uint32_t>(kB16PerBinade * b + ia), kb = ka - 1u;
  const uint32_t ca = s_cnt[ia], cb = s_cnt[ib];
  const bool ina = ca && ka >= floor16, inb = cb && kb >= floor16;
  double xa = 0.0, xb = 0.0;
  if (ina) xa = mass ? static_cast<double>(ca) * b16_weight(b16_value(ka), M, l2t) : static_cast<double>(ca);
  if (inb) xb = mass ? static_cast<double>(cb) * b16_weight(b16_value(kb), M, l2t) : static_cast<double>(cb);
  const double own = xa + xb;
  const double incl = wave_inclusive_sum(own);
  if (total) *total = read_lane(incl, kWave - 1);
  const double before = acc + lane_move<kDppWaveShr1>(incl);  // lane 0 receives 0
  const double after_a = before + xa;
  const bool ha = ina && after_a >= want, hb = inb && after_a + xb >= want;
  const uint64_t hit = __ballot(ha || hb);
  if (hit) {
    const int l = __builtin_ctzll(hit);
    return static_cast<uint32_t>(read_lane(static_cast<int>(ha ? ka : kb), l));
  }
  const uint64_t any = __ballot(ina || inb);
  if (!any) return floor16;
  const int l = 63 - __builtin_clzll(any);
  return static_cast<uint32_t>(read_lane(static_cast<int>(inb ? kb : ka), l));
}

// Block scan from the top over one value per thread, thread t holding
// binade 511 - t: the first binade (from the top) where the running sum
// reaches want = x (or x times the total of all values, with of_total),
// and the sum above it; -1 when none does.
__device__ inline int b16_find(double v, double x, bool of_total, double* s_wd, int* s_pos, double* s_above,
                               double* above_out, double* want_out) {
  const double inc = wave_inclusive_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();  // earlier readers of s_wd and s_pos are done
  if (threadIdx.x % kWave == kWave - 1) s_wd[w] = inc;
  if (threadIdx.x == 0) *s_pos = 0x7fffffff;
  __syncthreads();
  double base = 0.0, total = 0.0;
  for (int i = 0; i < kB16Waves; ++i) {
    if (i < w) base += s_wd[i];
    total += s_wd[i];
  }
  const double want = of_total ? x * total : x;
  *want_out = want;
  const double acc = base + inc - v;
  const bool hit = acc < want && acc + v >= want;
  if (hit) atomicMin(s_pos, static_cast<int>(threadIdx.x));
  __syncthreads();
  const int best = *s_pos;
  if (hit && static_cast<int>(threadIdx.x) == best) *s_above = acc;
  __syncthreads();
  *above_out = *s_above;
  return best == 0x7fffffff ? -1 : kB16Binades - 1 - best;
}

// Sum over the workgroup of one value per thread; every thread receives it.
__device__ inline double b16_block_sum(double v, double* s_wd) {
  const double inc = wave_inclusive_sum(v);
  __syncthreads();  // earlier readers of s_wd are done
  if (threadIdx.x % kWave == kWave - 1) s_wd[threadIdx.x / kWave] = inc;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kB16Waves; ++i) t += s_wd[i];
  return t;
}

// LDS of the finisher.
struct B16Shared {
  double wd[kB16Waves];
  double above, fm;
  int pos, lowbin;
  uint32_t key;
  uint32_t cnt[kB16PerBinade];  // counters of one binade, summed over the parts
};

// The last item of a row: both cuts from the S parts, stored in thr (with
// `stat`, also the row's maximum and the mass the cut keeps), and the parts
// cleared.
__device__ __attribute__((always_inline)) inline void b16_finish(const RowJob j, char* slot, int S, uint32_t* thr,
                                                                 RowStat* stat, B16Shared* sh) {
  const double l2t = kLog2e / static_cast<double>(j.T);
  const int bn = kB16Binades - 1 - static_cast<int>(threadIdx.x);  // this thread's binade, top first
  uint32_t* row_max = b16_row_max(slot);
  const uint32_t top1 = load_coherent(row_max);
  const double M = b16_value(top1 ? top1 - 1u : 0u);
  // the binade's count and mass over the parts, four parts' records per
  // round of loads; `seen` marks the parts where it is not empty (the first
  // 64), to clear them
  uint32_t cnt = 0u;
  double mass = 0.0;
  uint64_t seen = 0u;
  constexpr int kPC = 4;
  for (int s0 = 0; s0 < S; s0 += kPC) {
    uint64_t ck[kPC], mw[kPC];
#pragma unroll
    for (int u = 0; u < kPC; ++u) {
      const bool in = s0 + u < S;
      B16Rec* r = b16_recs(slot, in ? s0 + u : 0) + bn;
      ck[u] = in ? load_coherent(&r->ck) : 0ull;
      mw[u] = in ? load_coherent(&r->m) : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kPC; ++u) {
      const uint32_t c = static_cast<uint32_t>(ck[u]);
      if (!c) continue;
      cnt += c;
      if (s0 + u < 64) seen |= 1ull << (s0 + u);
      const double mr = __longlong_as_double(static_cast<long long>(mw[u]));
      if (mr > 0.0) mass += mr * b16_weight(b16_value(static_cast<uint32_t>(ck[u] >> 32)), M, l2t);
    }
  }

  uint32_t floor16 = 0u;
  int held = -1;  // the binade whose counters sh->cnt holds
  double above = 0.0;
  if (j.cut_k) {
    double want = 0.0;
    const int b = b16_find(static_cast<double>(cnt), j.k, false, sh->wd, &sh->pos, &sh->above, &above, &want);  // k < V
    b16_load_binade(slot, S, b < 0 ? 0 : b, sh->cnt);
    __syncthreads();
    if (threadIdx.x < kWave) {
      const uint32_t key = b16_walk(sh->cnt, b < 0 ? 0 : b, 0u, above, j.k, false, M, l2t, nullptr);
      if (threadIdx.x == 0) sh->key = key;
    }
    __syncthreads();
    floor16 = sh->key;
    held = b < 0 ? 0 : b;
  }
  uint32_t cut16 = floor16;
  if (j.cut_p) {
    // masses over the keys >= floor16: the floor's own binade value by value
    // (its counters are held), the binades below it none
    const int fb = static_cast<int>(floor16 >> 7);
    double m = bn < fb ? 0.0 : mass;
    if (j.cut_k) {
      if (threadIdx.x < kWave) {
        double fm = 0.0;
        b16_walk(sh->cnt, fb, floor16, 0.0, 0.0, true, M, l2t, &fm);
        if (threadIdx.x == 0) sh->fm = fm;
      }
      __syncthreads();
      if (bn == fb) m = sh->fm;
    }
    double want = 0.0;
    int b = b16_find(m, j.p, true, sh->wd, &sh->pos, &sh->above, &above, &want);
    double want_w = want;
    if (b < 0) {
      // rounding left `want` above the total: the lowest key >= floor16
      // present, in the lowest non-empty binade at or above the floor's
      if (threadIdx.x == 0) sh->lowbin = 0x7fffffff;
      __syncthreads();
      if (cnt && bn >= fb) atomicMin(&sh->lowbin, bn);
      __syncthreads();
      b = sh->lowbin == 0x7fffffff ? fb : sh->lowbin;
      above = 0.0;
      want_w = __builtin_inf();  // no key reaches it: the walk takes the lowest one
    }
    if (b != held) {
      __syncthreads();  // readers of sh->cnt are done
      b16_load_binade(slot, S, b, sh->cnt);
      __syncthreads();
      held = b;
    }
    if (threadIdx.x < kWave) {
      const uint32_t key = b16_walk(sh->cnt, b, floor16, above, want_w, true, M, l2t, nullptr);
      if (threadIdx.x == 0) sh->key = key;
    }
    __syncthreads();
    cut16 = sh->key;
  }
  if (stat) {
    // the kept mass: the binades above the cut's whole, the cut's own binade
    // value by value from the cut up (its counters are held unless the walk
    // fell back to a key outside it)
    const int cb = static_cast<int>(cut16 >> 7);
    const double up = b16_block_sum(bn > cb ? mass : 0.0, sh->wd);
    if (cb != held) {
      __syncthreads();  // readers of sh->cnt are done
      b16_load_binade(slot, S, cb, sh->cnt);
      __syncthreads();
    }
    if (threadIdx.x < kWave) {
      double own = 0.0;
      b16_walk(sh->cnt, cb, cut16, 0.0, 0.0, true, M, l2t, &own);
      if (threadIdx.x == 0) {
        stat->z = up + own;
        stat->m = static_cast<float>(M);
      }
    }
  }
  if (threadIdx.x == 0) {
    *thr = full_key<0>(cut16) + 1u;
    store_coherent(row_max, 0u);
  }

  // clear every word the row's items wrote: the workspace is zero between
  // calls
  for (int s = 0; s < S; ++s) {
    B16Rec* r = b16_recs(slot, s) + bn;
    const bool nz = s < 64 ? ((seen >> s) & 1u) != 0 : static_cast<uint32_t>(load_coherent(&r->ck)) != 0u;
    if (!nz) continue;
    store_coherent(&r->ck, 0ull);
    store_coherent(&r->m, 0ull);
    uint64_t* wd = b16_words(slot, s) + 32 * bn;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) store_coherent(wd + q, 0ull);
  }
}

__device__ inline char* slot_of(const FilterArgs& a, int local) {
  return static_cast<char*>(a.slots) + static_cast<size_t>(local) * b16_slot_bytes(a.S);
}

// A row's job as kept in LDS.
struct B16Job {
  float T, p;
  int32_t k;
  uint32_t cuts;  // bit 0: top-k, bit 1: top-p
};
__device__ inline B16Job b16_pack(const RowJob& j) {
  return B16Job{j.T, static_cast<float>(j.p), static_cast<int32_t>(j.k), (j.cut_k ? 1u : 0u) | (j.cut_p ? 2u : 0u)};
}
__device__ inline RowJob b16_unpack_job(const B16Job& b) {
  return RowJob{b.T, static_cast<double>(b.k), static_cast<double>(b.p), (b.cuts & 1u) != 0, (b.cuts & 2u) != 0};
}

// Where item `it` of the active rows' items reads: its row's job, the
// slice's first logit and length.
__device__ inline bool b16_item(const FilterArgs& a, const uint16_t* rows, const B16Job* jobs, long long it, RowJob& j,
                                const void*& base, int& n, int& row_id, int& slice, int& local) {
  local = rows[it / a.S];
  j = b16_unpack_job(jobs[it / a.S]);
  slice = static_cast<int>(it % a.S);
  row_id = a.row0 + local;
  const int s0 = slice * kB16Slice;
  n = min(kB16Slice, a.V - s0);
  base = static_cast<const char*>(row_ptr<0>(a, row_id)) + static_cast<size_t>(s0) * 2;
  return true;
}

// Every workgroup first lists the group's rows that need a cut (one row per
// thread, in passes); the items of those rows are then handed out in order
// by a counter in the workspace.  A workgroup takes its next item only once
// it has written its part (and finished the row, when it arrived last), so
// the rows' finishes do not pile up on the workgroups that took items
// early; on the vector path it then issues that item's loads at once.  The
// last workgroup to leave resets the counter.
template <bool VEC>
__global__ __launch_bounds__(kB16Threads) void filter_rows_bf16(FilterArgs a) {
  __shared__ uint4 s_pairs[(1 << 16) / 8];  // 65536 16-bit counters
  __shared__ B16Shared sh;
  __shared__ int s_wi[kB16Waves];
  __shared__ int s_last;
  __shared__ uint32_t s_next;
  __shared__ uint16_t s_rows[kFilterSlots];
  __shared__ B16Job s_jobs[kFilterSlots];
  __shared__ int s_nrows;
  static_assert(kFilterSlots % kB16Threads == 0, "whole passes over the rows");
  constexpr int kv = Elem<0>::kVec;
  uint32_t* pairs = reinterpret_cast<uint32_t*>(s_pairs);
  uint32_t* head = a.queue;
  uint32_t* exits = a.queue + 1;
  for (int i = threadIdx.x; i < (1 << 16) / 8; i += kB16Threads) s_pairs[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) s_next = __hip_atomic_fetch_add(head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  {
    // the rows that need a cut, in order: one row per thread in each pass
    int listed = 0;
    for (int r0 = 0; r0 < a.group; r0 += kB16Threads) {
      const int r = r0 + static_cast<int>(threadIdx.x);
      RowJob rj;
      const bool need = r < a.group && row_job(a, a.row0 + r, rj);
      const uint64_t bal = __ballot(need);
      const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
      if (lane == 0) s_wi[w] = __popcll(bal);
      __syncthreads();
      int before = listed, all = listed;
      for (int i = 0; i < kB16Waves; ++i) {
        if (i < w) before += s_wi[i];
        all += s_wi[i];
      }
      if (need) {
        const int q = before + __popcll(bal & ((1ull << lane) - 1ull));
        s_rows[q] = static_cast<uint16_t>(r);
        s_jobs[q] = b16_pack(rj);
      }
      listed = all;
      __syncthreads();  // s_wi is read before the next pass writes it
    }
    if (threadIdx.x == 0) s_nrows = listed;
    __syncthreads();
  }
  const long long items = static_cast<long long>(s_nrows) * a.S;
  long long item = s_next;
  RowJob j{};
  const void* base = nullptr;
  int n = 0, row_id = 0, slice = 0, local = 0;
  bool act = item < items && b16_item(a, s_rows, s_jobs, item, j, base, n, row_id, slice, local);
  uint4 w[kB16Batch];
  auto issue = [&](const void* bp, int nn) {
    const int nv = nn / kv;
#pragma unroll
    for (int q = 0; q < kB16Batch; ++q) {
      const int i = q * kB16Threads + static_cast<int>(threadIdx.x);
      w[q] = Elem<0>::raw(bp, (i < nv ? i : 0) * kv);
    }
  };
  if (VEC && act) issue(base, n);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave, sp = lane & 7;
  while (item < items) {
    if (act) {
      if constexpr (VEC) {
        const int nv = n / kv;  // kB16Batch * kB16Threads vectors cover a slice
#pragma unroll
        for (int q = 0; q < kB16Batch; ++q) {
          if (q * kB16Threads + static_cast<int>(threadIdx.x) >= nv) continue;
          const uint32_t wd[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // two bf16 patterns to their 16-bit order keys at once (a
            // negative one inverted, a positive one with its top bit set;
            // -0 lands on the key below +0, merged after the count)
            const uint32_t kp = wd[e] ^ (((wd[e] >> 15) & 0x00010001u) * 0x7fffu + 0x80008000u);
            atomicAdd(&pairs[(kp & 0xffffu) >> 1], (kp & 1u) * 0xffffu + 1u);
            atomicAdd(&pairs[kp >> 17], ((kp >> 16) & 1u) * 0xffffu + 1u);
          }
        }
      } else {
        for_slice<0, false, kB16Threads>(base, n, [&](float x) {
          const uint32_t k = order_key(x) >> 16;
          atomicAdd(&pairs[k >> 1], 1u << ((k & 1u) << 4));
        });
      }
    }
    __syncthreads();
    if (act) {
      // -0 counts as +0 (their values are equal): key 0x7fff joins key 0x8000
      if (threadIdx.x == 0) {
        const uint32_t neg0 = pairs[0x7fff >> 1] >> 16;
        if (neg0) {
          pairs[0x7fff >> 1] &= 0xffffu;
          pairs[0x8000 >> 1] += neg0;
        }
      }
      __syncthreads();
      // the slice's part, by binade: eight lanes to a binade (sixteen keys
      // each, consecutive lanes on consecutive LDS words), eight binades to a
      // wave per step; the LDS counters read are cleared
      char* slot = slot_of(a, local);
      const double l2t = kLog2e / static_cast<double>(j.T);
      B16Rec* recs = b16_recs(slot, slice);
      uint64_t* words = b16_words(slot, slice);
      int kmax = -1;  // the largest key this thread saw
#pragma unroll 2
      for (int it = 0; it < kB16Binades / (8 * kB16Waves); ++it) {
        const int bn = it * (8 * kB16Waves) + wave * 8 + (lane >> 3);
        const int pre = 8 * bn + sp;  // keys 16 pre .. 16 pre + 15
        const uint4 lo = s_pairs[2 * pre], hi = s_pairs[2 * pre + 1];
        const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (!__ballot((lo.x | lo.y | lo.z | lo.w | hi.x | hi.y | hi.z | hi.w) != 0u)) continue;  // eight empty binades
        // the 16 counters' total from the words' sum: both halves' sums stay
        // below 65536 (a slice's counts do), so neither carries
        uint32_t sum = 0u;
#pragma unroll
        for (int q = 0; q < 8; ++q) sum += wd[q];
        const uint32_t tot = (sum & 0xffffu) + (sum >> 16);
        int top = -1;  // the highest key with a count
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (wd[q]) top = 16 * pre + 2 * q + ((wd[q] >> 16) ? 1 : 0);
        const uint32_t bc = static_cast<uint32_t>(group8_reduce(static_cast<int>(tot), [](int x, int y) { return x + y; }));
        const int bt = group8_reduce(top, [](int x, int y) { return max(x, y); });
        if (!bc) continue;  // the binade's eight lanes alike
        if (tot) {
          s_pairs[2 * pre] = make_uint4(0u, 0u, 0u, 0u);
          s_pairs[2 * pre + 1] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            store_coherent(words + 4 * pre + q,
                           static_cast<uint64_t>(wd[2 * q]) | (static_cast<uint64_t>(wd[2 * q + 1]) << 32));
        }
        // masses only where a top-p cut or the kept mass needs them
        const bool masses = j.cut_p || a.stats != nullptr;
        double mp = 0.0;
        if (masses && tot) {
          uint32_t c[16];
          b16_unpack(wd, c);
          mp = b16_mass(c, pre, b16_value(static_cast<uint32_t>(bt)), l2t);
        }
        const double m = masses ? group8_reduce(mp, [](double x, double y) { return x + y; }) : 0.0;
        if (sp == 0) {
          store_coherent(&recs[bn].ck, static_cast<uint64_t>(bc) | (static_cast<uint64_t>(bt) << 32));
          store_coherent(&recs[bn].m, static_cast<uint64_t>(__double_as_longlong(m)));
        }
        kmax = max(kmax, bt);
      }
      kmax = wave_max_int(kmax);
      if (lane == 0 && kmax >= 0)
        __hip_atomic_fetch_max(b16_row_max(slot), static_cast<uint32_t>(kmax) + 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      wait_memory();
      __syncthreads();
      uint32_t* arrivals = reinterpret_cast<uint32_t*>(slot);
      if (threadIdx.x == 0) s_last = arrive(arrivals) == static_cast<uint32_t>(a.S - 1);
      __syncthreads();
      if (s_last) {
        if (threadIdx.x == 0) store_coherent(arrivals, 0u);
        b16_finish(j, slot, a.S, a.thr + row_id, a.stats ? a.stats + row_id : nullptr, &sh);
      }
    }
    // the next item is taken only now (a workgroup that finished a row takes
    // it later than one that did not), and its loads go out
    __syncthreads();
    if (threadIdx.x == 0) s_next = __hip_atomic_fetch_add(head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const long long nitem = s_next;
    RowJob nj{};
    const void* nbase = nullptr;
    int nn = 0, nrow = 0, nslice = 0, nlocal = 0;
    const bool nact = nitem < items && b16_item(a, s_rows, s_jobs, nitem, nj, nbase, nn, nrow, nslice, nlocal);
    if (VEC && nact) issue(nbase, nn);
    item = nitem;
    j = nj;
    base = nbase;
    n = nn;
    row_id = nrow;
    slice = nslice;
    local = nlocal;
    act = nact;
  }
  // the last workgroup out resets the counter for the next call
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
    store_coherent(head, 0u);
    store_coherent(exits, 0u);
  }
}
}  // namespace

int b16_slices(int V) { return (V + kB16Slice - 1) / kB16Slice; }

// Rows searched together: at most kFilterSlots, and for bf16 rows no more
// than fit in kB16GroupBytes of parts.
constexpr size_t kB16GroupBytes = size_t(256) << 20;
long long filter_group_rows(int V, int dtype) {
  if (dtype != SV_BF16) return kFilterSlots;
  const long long fit = static_cast<long long>(kB16GroupBytes / b16_slot_bytes(b16_slices(V)));
  return fit < 1 ? 1 : (fit < kFilterSlots ? fit : kFilterSlots);
}

// Compute units of the current device (cached per device).
long long device_cus() {
  static std::atomic<long long> cached[64];  // per device, filled on first use (any thread)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev].load(std::memory_order_relaxed) == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cached[dev].load(std::memory_order_relaxed);
}

size_t filter_workspace_bytes(int B, int gamma, int V, int dtype) {
  const long long rows = static_cast<long long>(B) * (2 * gamma + 1);
  const long long group = filter_group_rows(V, dtype);
  const long long slots = rows < group ? rows : group;
  return kQueueBytes +
         align_up(static_cast<size_t>(slots) * (dtype == SV_BF16 ? b16_slot_bytes(b16_slices(V)) : sizeof(FilterSlot)));
}

int launch_filter_rows(const void* target, const void* draft, const float* temperature, const int32_t* top_k,
                       const float* top_p, int B, int gamma, int V, int dtype, uint32_t* thr, void* stats,
                       void* slots, hipStream_t stream) {
  FilterArgs a{};
  a.target = target;
  a.draft = gamma > 0 ? draft : nullptr;
  a.temperature = temperature;
  a.top_k = top_k;
  a.top_p = top_p;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.S = dtype == SV_BF16 ? b16_slices(V) : (V + kSlice - 1) / kSlice;
  a.queue = static_cast<uint32_t*>(slots);
  a.slots = static_cast<char*>(slots) + kQueueBytes;
  a.thr = thr;
  a.stats = dtype == SV_BF16 ? static_cast<RowStat*>(stats) : nullptr;
  const long long rows = static_cast<long long>(B) * (2 * gamma + 1);
  if (rows == 0 || (!top_k && !top_p)) return SV_OK;
  const int kv = dtype == SV_BF16 ? Elem<0>::kVec : Elem<1>::kVec;
  const bool vec = (V % kv == 0) && aligned(target, 16) && (!a.draft || aligned(a.draft, 16));
  const long long group = filter_group_rows(V, dtype);
  for (long long r0 = 0; r0 < rows; r0 += group) {
    a.row0 = static_cast<int>(r0);
    const long long n = rows - r0 < group ? rows - r0 : group;
    a.group = static_cast<int>(n);
    const dim3 grid(static_cast<unsigned>(n * a.S));
    if (dtype == SV_BF16) {
      // persistent: one workgroup per CU (the LDS table allows no more)
      const long long items = n * a.S;
      const dim3 pgrid(static_cast<unsigned>(items < device_cus() ? items : device_cus()));
      if (vec) launch(SV_K_FILTER_ROWS, filter_rows_bf16<true>, pgrid, dim3(kB16Threads), 0, stream, a);
      else launch(SV_K_FILTER_ROWS, filter_rows_bf16<false>, pgrid, dim3(kB16Threads), 0, stream, a);
    } else {
      if (vec) launch(SV_K_FILTER_ROWS, filter_rows<1, true>, grid, dim3(kFilterThreads), 0, stream, a);
      else launch(SV_K_FILTER_ROWS, filter_rows<1, false>, grid, dim3(kFilterThreads), 0, stream, a);
    }
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace sv
