// Library-wide C-ABI entry points: status strings, version, workspace clear,
// kernel timing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "sv_host.hpp"

namespace sv {

__global__ void fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0)
    for (size_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

// ---------------------------------------------------------------------------
// kernel timing sessions
// ---------------------------------------------------------------------------
namespace {
struct TimedLaunch {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
std::atomic<bool> g_timing_on{false};
std::vector<TimedLaunch> g_timed;  // the session's event pairs
size_t g_timed_used = 0;

void destroy_events() {
  for (TimedLaunch& t : g_timed) {
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  g_timed.clear();
  g_timed_used = 0;
}
}  // namespace

void timing_slot(int kernel, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!g_timing_on.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (!g_timing_on.load(std::memory_order_relaxed) || g_timed_used >= g_timed.size()) return;
  TimedLaunch& t = g_timed[g_timed_used++];
  t.kernel = kernel;
  *start = t.start;
  *stop = t.stop;
}

}  // namespace sv

extern "C" const char* sv_kernel_name(int kernel) {
  static const char* const names[SV_K_COUNT] = {
      "chain_verify", "chain_stream", "chain_decide", "chain_units", "tree_init", "tree_node_pass",
      "tree_choose", "probs_row_stats", "probs_residual", "probs_finalize", "fill_zero", "tree_verify",
      "tree_mask", "tree_mss", "topk_rows", "topk_decide", "filter_rows"};
  return (kernel >= 0 && kernel < SV_K_COUNT) ? names[kernel] : "unknown";
}

extern "C" int sv_timing_begin(int capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return SV_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(sv::g_timing_mu);
  sv::g_timing_on.store(false, std::memory_order_release);
  sv::destroy_events();
  sv::g_timed.resize(static_cast<size_t>(capacity), sv::TimedLaunch{-1, nullptr, nullptr});
  for (sv::TimedLaunch& t : sv::g_timed) {
    if (hipEventCreate(&t.start) != hipSuccess || hipEventCreate(&t.stop) != hipSuccess) {
      sv::destroy_events();
      return SV_ERR_HIP;
    }
  }
  sv::g_timing_on.store(true, std::memory_order_release);
  return SV_OK;
}

extern "C" int sv_timing_end(double* total_ms, int* launches, int n) {
  std::lock_guard<std::mutex> lk(sv::g_timing_mu);
  sv::g_timing_on.store(false, std::memory_order_release);
  int status = SV_OK;
  for (size_t i = 0; i < sv::g_timed_used; ++i) {
    const sv::TimedLaunch& t = sv::g_timed[i];
    float ms = 0.0f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) {
      status = SV_ERR_HIP;
      continue;
    }
    if (t.kernel >= 0 && t.kernel < n) {
      if (total_ms) total_ms[t.kernel] += ms;
      if (launches) launches[t.kernel] += 1;
    }
  }
  sv::destroy_events();
  return status;
}

extern "C" const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "unsupported shape (B, gamma, V, N or max_depth out of range)";
    case SV_ERR_DTYPE: return "unknown dtype";
    case SV_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case SV_ERR_ALIGN: return "logit pointer not aligned to its element size";
    case SV_ERR_HIP: return "HIP runtime error (launch failed)";
    case SV_ERR_SCRATCH: return "shape needs more workspace than the static scratch array holds";
    default: return "unknown status";
  }
}

extern "C" const char* sv_version(void) { return "0.1.0"; }

namespace {
std::atomic<long long> g_test_hooks[SV_HOOK_COUNT];
}  // namespace

long long sv::test_hook(int hook) {
  return (hook >= 0 && hook < SV_HOOK_COUNT) ? g_test_hooks[hook].load(std::memory_order_relaxed) : 0;
}

extern "C" int sv_set_test_hook(int hook, long long value) {
  if (hook < 0 || hook >= SV_HOOK_COUNT || value < 0) return SV_ERR_SHAPE;
  g_test_hooks[hook].store(value, std::memory_order_relaxed);
  return SV_OK;
}

extern "C" int sv_workspace_clear(void* workspace, size_t bytes, void* hip_stream) {
  if (bytes == 0) return SV_OK;
  if (!workspace) return SV_ERR_NULL;
  if (!sv::aligned(workspace, 16)) return SV_ERR_WORKSPACE;
  const size_t n16 = bytes / 16;
  unsigned char* tail = static_cast<unsigned char*>(workspace) + n16 * 16;
  const size_t ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  sv::launch(SV_K_WORKSPACE_CLEAR, sv::fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
             static_cast<hipStream_t>(hip_stream), static_cast<uint4*>(workspace), n16, tail, ntail);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
