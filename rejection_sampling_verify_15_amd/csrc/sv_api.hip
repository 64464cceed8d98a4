// Library-wide C-ABI entry points: status strings, version, workspace clear.
#include <hip/hip_runtime.h>

#include "sv_host.hpp"

namespace sv {

__global__ void fill_zero(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0)
    for (size_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

}  // namespace sv

extern "C" const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "unsupported shape (B, gamma, V, N or max_depth out of range)";
    case SV_ERR_DTYPE: return "unknown dtype";
    case SV_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case SV_ERR_ALIGN: return "logit pointer not aligned to its element size";
    case SV_ERR_HIP: return "HIP runtime error (launch failed)";
    default: return "unknown status";
  }
}

extern "C" const char* sv_version(void) { return "0.1.0"; }

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
  hipLaunchKernelGGL(sv::fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), static_cast<uint4*>(workspace), n16,
                     tail, ntail);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
