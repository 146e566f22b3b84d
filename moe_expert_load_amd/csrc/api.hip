// Host-only helpers of the C-ABI (version, status text) and the plain device copy
// that serves as the measured HBM reference line for the bandwidth-bound kernels.
#include "common.h"

namespace uep {

constexpr int kCpThreads = 256;
constexpr int kCpVec = 4;   // 16-byte vectors per thread: 16 KiB per workgroup

__global__ __launch_bounds__(kCpThreads) void device_copy_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst,
                                                                 int64_t nvec) {
  const int64_t v0 = (int64_t)blockIdx.x * kCpThreads * kCpVec + threadIdx.x;
  u32x4 buf[kCpVec];
#pragma unroll
  for (int k = 0; k < kCpVec; ++k) {
    const int64_t v = v0 + k * kCpThreads;
    if (v < nvec) buf[k] = src[v];
  }
#pragma unroll
  for (int k = 0; k < kCpVec; ++k) {
    const int64_t v = v0 + k * kCpThreads;
    if (v < nvec) dst[v] = buf[k];
  }
}

// Same workgroup shape as the copy, stores only: the write-only reference line, and a
// fill that callers can put into a captured graph where a memset node is unwanted.
__global__ __launch_bounds__(kCpThreads) void device_fill_kernel(u32x4* __restrict__ dst,
                                                                 int64_t nvec, uint32_t value) {
  const int64_t v0 = (int64_t)blockIdx.x * kCpThreads * kCpVec + threadIdx.x;
  const u32x4 val = {value, value, value, value};
#pragma unroll
  for (int k = 0; k < kCpVec; ++k) {
    const int64_t v = v0 + k * kCpThreads;
    if (v < nvec) dst[v] = val;
  }
}

}  // namespace uep

using namespace uep;

extern "C" const char* uep_version(void) { return "uep 0.1.0 (gfx950)"; }

extern "C" const char* uep_status_string(uep_status s) {
  switch (s) {
    case UEP_OK: return "ok";
    case UEP_EINVAL: return "invalid argument";
    case UEP_EGEOM: return "unsupported geometry";
    case UEP_EWORKSPACE: return "workspace too small";
    case UEP_EHIP: return "HIP launch or runtime failure";
    default: return "unknown status";
  }
}

extern "C" uep_status uep_device_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return UEP_EINVAL;
  if (bytes == 0) return UEP_OK;
  if (!src || !dst) return UEP_EINVAL;
  if (bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return UEP_EGEOM;
  const int64_t nvec = bytes / 16;
  const int64_t per_block = (int64_t)kCpThreads * kCpVec;
  const int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 0x7fffffffll) return UEP_EGEOM;
  hipLaunchKernelGGL(device_copy_kernel, dim3((unsigned)blocks), dim3(kCpThreads), 0,
                     uep_stream(stream), reinterpret_cast<const u32x4*>(src),
                     reinterpret_cast<u32x4*>(dst), nvec);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}

extern "C" uep_status uep_device_fill(void* dst, int64_t bytes, uint32_t value, void* stream) {
  if (bytes < 0) return UEP_EINVAL;
  if (bytes == 0) return UEP_OK;
  if (!dst) return UEP_EINVAL;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return UEP_EGEOM;
  const int64_t nvec = bytes / 16;
  const int64_t per_block = (int64_t)kCpThreads * kCpVec;
  const int64_t blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 0x7fffffffll) return UEP_EGEOM;
  hipLaunchKernelGGL(device_fill_kernel, dim3((unsigned)blocks), dim3(kCpThreads), 0,
                     uep_stream(stream), reinterpret_cast<u32x4*>(dst), nvec, value);
  UEP_CHECK_LAUNCH();
  return UEP_OK;
}
