// Streaming-read probe: the practical HBM read ceiling against which the verification
// kernel's bandwidth is measured.  A plain read of a large buffer in the access pattern of the
// verification kernel: each of two workgroups per CU streams one contiguous range in 32 KB
// blocks (every thread issues eight 16-byte non-temporal loads per block).  A measurement
// helper, not part of the method.
#include "dsv_internal.h"

namespace dsv {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlock = kProbeThreads * 8;  // 16-byte elements per 32 KB block

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4 *__restrict__ a, int64_t n16,
                                                                  int64_t per_wg, float *sink) {
  const int64_t lo = (int64_t)blockIdx.x * per_wg;
  const int64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = lo + threadIdx.x;
  for (; i + 7 * kProbeThreads < hi; i += kProbeBlock) {
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = gload_stream<u32x4>(a + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  for (; i < hi; i += kProbeThreads) acc ^= gload_stream<u32x4>(a + i);
  // keep the loads alive without writing per thread
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u && threadIdx.x == 0) gstore(sink, 0.f);
}

}  // namespace dsv

extern "C" dsv_status dsv_probe_stream_read(const void *buf, size_t bytes, float *sink,
                                            hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || ((uintptr_t)buf % 16)) return DSV_ERR_INVALID_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return DSV_ERR_HIP;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t wgs = 2 * (int64_t)cus;
  // each workgroup's range: a whole number of 32 KB blocks
  const int64_t per_wg = ((n16 + wgs - 1) / wgs + dsv::kProbeBlock - 1) / dsv::kProbeBlock * dsv::kProbeBlock;
  const int64_t grid = (n16 + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(dsv::stream_read_kernel, dim3((unsigned)grid), dim3(dsv::kProbeThreads), 0, stream,
                     static_cast<const dsv::u32x4 *>(buf), n16, per_wg, sink);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
