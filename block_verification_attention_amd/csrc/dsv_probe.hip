// Streaming-read probe: the practical HBM read ceiling against which the verification
// kernel's bandwidth is judged (a plain read of a large buffer, 16-byte loads, four in flight
// per lane, non-temporal).  A measurement helper, not part of the method.
#include "dsv_internal.h"

namespace dsv {

__global__ __launch_bounds__(256) void stream_read_kernel(const f32x4 *__restrict__ a, int64_t n16,
                                                          float *sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const f32x4 x0 = __builtin_nontemporal_load(a + i), x1 = __builtin_nontemporal_load(a + i + stride);
    const f32x4 x2 = __builtin_nontemporal_load(a + i + 2 * stride);
    const f32x4 x3 = __builtin_nontemporal_load(a + i + 3 * stride);
    acc += (x0 + x1) + (x2 + x3);
  }
  for (; i < n16; i += stride) acc += __builtin_nontemporal_load(a + i);
  // keep the loads alive without writing per thread
  if (acc[0] + acc[1] + acc[2] + acc[3] == -1.2345e-30f) sink[0] = acc[0];
}

}  // namespace dsv

extern "C" dsv_status dsv_probe_stream_read(const void *buf, size_t bytes, float *sink,
                                            hipStream_t stream) {
  if (!buf || !sink || bytes < 16 || ((uintptr_t)buf % 16)) return DSV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(dsv::stream_read_kernel, dim3(1024), dim3(256), 0, stream,
                     static_cast<const dsv::f32x4 *>(buf), (int64_t)(bytes / 16), sink);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
