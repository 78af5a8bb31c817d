// Counter-based uniforms for the sampling verifier's draws (DScale Sec. III-D, Prefix verifier,
// sampling mode: the accept test and the successor draw take uniforms).
//
// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): a 256-bit counter block and a 128-bit key pass through ten rounds; each round forms
// the 128-bit products of words 0 and 2 with the two round multipliers and rearranges the
// halves with the key, and the key is bumped by the two Weyl constants between rounds.  Word
// i of a stream is word i % 4 of the block at the 128-bit counter base + i / 4; its uniform is
// the word's top 24 bits times 2^-24 (exact in fp32, in [0, 1)).  One thread per block: the
// four 64-bit words come from ten dependent rounds of two 64x64 multiplies, the output is a
// 16-byte store per thread.
#include "dsv_internal.h"

namespace dsv {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;
constexpr int kRngThreads = 256;

__global__ __launch_bounds__(kRngThreads) void philox_uniforms_kernel(uint64_t k0, uint64_t k1,
                                                                      uint64_t c_lo, uint64_t c_hi,
                                                                      int64_t n, float *__restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kRngThreads + threadIdx.x;  // counter block
  if (4 * b >= n) return;
  const uint64_t lo = c_lo + (uint64_t)b;
  uint64_t x0 = lo, x1 = c_hi + (lo < c_lo ? 1u : 0u), x2 = 0, x3 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t h0 = __umul64hi(kPhiloxM0, x0), l0 = kPhiloxM0 * x0;
    const uint64_t h1 = __umul64hi(kPhiloxM1, x2), l1 = kPhiloxM1 * x2;
    x0 = h1 ^ x1 ^ k0;
    x1 = l1;
    x2 = h0 ^ x3 ^ k1;
    x3 = l0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  const float s = 0x1p-24f;
  const f32x4 u = {(float)(uint32_t)(x0 >> 40) * s, (float)(uint32_t)(x1 >> 40) * s,
                   (float)(uint32_t)(x2 >> 40) * s, (float)(uint32_t)(x3 >> 40) * s};
  if (4 * b + 4 <= n && ((uintptr_t)out & 15) == 0) {
    gstore(out + 4 * b, u);
  } else {
    for (int j = 0; j < 4 && 4 * b + j < n; ++j) out[4 * b + j] = u[j];
  }
}

}  // namespace dsv

extern "C" dsv_status dsv_philox_uniforms(uint64_t key0, uint64_t key1, uint64_t counter_lo,
                                          uint64_t counter_hi, int64_t n, float *out,
                                          hipStream_t stream) {
  using namespace dsv;
  if (n < 0 || (n > 0 && !out)) return DSV_ERR_INVALID_ARG;
  if (n == 0) return DSV_OK;
  const int64_t blocks = (n + 3) / 4;
  const int64_t grid = (blocks + kRngThreads - 1) / kRngThreads;
  if (!launch_fits(grid, kRngThreads)) return DSV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(philox_uniforms_kernel, dim3((unsigned)grid), dim3(kRngThreads), 0, stream,
                     key0, key1, counter_lo, counter_hi, n, out);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
