// Flat-buffer packer: exclusive-scan offsets and identical-row-mapping slot fields.
//
// DScale (arXiv HTML), Sec. III-C "Flat-buffer packer" and Fig. 6: allocated prefixes of
// lengths k_i occupy one buffer of capacity M_bs at prefix-sum offsets, and the same mapping
// is applied to token ids, positions and cache references; inactive lengths are zero and
// tail slots hold placeholders.  Sec. II-C (Challenge 3) is why the offsets are recomputed
// on the device every step: when lengths change from [4,12,8] to [10,8,6] the request
// boundaries move, and no host readback may sit between the decision and verification.
//
// One workgroup: the scan over n_bs requests is a blocked scan (each thread owns a contiguous
// run of requests), and the slot fill is request-parallel.  The step is latency-bound (a few
// microseconds), so one workgroup sized to the batch avoids any inter-block protocol.
#include "dsv_internal.h"

namespace dsv {

constexpr int kPackMaxThreads = 1024;

// Inclusive scan of v across the 64 lanes of a wavefront.
__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int64_t o = (int64_t)__shfl_up((long long)v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// One workgroup of NT threads (a multiple of 64, at most 1024).  Thread t owns the contiguous
// run of requests [t * per, (t + 1) * per); the per-thread sums are scanned with wavefront
// scans and one cross-wave pass, so the scan costs two barriers.
__global__ __launch_bounds__(kPackMaxThreads) void pack_slots_kernel(
    int n_bs, int W, int m_bs, const int32_t *__restrict__ k, const int32_t *__restrict__ ctx_len,
    const int64_t *__restrict__ kv_base, const int32_t *__restrict__ block_tokens,
    int32_t *__restrict__ offsets, int32_t *__restrict__ slot_req, int32_t *__restrict__ slot_tok,
    int32_t *__restrict__ slot_pos, int64_t *__restrict__ slot_cache_loc, int32_t *status) {
  __shared__ int64_t wave_sum[kPackMaxThreads / kWave];
  const int t = threadIdx.x, nt = blockDim.x, lane = t & (kWave - 1), wv = t / kWave;
  const int per = (n_bs + nt - 1) / nt;
  const int lo = min(n_bs, t * per), hi = min(n_bs, lo + per);

  // Effective length of request i: k_i if the request is well formed, else 0.
  auto eff = [&](int i) -> int {
    int ki = k[i];
    bool ok = ki >= 0 && ki <= W && ctx_len[i] >= 0 && kv_base[i] >= 0;
    return ok ? ki : 0;
  };

  int64_t local = 0;
  bool bad = false;
  for (int i = lo; i < hi; ++i) {
    int ki = k[i];
    bool ok = ki >= 0 && ki <= W && ctx_len[i] >= 0 && kv_base[i] >= 0;
    bad |= !ok;
    local += ok ? ki : 0;
  }
  if (bad) status_or(status, DSV_STATUS_BAD_REQUEST);
  const int64_t incl = wave_inclusive_scan(local, lane);
  if (lane == kWave - 1) wave_sum[wv] = incl;
  __syncthreads();
  int64_t before = 0, total = 0;
  for (int w = 0; w < nt / kWave; ++w) {
    before += w < wv ? wave_sum[w] : 0;
    total += wave_sum[w];
  }
  const bool drop_all = total > (int64_t)m_bs;
  if (t == 0 && drop_all) status_or(status, DSV_STATUS_BUDGET);
  int64_t run = drop_all ? 0 : before + incl - local;  // exclusive prefix of this thread's run
  for (int i = lo; i < hi; ++i) {
    offsets[i] = (int32_t)run;
    int ki = drop_all ? 0 : eff(i);
    int base = (int)run;
    int c = ctx_len[i];
    int64_t kb = kv_base[i];
    for (int j = 0; j < ki; ++j) {
      int s = base + j;
      slot_req[s] = i;
      slot_tok[s] = block_tokens[(int64_t)i * W + j];
      slot_pos[s] = c + j;
      slot_cache_loc[s] = kb + c + j;
    }
    run += ki;
  }
  const int end = drop_all ? 0 : (int)total;
  if (t == 0) offsets[n_bs] = end;
  for (int s = end + t; s < m_bs; s += nt) {
    slot_req[s] = -1;
    slot_tok[s] = 0;
    slot_pos[s] = 0;
    slot_cache_loc[s] = -1;
  }
}

}  // namespace dsv

extern "C" dsv_status dsv_pack_slots(int32_t n_bs, int32_t W, int32_t m_bs, const int32_t *k,
                                     const int32_t *ctx_len, const int64_t *kv_base,
                                     const int32_t *block_tokens, int32_t *offsets,
                                     int32_t *slot_req, int32_t *slot_tok, int32_t *slot_pos,
                                     int64_t *slot_cache_loc, int32_t *status,
                                     hipStream_t stream) {
  if (n_bs < 0 || n_bs > (1 << 20) || W < 1 || W > DSV_MAX_W || m_bs < 0) return DSV_ERR_INVALID_ARG;
  if (!offsets || !status) return DSV_ERR_INVALID_ARG;
  if (n_bs > 0 && (!k || !ctx_len || !kv_base || !block_tokens)) return DSV_ERR_INVALID_ARG;
  if (m_bs > 0 && (!slot_req || !slot_tok || !slot_pos || !slot_cache_loc)) return DSV_ERR_INVALID_ARG;
  // enough threads for one request each (or for the tail fill), up to one 1024-thread block
  int64_t want = n_bs > m_bs ? n_bs : m_bs;
  if (want < 64) want = 64;
  const int nt = (int)(want >= dsv::kPackMaxThreads ? dsv::kPackMaxThreads : (want + 63) / 64 * 64);
  hipLaunchKernelGGL(dsv::pack_slots_kernel, dim3(1), dim3(nt), 0, stream, n_bs, W,
                     m_bs, k, ctx_len, kv_base, block_tokens, offsets, slot_req, slot_tok, slot_pos,
                     slot_cache_loc, status);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
