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

  auto eff = [&](int i) -> int { return pack_effective_length(k[i], ctx_len[i], kv_base[i], W); };

  int64_t local = 0;
  bool bad = false;
  for (int i = lo; i < hi; ++i) {
    bad |= !pack_request_ok(k[i], ctx_len[i], kv_base[i], W);
    local += eff(i);
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
    write_request_slots(i, ki, base, W, ctx_len[i], kv_base[i], block_tokens, slot_req, slot_tok,
                        slot_pos, slot_cache_loc);
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

// ---------------------------------------------------------------------------
// Budget allocator fused with the packer (DScale Sec. III-C, "Acceptance predictor" from
// the sigmoid scores on, "Budget allocator", Fig. 6).  One workgroup, one thread per
// request (n_bs <= 1024), no host round trip.
//
// The pages adjust the seeded lengths one slot at a time: grow the request whose next slot
// has the highest score, or shrink the one whose last slot has the lowest score, until the
// live budget is met.  Because every request's prefix scores are nonincreasing, the |delta|
// slots that loop moves are exactly the |delta| largest candidates under the order (score
// desc, request asc, slot asc) when growing -- candidates are the slots j in [k0_i, W) -- or
// the smallest under (score asc, request asc, slot desc) when shrinking (slots j in
// [1, k0_i)).  The kernel selects them directly: a 32-step bisection on the order-preserving
// score bits finds the score of the last moved slot, every slot beyond it moves, and the
// slots equal to it move in request order (an exclusive scan).  Same result as the loop;
// 32 block-wide counts instead of up to 7N sequential arg-max steps.
// ---------------------------------------------------------------------------
constexpr int kAllocMaxRequests = 1024;

// Sum over the workgroup of small per-thread counts 0 <= v < 32: within a wavefront from
// five ballots (bit b of every lane's count, population-counted), no cross-lane data
// movement; across wavefronts through LDS (a one-wavefront workgroup needs no barrier).
__device__ __forceinline__ int block_sum_small(int v, int *red, int lane, int wv, int nwv) {
  int t = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) t += __popcll(__ballot((v >> b) & 1)) << b;
  if (nwv == 1) return t;
  __syncthreads();  // previous readers of red[] are done
  if (lane == 0) red[wv] = t;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < nwv; ++w) s += red[w];
  return s;
}

// Exclusive scan of small counts 0 <= v < 32 over the workgroup's threads in order (ballots
// masked to the lower lanes within a wavefront, LDS across wavefronts); *total receives the
// sum.
__device__ __forceinline__ int block_exclusive_scan_small(int v, int *red, int lane, int wv, int nwv,
                                                          int *total) {
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int pre = 0, t = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    pre += __popcll(m & below) << b;
    t += __popcll(m) << b;
  }
  if (nwv == 1) {
    *total = t;
    return pre;
  }
  __syncthreads();
  if (lane == 0) red[wv] = t;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nwv; ++w) {
    before += w < wv ? red[w] : 0;
    all += red[w];
  }
  *total = all;
  return before + pre;
}

__global__ __launch_bounds__(kAllocMaxRequests) void allocate_pack_kernel(
    int n_live, int n_bs, int W, int m_live, int m_bs, const float *__restrict__ score,
    const int32_t *__restrict__ ctx_len, const int64_t *__restrict__ kv_base,
    const int32_t *__restrict__ block_tokens, int32_t *__restrict__ k_out, int32_t *__restrict__ k0_out,
    int32_t *__restrict__ offsets, int32_t *__restrict__ slot_req, int32_t *__restrict__ slot_tok,
    int32_t *__restrict__ slot_pos, int64_t *__restrict__ slot_cache_loc, int32_t *status) {
  __shared__ int red[kAllocMaxRequests / kWave];
  const int i = threadIdx.x, lane = i & (kWave - 1), wv = i / kWave, nwv = blockDim.x / kWave;
  const bool live = i < n_live;

  // prefix scores (q[0] = 1 for the anchor, cumulative minimum after) and the rounded seed
  uint32_t u[DSV_MAX_W];  // order-preserving bits of q[j]
  int k0 = 0;
  if (live) {
    float prev = 1.0f, l = 0.0f;
    bool nan = false;
    u[0] = ordered_bits(1.0f);
#pragma unroll
    for (int j = 1; j < DSV_MAX_W; ++j) {
      if (j < W) {
        float x = score[(int64_t)i * (W - 1) + (j - 1)];
        nan |= x != x;
        x = x != x ? 0.0f : x;
        prev = x < prev ? x : prev;
        l = l + prev;
        u[j] = ordered_bits(prev);
      }
    }
    if (nan) status_or(status, DSV_STATUS_NAN);
    const float r = rintf(l);
    k0 = r < 1.0f ? 1 : (r > (float)W ? W : (int)r);
  }
  const int total0 = block_sum_small(k0, red, lane, wv, nwv);
  const int delta = m_live - total0;  // uniform
  int k = k0;
  if (delta != 0 && n_live > 0) {
    const bool grow = delta > 0;
    // candidate j of this request: growing j in [k0, W) with key u[j]; shrinking j in
    // [1, k0) with key ~u[j] (larger key = moved earlier)
    const int jlo = grow ? k0 : 1, jhi = grow ? W : k0;
    auto key = [&](int j) __attribute__((always_inline)) { return grow ? u[j] : ~u[j]; };
    auto count_ge = [&](uint32_t t) __attribute__((always_inline)) {
      int c = 0;
      if (live) {
#pragma unroll
        for (int j = 0; j < DSV_MAX_W; ++j) c += (j >= jlo && j < jhi && key(j) >= t) ? 1 : 0;
      }
      return c;
    };
    int want = grow ? delta : -delta;
    const int avail = block_sum_small(live ? (jhi > jlo ? jhi - jlo : 0) : 0, red, lane, wv, nwv);
    want = want < avail ? want : avail;  // if nobody can move further, move everything
    int moved = 0;
    if (want > 0) {
      // largest threshold T with count(key >= T) >= want
      uint32_t T = 0;
      for (int b = 31; b >= 0; --b) {
        const uint32_t t = T | (1u << b);
        if (block_sum_small(count_ge(t), red, lane, wv, nwv) >= want) T = t;
      }
      int gt = 0, eq = 0;
      if (live) {
#pragma unroll
        for (int j = 0; j < DSV_MAX_W; ++j) {
          const bool in = j >= jlo && j < jhi;
          gt += (in && key(j) > T) ? 1 : 0;
          eq += (in && key(j) == T) ? 1 : 0;
        }
      }
      const int n_gt = block_sum_small(gt, red, lane, wv, nwv);
      int eq_total;
      const int eq_before = block_exclusive_scan_small(eq, red, lane, wv, nwv, &eq_total);
      int take = want - n_gt - eq_before;
      take = take < 0 ? 0 : (take > eq ? eq : take);
      moved = gt + take;
    }
    k = grow ? k0 + moved : k0 - moved;
  }

  // flat-buffer pack of the adjusted lengths
  int end;
  const int off = block_exclusive_scan_small(k, red, lane, wv, nwv, &end);
  if (end > m_bs) {  // cannot happen for m_live <= m_bs; kept as the packer's rule
    if (i == 0) status_or(status, DSV_STATUS_BUDGET);
  }
  const bool fits = end <= m_bs;
  if (i < n_bs) {
    k_out[i] = k;
    if (k0_out) k0_out[i] = k0;
    offsets[i] = fits ? off : 0;
    if (fits) {
      write_request_slots(i, k, off, W, ctx_len[i], kv_base[i], block_tokens, slot_req, slot_tok,
                          slot_pos, slot_cache_loc);
    }
  }
  const int tail = fits ? end : 0;
  if (i == 0) offsets[n_bs] = tail;
  for (int s = tail + i; s < m_bs; s += blockDim.x) {
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
  {
    using dsv::span_bytes;
    const dsv::Span out[] = {{offsets, span_bytes(n_bs + 1, 4)}, {slot_req, span_bytes(m_bs, 4)},
                             {slot_tok, span_bytes(m_bs, 4)},    {slot_pos, span_bytes(m_bs, 4)},
                             {slot_cache_loc, span_bytes(m_bs, 8)}, {status, 4}};
    const dsv::Span in[] = {{k, span_bytes(n_bs, 4)}, {ctx_len, span_bytes(n_bs, 4)},
                            {kv_base, span_bytes(n_bs, 8)},
                            {block_tokens, span_bytes((int64_t)n_bs * W, 4)}};
    if (dsv::outputs_alias(out, in)) return DSV_ERR_INVALID_ARG;
  }
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

extern "C" dsv_status dsv_allocate_pack(int32_t n_live, int32_t n_bs, int32_t W, int32_t m_live,
                                        int32_t m_bs, const float *scores, const int32_t *ctx_len,
                                        const int64_t *kv_base, const int32_t *block_tokens,
                                        int32_t *k, int32_t *k0, int32_t *offsets, int32_t *slot_req,
                                        int32_t *slot_tok, int32_t *slot_pos, int64_t *slot_cache_loc,
                                        int32_t *status, hipStream_t stream) {
  if (n_live < 0 || n_bs < n_live || n_bs > dsv::kAllocMaxRequests || W < 1 || W > DSV_MAX_W ||
      m_live < 0 || m_bs < m_live)
    return DSV_ERR_INVALID_ARG;
  if (!k || !offsets || !status) return DSV_ERR_INVALID_ARG;
  if (n_live > 0 && W > 1 && !scores) return DSV_ERR_INVALID_ARG;
  if (n_bs > 0 && (!ctx_len || !kv_base || !block_tokens)) return DSV_ERR_INVALID_ARG;
  if (m_bs > 0 && (!slot_req || !slot_tok || !slot_pos || !slot_cache_loc)) return DSV_ERR_INVALID_ARG;
  {
    using dsv::span_bytes;
    const dsv::Span out[] = {{k, span_bytes(n_bs, 4)},           {k0, span_bytes(n_bs, 4)},
                             {offsets, span_bytes(n_bs + 1, 4)}, {slot_req, span_bytes(m_bs, 4)},
                             {slot_tok, span_bytes(m_bs, 4)},    {slot_pos, span_bytes(m_bs, 4)},
                             {slot_cache_loc, span_bytes(m_bs, 8)}, {status, 4}};
    const dsv::Span in[] = {{scores, span_bytes((int64_t)n_live * (W - 1), 4)},
                            {ctx_len, span_bytes(n_bs, 4)}, {kv_base, span_bytes(n_bs, 8)},
                            {block_tokens, span_bytes((int64_t)n_bs * W, 4)}};
    if (dsv::outputs_alias(out, in)) return DSV_ERR_INVALID_ARG;
  }
  int want = n_bs > 64 ? n_bs : 64;
  const int nt = (want + 63) / 64 * 64;
  hipLaunchKernelGGL(dsv::allocate_pack_kernel, dim3(1), dim3(nt), 0, stream, n_live, n_bs, W, m_live,
                     m_bs, scores, ctx_len, kv_base, block_tokens, k, k0, offsets, slot_req, slot_tok,
                     slot_pos, slot_cache_loc, status);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
