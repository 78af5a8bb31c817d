// Sampling-mode prefix verifier and output builder.
//
// DScale (arXiv HTML), Sec. III-D "Prefix verifier": with the target's next-token
// distribution P at each row, a deterministic top-1 draft x is accepted with probability
// P(x); at the first rejection the successor comes from P with x taken out and the rest
// renormalised, and when every candidate passes it comes from the unmodified P.  After a_i
// accepted candidates, row offset_i + a_i supplies the successor; the output is the accepted
// candidates followed by it.  P is the softmax of the logits divided by the temperature T.
// The uniforms come from the caller: u_accept[s] decides the candidate that row s tests (the
// one at slot s + 1), u_draw[i] drives the inverse-CDF draw of request i's successor.
//
// Three kernels:
//  1. softmax_stats_kernel -- the HBM-bound sweep: one workgroup per (row, chunk) streams the
//     chunk (eight 16-byte non-temporal loads in flight per thread, the next block's loads
//     issued before the current block is reduced) and reduces it to (max logit m, sum of
//     2^((l - m) log2(e) / T)) in fp32.
//  2. sample_draw_kernel -- one workgroup per (request, chunk of the vocabulary).  Its first
//     wavefront merges the statistics of the request's rows (lane j: row offset + j), forms
//     P(x) for each tested candidate and takes the accept decisions, which gives a_i, the
//     successor row and the token to exclude.  The workgroup then sums, in fp64, the
//     successor row's weights exp((l - m) / T) over its chunk (x excluded).  Every workgroup
//     of a request takes the same decisions from the same data; the first one publishes them.
//  3. sample_finalize_kernel -- one workgroup per request: an fp64 scan of the chunk sums
//     locates the chunk holding u_draw * S, a scan of that chunk's weights (recomputed with
//     the same expression) finds the token, and the output row is written.
// Only the successor rows are read a second time (one row per request), so the extra
// traffic over the sweep is n_bs rows.
#include "dsv_internal.h"

namespace dsv {

constexpr int kSmpThreads = 256;
constexpr int kSmpLoads = 8;                              // 16-byte loads in flight per thread
constexpr int kSmpBlock = kSmpThreads * 4 * kSmpLoads;    // floats per 32 KB block
constexpr int kDrawMaxChunks = kSmpThreads;               // chunk sums scanned one per thread
constexpr int kDrawMaxChunk = 4096;                       // elements per draw chunk, at most

struct SoftStat {
  float m;  // largest logit of the chunk (-inf if none is finite)
  float s;  // sum of 2^((l - m) * c), c = log2(e) / T; NaN marks a NaN or +inf logit
};

// Request state published by the draw kernel: kind 0 inactive, 1 ok, 2 NaN/+inf or no finite
// entry in one of its rows, 3 malformed; a accepted drafts; ex the excluded token (or -1);
// m_bits the successor row's maximum.
struct SampleState {
  int32_t kind, a, ex;
  uint32_t m_bits;
};

// Merge (m2, s2) into (m, s); s is relative to m.
__device__ __forceinline__ void stat_merge(float &m, float &s, float m2, float s2, float c) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) {
    s = s + s2;
    return;
  }
  s = s * __builtin_amdgcn_exp2f((m - mn) * c) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * c);
  m = mn;
}

__global__ __launch_bounds__(kSmpThreads) void softmax_stats_kernel(
    const float *__restrict__ logits, int64_t vocab, int chunk, int n_chunks, int m_bs,
    const int32_t *__restrict__ offsets, int n_bs, float c, bool vec4,
    SoftStat *__restrict__ stats) {
  const int64_t bid = blockIdx.x;
  const int row = (int)(bid / n_chunks), ch = (int)(bid % n_chunks);
  int end = offsets[n_bs];
  end = end < 0 ? 0 : (end > m_bs ? m_bs : end);
  if (row >= end) return;
  const int64_t lo = (int64_t)ch * chunk;
  const int64_t hi = min(vocab, lo + chunk);
  const float *x = logits + (int64_t)row * vocab;
  const int t = threadIdx.x;
  float m = -INFINITY, s = 0.f;
  bool bad = false;
  if (vec4) {
    constexpr int64_t kStep = 4 * kSmpThreads;
    auto load = [&](f32x4 (&f)[kSmpLoads], int64_t v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kSmpLoads; ++u) {
        const int64_t v = v0 + u * kStep;
        f[u] = v < hi ? gload_stream<f32x4>(x + v) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    };
    // one rescale per block of 32 values: the block maximum first, then the exponentials
    auto reduce = [&](const f32x4 (&f)[kSmpLoads]) __attribute__((always_inline)) {
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < kSmpLoads; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e = f[u][q];
          bad |= !(e < INFINITY) && e != -INFINITY;  // NaN or +inf
          bm = fmaxf(bm, e);
        }
      if (bm > m) {
        s *= __builtin_amdgcn_exp2f((m - bm) * c);
        m = bm;
      }
      if (m != -INFINITY) {
#pragma unroll
        for (int u = 0; u < kSmpLoads; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) s += __builtin_amdgcn_exp2f((f[u][q] - m) * c);
      }
    };
    f32x4 fa[kSmpLoads], fb[kSmpLoads];
    int64_t v0 = lo + 4 * t;
    if (v0 < hi) load(fa, v0);
    for (; v0 < hi; v0 += 2 * kSmpBlock) {
      if (v0 + kSmpBlock < hi) load(fb, v0 + kSmpBlock);
      reduce(fa);
      if (v0 + kSmpBlock >= hi) break;
      if (v0 + 2 * kSmpBlock < hi) load(fa, v0 + 2 * kSmpBlock);
      reduce(fb);
    }
  } else {
    for (int64_t v = lo + t; v < hi; v += kSmpThreads) {
      const float e = x[v];
      bad |= !(e < INFINITY) && e != -INFINITY;
      if (e > m) {
        s *= __builtin_amdgcn_exp2f((m - e) * c);
        m = e;
      }
      if (m != -INFINITY) s += __builtin_amdgcn_exp2f((e - m) * c);
    }
  }
  if (bad) s = __uint_as_float(0x7fc00000u);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float m2 = __shfl_xor(m, d), s2 = __shfl_xor(s, d);
    stat_merge(m, s, m2, s2, c);
  }
  __shared__ float red_m[kSmpThreads / kWave], red_s[kSmpThreads / kWave];
  if ((t & (kWave - 1)) == 0) {
    red_m[t / kWave] = m;
    red_s[t / kWave] = s;
  }
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < kSmpThreads / kWave; ++w) stat_merge(m, s, red_m[w], red_s[w], c);
    stats[(int64_t)row * n_chunks + ch] = SoftStat{m, s};
  }
}

// Weight of token v in the successor draw: exp((l - m) / T) in fp64, 0 for the excluded
// token.  The draw and finalize kernels evaluate the same expression, so their sums agree up
// to summation order.
__device__ __forceinline__ double draw_weight(float l, double m, double T, int64_t v, int32_t ex) {
  return v == ex ? 0.0 : exp(((double)l - m) / T);
}

__device__ __forceinline__ double block_sum_f64(double v, double *lds) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int q = 0; q < kSmpThreads / kWave; ++q) r += lds[q];
  return r;
}

// Inclusive scan over the workgroup in thread order.
__device__ __forceinline__ double block_incl_scan_f64(double v, double *lds) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  __syncthreads();
  if (lane == kWave - 1) lds[w] = v;
  __syncthreads();
  double add = 0.0;
  for (int q = 0; q < w; ++q) add += lds[q];
  return v + add;
}

__device__ __forceinline__ int block_min_i32(int v, int *lds) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  int r = lds[0];
  for (int q = 1; q < kSmpThreads / kWave; ++q) r = min(r, lds[q]);
  return r;
}

__device__ __forceinline__ int block_count(bool pred, int *lds) {
  const int n = __popcll(__ballot(pred));
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = n;
  __syncthreads();
  int r = 0;
  for (int q = 0; q < kSmpThreads / kWave; ++q) r += lds[q];
  return r;
}

__device__ __forceinline__ int block_max_i32(int v, int *lds) {
  return -block_min_i32(-v, lds);
}

__global__ __launch_bounds__(kSmpThreads) void sample_draw_kernel(
    int n_bs, int m_bs, int W, int64_t vocab, const float *__restrict__ logits, float c,
    double T, const int32_t *__restrict__ slot_tok, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ k, const float *__restrict__ u_accept,
    const SoftStat *__restrict__ stats, int nc1, int chunk2, int nc2,
    double *__restrict__ wsum, SampleState *__restrict__ state, float *__restrict__ p_cand) {
  const int64_t bid = blockIdx.x;
  const int i = (int)(bid / nc2), ch = (int)(bid % nc2);
  const int t = threadIdx.x;
  __shared__ SampleState st;
  __shared__ double red[kSmpThreads / kWave];
  if (t < kWave) {
    const int lane = t;
    int end = offsets[n_bs];
    end = end < 0 ? 0 : (end > m_bs ? m_bs : end);
    const int ki = k[i], off = offsets[i];
    const bool ok = ki >= 0 && ki <= W && off >= 0 && (int64_t)off + ki <= end;
    SampleState r{ok ? (ki == 0 ? 0 : 1) : 3, 0, -1, 0u};
    if (ok && ki > 0) {
      // lane j tests the candidate of row off + j: its loads go out first
      const int j = lane;
      const int64_t row = (int64_t)off + j;
      const bool tests = j + 1 < ki;
      const int32_t x = tests ? slot_tok[row + 1] : -1;
      const bool in_vocab = x >= 0 && x < vocab;
      const float lx = tests && in_vocab ? logits[row * vocab + x] : 0.f;
      const float ua = tests ? u_accept[row] : 0.f;
      // four lanes per row merge its chunk statistics: lane 4r + q takes chunks q, q + 4, ...,
      // with the loads of up to four chunks in flight before any merge
      const int jr = lane >> 2, q0 = lane & 3;
      float M = -INFINITY, S = 0.f;
      if (jr < ki) {
        const int64_t rrow = (int64_t)off + jr;
        for (int base = q0; base < nc1; base += 16) {
          SoftStat z[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int q = base + 4 * u;
            z[u] = q < nc1 ? stats[rrow * nc1 + q] : SoftStat{-INFINITY, 0.f};
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) stat_merge(M, S, z[u].m, z[u].s, c);
        }
      }
#pragma unroll
      for (int d = 1; d <= 2; d <<= 1) {
        const float m2 = __shfl_xor(M, d), s2 = __shfl_xor(S, d);
        stat_merge(M, S, m2, s2, c);
      }
      M = __shfl(M, 4 * (j & 15));
      S = __shfl(S, 4 * (j & 15));
      const bool row_bad = j < ki && (S != S || M == -INFINITY);
      float P = -1.f;
      if (tests) P = in_vocab ? __builtin_amdgcn_exp2f((lx - M) * c) / S : 0.f;
      const bool rej = tests && !(ua < P);
      const uint64_t badm = __ballot(row_bad), rejm = __ballot(rej);
      const int a = rejm ? __ffsll((long long)rejm) - 1 : ki - 1;
      const int32_t xa = __shfl(x, a);
      const float Ma = __shfl(M, a);
      if (ch == 0 && p_cand && j < ki) p_cand[row] = P;
      r.kind = badm ? 2 : 1;
      r.a = a;
      r.ex = (rejm && xa >= 0 && xa < vocab) ? xa : -1;
      r.m_bits = __float_as_uint(Ma);
    }
    if (lane == 0) {
      st = r;
      if (ch == 0) state[i] = r;
    }
  }
  __syncthreads();
  if (st.kind != 1) return;
  const int64_t row = (int64_t)offsets[i] + st.a;
  const float *x = logits + row * vocab;
  const double M = (double)__uint_as_float(st.m_bits);
  const int64_t lo = (int64_t)ch * chunk2, hi = min(vocab, lo + chunk2);
  double acc = 0.0;
  for (int64_t v = lo + t; v < hi; v += kSmpThreads) acc += draw_weight(x[v], M, T, v, st.ex);
  acc = block_sum_f64(acc, red);
  if (t == 0) wsum[(int64_t)i * nc2 + ch] = acc;
}

__global__ __launch_bounds__(kSmpThreads) void sample_finalize_kernel(
    int W, int64_t vocab, const float *__restrict__ logits, double T,
    const int32_t *__restrict__ slot_tok, const int32_t *__restrict__ offsets,
    const float *__restrict__ u_draw, int chunk2, int nc2, const double *__restrict__ wsum,
    const SampleState *__restrict__ state, int32_t *__restrict__ accepted,
    int32_t *__restrict__ bonus, int32_t *__restrict__ progress,
    int32_t *__restrict__ out_tokens, int32_t *status) {
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  // every load that does not depend on the request's state goes out with it
  const SampleState st = state[i];
  const double w = t < nc2 ? wsum[(int64_t)i * nc2 + t] : 0.0;
  const int off = offsets[i];
  const float ud = u_draw[i];
  if (st.kind != 1) {
    if (t == 0) {
      if (st.kind == 2) status_or(status, DSV_STATUS_NAN);
      if (st.kind == 3) status_or(status, DSV_STATUS_BAD_REQUEST);
      accepted[i] = st.kind == 0 ? 0 : -1;
      bonus[i] = -1;
      progress[i] = 0;
    }
    if (out_tokens && t < W) out_tokens[(int64_t)i * W + t] = -1;
    return;
  }
  __shared__ double red[kSmpThreads / kWave];
  __shared__ int redi[kSmpThreads / kWave];
  __shared__ double sh_incl[kDrawMaxChunks], sh_w[kDrawMaxChunks];
  // locate the chunk: the first c whose inclusive prefix exceeds u * S
  const double incl = block_incl_scan_f64(w, red);
  sh_incl[t] = incl;
  sh_w[t] = w;
  __syncthreads();
  const double S = sh_incl[nc2 - 1];
  const double target = (double)ud * S;
  // the number of chunks whose inclusive prefix is <= target (prefixes are nondecreasing)
  int cstar = block_count(t < nc2 && incl <= target, redi);
  if (cstar >= nc2) cstar = block_max_i32(t < nc2 && w > 0.0 ? t : -1, redi);
  const int64_t row = (int64_t)off + st.a;
  int32_t y = -1;
  if (cstar >= 0) {
    // thread t owns a contiguous run of the chunk; the weights of its first kPer elements stay
    // in registers between the sum and the search
    constexpr int kPer = kDrawMaxChunk / kSmpThreads;
    const double tl = target - (sh_incl[cstar] - sh_w[cstar]);
    const float *x = logits + row * vocab;
    const double M = (double)__uint_as_float(st.m_bits);
    const int64_t lo = (int64_t)cstar * chunk2, hi = min(vocab, lo + chunk2);
    const int64_t per = (hi - lo + kSmpThreads - 1) / kSmpThreads;
    const int64_t a0 = min(hi, lo + t * per), a1 = min(hi, a0 + per);
    float lv[kPer];
    double wr[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) lv[u] = a0 + u < a1 ? x[a0 + u] : 0.f;
    double part = 0.0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      wr[u] = a0 + u < a1 ? draw_weight(lv[u], M, T, a0 + u, st.ex) : 0.0;
      part += wr[u];
    }
    for (int64_t v = a0 + kPer; v < a1; ++v) part += draw_weight(x[v], M, T, v, st.ex);
    const double excl = block_incl_scan_f64(part, red) - part;
    int found = INT32_MAX, last = -1;
    double cum = excl;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (wr[u] > 0.0) {
        last = (int)(a0 + u);
        cum += wr[u];
        if (found == INT32_MAX && tl < cum) found = (int)(a0 + u);
      }
    }
    for (int64_t v = a0 + kPer; v < a1; ++v) {
      const double wv = draw_weight(x[v], M, T, v, st.ex);
      if (wv > 0.0) {
        last = (int)v;
        cum += wv;
        if (found == INT32_MAX && tl < cum) found = (int)v;
      }
    }
    const int f = block_min_i32(found, redi);
    y = f != INT32_MAX ? f : block_max_i32(last, redi);
  }
  const int a = st.a;
  if (t == 0) {
    accepted[i] = a;
    bonus[i] = y;
    progress[i] = 1 + a;
  }
  if (out_tokens && t < W)
    out_tokens[(int64_t)i * W + t] = t < a ? slot_tok[off + 1 + t] : (t == a ? y : -1);
}

// Sweep chunking: about 2048 workgroups, chunks of whole 1024-element groups (four per lane).
static void plan_stats(int64_t rows, int64_t vocab, int *n_chunks, int *chunk) {
  int64_t want = rows > 0 ? (2048 + rows - 1) / rows : 1;
  int64_t cap = (vocab + kSmpBlock - 1) / kSmpBlock;
  if (cap < 1) cap = 1;
  int64_t n = want < 1 ? 1 : (want > cap ? cap : want);
  int64_t c = (vocab + n - 1) / n;
  c = (c + 1023) / 1024 * 1024;
  n = (vocab + c - 1) / c;
  *n_chunks = (int)(n < 1 ? 1 : n);
  *chunk = (int)c;
}

// Draw chunking: about 1024 workgroups over the requests, at most kDrawMaxChunk elements per
// chunk (the finalize kernel scans one chunk) and at most kDrawMaxChunks chunks per row.
static void plan_draw(int64_t n_bs, int64_t vocab, int *n_chunks, int *chunk) {
  int64_t n = n_bs > 0 ? (1024 + n_bs - 1) / n_bs : 1;
  const int64_t need = (vocab + kDrawMaxChunk - 1) / kDrawMaxChunk;
  n = n < need ? need : n;
  const int64_t cap = (vocab + 255) / 256;
  n = n > cap ? cap : n;
  n = n > kDrawMaxChunks ? kDrawMaxChunks : (n < 1 ? 1 : n);
  int64_t c = (vocab + n - 1) / n;
  c = (c + 255) / 256 * 256;
  n = (vocab + c - 1) / c;
  *n_chunks = (int)(n < 1 ? 1 : n);
  *chunk = (int)c;
}

static size_t align256s(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace dsv

extern "C" size_t dsv_accept_sample_workspace_bytes(int32_t n_bs, int32_t m_bs, int32_t vocab) {
  if (n_bs <= 0 || m_bs <= 0 || vocab <= 0) return 0;
  int nc1, ch1, nc2, ch2;
  dsv::plan_stats(m_bs, vocab, &nc1, &ch1);
  dsv::plan_draw(n_bs, vocab, &nc2, &ch2);
  return dsv::align256s((size_t)m_bs * nc1 * sizeof(dsv::SoftStat)) +
         dsv::align256s((size_t)n_bs * sizeof(dsv::SampleState)) +
         dsv::align256s((size_t)n_bs * nc2 * sizeof(double));
}

extern "C" dsv_status dsv_accept_sample(int32_t n_bs, int32_t m_bs, int32_t W, int32_t vocab,
                                        const float *target_logits, float temperature,
                                        const int32_t *slot_tok, const int32_t *offsets,
                                        const int32_t *k, const float *u_accept,
                                        const float *u_draw, int32_t *accepted, int32_t *bonus,
                                        int32_t *progress, int32_t *out_tokens, float *p_cand,
                                        void *workspace, size_t workspace_bytes,
                                        int32_t *status, hipStream_t stream) {
  using namespace dsv;
  if (n_bs < 0 || m_bs < 0 || W < 1 || W > DSV_MAX_W || vocab < 1 || !status)
    return DSV_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return DSV_ERR_INVALID_ARG;
  if (!target_logits || !slot_tok || !offsets || !k || !u_accept || !u_draw || !accepted ||
      !bonus || !progress)
    return DSV_ERR_INVALID_ARG;
  if (n_bs == 0) return DSV_OK;
  const size_t need = dsv_accept_sample_workspace_bytes(n_bs, m_bs > 0 ? m_bs : 1, vocab);
  if (!workspace || workspace_bytes < need) return DSV_ERR_WORKSPACE;
  {
    const Span out[] = {{accepted, span_bytes(n_bs, 4)},  {bonus, span_bytes(n_bs, 4)},
                        {progress, span_bytes(n_bs, 4)},  {out_tokens, span_bytes((int64_t)n_bs * W, 4)},
                        {p_cand, span_bytes(m_bs, 4)},    {workspace, need},
                        {status, 4}};
    const Span in[] = {{target_logits, span_bytes((int64_t)m_bs * vocab, 4)},
                       {slot_tok, span_bytes(m_bs, 4)}, {offsets, span_bytes(n_bs + 1, 4)},
                       {k, span_bytes(n_bs, 4)},        {u_accept, span_bytes(m_bs, 4)},
                       {u_draw, span_bytes(n_bs, 4)}};
    if (outputs_alias(out, in)) return DSV_ERR_INVALID_ARG;
  }
  int nc1, ch1, nc2, ch2;
  plan_stats(m_bs > 0 ? m_bs : 1, vocab, &nc1, &ch1);
  plan_draw(n_bs, vocab, &nc2, &ch2);
  if (!launch_fits((int64_t)(m_bs > 0 ? m_bs : 1) * nc1, kSmpThreads) ||
      !launch_fits((int64_t)n_bs * nc2, kSmpThreads))
    return DSV_ERR_INVALID_ARG;
  char *ws = static_cast<char *>(workspace);
  SoftStat *stats = reinterpret_cast<SoftStat *>(ws);
  ws += align256s((size_t)(m_bs > 0 ? m_bs : 1) * nc1 * sizeof(SoftStat));
  SampleState *state = reinterpret_cast<SampleState *>(ws);
  ws += align256s((size_t)n_bs * sizeof(SampleState));
  double *wsum = reinterpret_cast<double *>(ws);
  // 2^((l - m) * c) = e^((l - m) / T)
  const float c = (float)(1.4426950408889634 / (double)temperature);
  if (m_bs > 0) {
    const bool vec = (vocab % 4 == 0) && ((uintptr_t)target_logits % 16 == 0);
    hipLaunchKernelGGL(softmax_stats_kernel, dim3((unsigned)((int64_t)m_bs * nc1)),
                       dim3(kSmpThreads), 0, stream, target_logits, (int64_t)vocab, ch1, nc1,
                       m_bs, offsets, n_bs, c, vec, stats);
    DSV_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(sample_draw_kernel, dim3((unsigned)((int64_t)n_bs * nc2)), dim3(kSmpThreads),
                     0, stream, n_bs, m_bs, W, (int64_t)vocab, target_logits, c,
                     (double)temperature, slot_tok, offsets, k, u_accept, stats, nc1, ch2, nc2,
                     wsum, state, p_cand);
  DSV_LAUNCH_CHECK();
  hipLaunchKernelGGL(sample_finalize_kernel, dim3((unsigned)n_bs), dim3(kSmpThreads), 0, stream, W,
                     (int64_t)vocab, target_logits, (double)temperature, slot_tok, offsets, u_draw,
                     ch2, nc2, wsum, state, accepted, bonus, progress, out_tokens, status);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
