// Greedy prefix verifier, output builder and draft top-1/top-2 margin.
//
// DScale (arXiv HTML), Sec. III-D "Prefix verifier": in greedy decoding a deterministic
// top-1 draft is accepted when the target picks it; after a_i accepted candidates, row
// offset_i + a_i supplies the successor, and the output is the accepted candidates followed
// by that successor.  Sec. II-B / Fig. 2: progress counts one anchor plus accepted drafts.
// Sec. II-B / Fig. 4 and DFlash-Mini-Lab (DFlash7-ACT): the gap between the top-1 and top-2
// draft logits is the acceptance signal.
//
// Both vocabulary sweeps are HBM-bound streams over fp32 logits.  Each row is cut into
// chunks so that the launch has about 2048 workgroups, each streaming one contiguous chunk
// in 32 KB blocks (eight 16-byte non-temporal loads in flight per thread, the next block's
// loads issued before the current block is reduced);
// a chunk reduces to one 64-bit key per row (argmax) or one (top-1 key, top-2 value) pair
// (margin), and a small per-request kernel merges the chunks in a fixed order, so results
// are deterministic.
//
// Argmax key: (order-preserving bits of the value) << 32 | ~index.  The largest key has the
// largest value and, among equal values, the lowest index; -0.0 is folded onto +0.0.  A NaN
// anywhere in a row makes the chunk report the all-ones key, which dominates the merge.
#include "dsv_internal.h"

namespace dsv {

constexpr int kAccThreads = 256;
constexpr int kAccLoads = 8;                            // 16-byte loads in flight per thread
constexpr int kAccBlock = kAccThreads * 4 * kAccLoads;  // floats per 32 KB block
constexpr uint64_t kNanKey = ~0ull;
// Workgroups a vocabulary sweep aims at (eight per CU over the launch).  Greedy accept on
// 128 x 151,936 logits: 512 -> 15.6 us for the sweep kernel, 1024 -> 20.6 us per call,
// 2048 -> 19.6-19.9 us per call, 4096 -> 19.9 us per call.
constexpr int64_t kSweepWgs = 2048;

struct Top2 {
  uint64_t k1;  // key of the largest element (value bits << 32 | ~index); 0 = none
  uint32_t v2;  // ordered bits of the second element of the descending multiset; 0 = none
  uint32_t nan;
};

__device__ __forceinline__ void top2_push(Top2 &t, float x, uint32_t idx) {
  if (x != x) {
    t.nan = 1;
    return;
  }
  uint32_t o = ordered_bits(x);
  uint64_t key = ((uint64_t)o << 32) | (uint32_t)~idx;
  if (key > t.k1) {
    uint32_t prev = (uint32_t)(t.k1 >> 32);
    t.v2 = prev > t.v2 ? prev : t.v2;
    t.k1 = key;
  } else {
    t.v2 = o > t.v2 ? o : t.v2;
  }
}

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  r.k1 = a.k1 > b.k1 ? a.k1 : b.k1;
  uint64_t lo = a.k1 > b.k1 ? b.k1 : a.k1;
  uint32_t v = a.v2 > b.v2 ? a.v2 : b.v2;
  uint32_t lo_v = (uint32_t)(lo >> 32);
  r.v2 = lo_v > v ? lo_v : v;
  r.nan = a.nan | b.nan;
  return r;
}

// One workgroup per (row, chunk) of a [rows][vocab] fp32 matrix.
template <bool kVec4>
__global__ __launch_bounds__(kAccThreads) void argmax_partial_kernel(
    const float *__restrict__ logits, int64_t vocab, int chunk, int n_chunks, int m_bs,
    const int32_t *__restrict__ offsets, int n_bs, uint64_t *__restrict__ keys, int32_t *status) {
  const int64_t bid = blockIdx.x;
  const int row = (int)(bid / n_chunks), c = (int)(bid % n_chunks);
  // rows at or past the end boundary have no choice to make; the boundary's load goes out
  // with the first block's loads (a row below m_bs is inside the matrix either way)
  int end = offsets[n_bs];
  const int64_t lo = (int64_t)c * chunk;
  const int64_t hi = min(vocab, lo + chunk);
  const float *x = logits + (int64_t)row * vocab;
  uint64_t best = 0;
  bool nan = false;
  const int t = threadIdx.x;
  if (kVec4) {
    // kAccLoads independent 16-byte loads in flight per thread; the next block's loads are
    // issued before the current block is reduced
    constexpr int64_t kStep = 4 * kAccThreads;
    auto load = [&](f32x4 (&f)[kAccLoads], int64_t v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kAccLoads; ++u) {
        const int64_t v = v0 + u * kStep;
        f[u] = v < hi ? gload_stream<f32x4>(x + v) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    };
    // A thread visits its elements in increasing index order, so a strict comparison keeps
    // the lowest index among equal values (and -0.0 == +0.0); the value/index pair becomes a
    // key only once, for the cross-thread merge.
    float bv = -INFINITY;
    int64_t bi = -1;
    auto reduce = [&](const f32x4 (&f)[kAccLoads], int64_t v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kAccLoads; ++u) {
        const int64_t v = v0 + u * kStep;
        if (v >= hi) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float e = f[u][q];
          nan |= e != e;
          const bool gt = e > bv || bi < 0;
          bv = gt ? e : bv;
          bi = gt ? v + q : bi;
        }
      }
    };
    f32x4 fa[kAccLoads], fb[kAccLoads];
    int64_t v0 = lo + 4 * t;
    if (v0 < hi) load(fa, v0);
    end = end < 0 ? 0 : (end > m_bs ? m_bs : end);
    if (row >= end) return;
    for (; v0 < hi; v0 += 2 * kAccBlock) {
      if (v0 + kAccBlock < hi) load(fb, v0 + kAccBlock);
      reduce(fa, v0);
      if (v0 + kAccBlock >= hi) break;
      if (v0 + 2 * kAccBlock < hi) load(fa, v0 + 2 * kAccBlock);
      reduce(fb, v0 + kAccBlock);
    }
    if (bi >= 0) best = ((uint64_t)ordered_bits(bv) << 32) | (uint32_t)~(uint32_t)bi;
  } else {
    end = end < 0 ? 0 : (end > m_bs ? m_bs : end);
    if (row >= end) return;
    for (int64_t v = lo + t; v < hi; v += kAccThreads) {
      float e = x[v];
      nan |= e != e;
      uint64_t key = ((uint64_t)ordered_bits(e) << 32) | (uint32_t)~(uint32_t)v;
      best = key > best ? key : best;
    }
  }
  if (nan) best = kNanKey;
  best = wave_max_u64(best);
  __shared__ uint64_t red[kAccThreads / kWave];
  if ((t & (kWave - 1)) == 0) red[t / kWave] = best;
  __syncthreads();
  if (t == 0) {
    uint64_t r = red[0];
    for (int w = 1; w < kAccThreads / kWave; ++w) r = red[w] > r ? red[w] : r;
    keys[(int64_t)row * n_chunks + c] = r;
    if (r == kNanKey) status_or(status, DSV_STATUS_NAN);
  }
}

template <bool kVec4>
__global__ __launch_bounds__(kAccThreads) void top2_partial_kernel(
    const float *__restrict__ logits, int64_t vocab, int chunk, int n_chunks,
    Top2 *__restrict__ part, int32_t *status) {
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / n_chunks;
  const int c = (int)(bid % n_chunks);
  const int64_t lo = (int64_t)c * chunk;
  const int64_t hi = min(vocab, lo + chunk);
  const float *x = logits + row * vocab;
  Top2 acc{0ull, 0u, 0u};
  const int t = threadIdx.x;
  if (kVec4) {
    constexpr int64_t kStep = 4 * kAccThreads;
    for (int64_t v0 = lo + 4 * t; v0 < hi; v0 += kAccBlock) {
      f32x4 f[kAccLoads];
#pragma unroll
      for (int u = 0; u < kAccLoads; ++u) {
        const int64_t v = v0 + u * kStep;
        f[u] = v < hi ? gload_stream<f32x4>(x + v) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kAccLoads; ++u) {
        const int64_t v = v0 + u * kStep;
        if (v >= hi) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) top2_push(acc, f[u][q], (uint32_t)(v + q));
      }
    }
  } else {
    for (int64_t v = lo + t; v < hi; v += kAccThreads) top2_push(acc, x[v], (uint32_t)v);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    Top2 o;
    o.k1 = shfl_xor_u64(acc.k1, m);
    o.v2 = (uint32_t)__shfl_xor((int)acc.v2, m);
    o.nan = (uint32_t)__shfl_xor((int)acc.nan, m);
    acc = top2_merge(acc, o);
  }
  __shared__ Top2 red[kAccThreads / kWave];
  if ((t & (kWave - 1)) == 0) red[t / kWave] = acc;
  __syncthreads();
  if (t == 0) {
    Top2 r = red[0];
    for (int w = 1; w < kAccThreads / kWave; ++w) r = top2_merge(r, red[w]);
    part[row * n_chunks + c] = r;
    if (r.nan) status_or(status, DSV_STATUS_NAN);
  }
}

__device__ __forceinline__ int32_t key_to_index(uint64_t r) {
  return r == kNanKey ? -1 : (int32_t)(~(uint32_t)r);
}

// Largest chunk key of slot s, considering chunks c0, c0 + step, ... (four loads in flight).
__device__ __forceinline__ uint64_t max_chunk_key(const uint64_t *keys, int64_t s, int n_chunks,
                                                  int c0, int step) {
  uint64_t r = 0;
  for (int c = c0; c < n_chunks; c += 4 * step) {
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = c + u * step < n_chunks ? keys[s * n_chunks + c + u * step] : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) r = v[u] > r ? v[u] : r;
  }
  return r;
}

// The first four chunk keys (c0, c0 + 4, c0 + 8, c0 + 12) a lane reduces for slot row s; loads
// are unconditional (indices clamped into the row), so that the caller issues all of them
// before any is used.
__device__ __forceinline__ void first_chunk_keys(const uint64_t *keys, int64_t s, int n_chunks, int c0,
                                                 uint64_t (&v)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = c0 + 4 * u;
    v[u] = keys[s * n_chunks + (c < n_chunks ? c : n_chunks - 1)];
  }
}
// Largest chunk key of row s from its first four (first_chunk_keys) and the remaining chunks
// of this lane (c0 + 16, c0 + 20, ...), reduced over the four lanes of the row.
__device__ __forceinline__ uint64_t row_key(const uint64_t *keys, int64_t s, int n_chunks, int c0,
                                            const uint64_t (&v)[4]) {
  uint64_t r = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) r = (c0 + 4 * u < n_chunks && v[u] > r) ? v[u] : r;
  if (n_chunks > 16) {
    const uint64_t t = max_chunk_key(keys, s, n_chunks, c0 + 16, 4);
    r = t > r ? t : r;
  }
  uint64_t o = shfl_xor_u64(r, 1);
  r = o > r ? o : r;
  o = shfl_xor_u64(r, 2);
  return o > r ? o : r;
}

// One wavefront per request.  Two memory round trips before the outputs: the request's fields
// and the end boundary, then every chunk key and draft token it needs, issued together.
__global__ __launch_bounds__(kWave) void accept_finalize_kernel(
    int n_bs, int m_bs, int W, const int32_t *__restrict__ slot_tok,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ k,
    const uint64_t *__restrict__ keys, int n_chunks, int32_t *__restrict__ slot_argmax,
    int32_t *__restrict__ accepted, int32_t *__restrict__ bonus, int32_t *__restrict__ progress,
    int32_t *__restrict__ out_tokens, const Top2 *__restrict__ dpart, int n_pos,
    int n_chunks_d, float *__restrict__ margin, int32_t *__restrict__ draft_top1,
    int32_t *status) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  if (keys) {
    const int ki = k[i], off = offsets[i];
    int end = offsets[n_bs];
    end = end < 0 ? 0 : (end > m_bs ? m_bs : end);
    const bool ok = ki >= 0 && ki <= W && off >= 0 && (int64_t)off + ki <= end;
    // four lanes per row, 16 rows per wavefront pass: the request's rows off .. off + k_i - 1
    // and the first pass of the every-slot sweep (slots 16 i ..), with the draft tokens
    const int jr = lane >> 2, q = lane & 3;
    const int64_t s_own = ok && jr < ki ? off + jr : 0;
    const int64_t s_all = (int64_t)i * 16 + jr;
    uint64_t v_own[4], v_all[4];
    first_chunk_keys(keys, s_own, n_chunks, q, v_own);
    first_chunk_keys(keys, s_all < m_bs ? s_all : 0, n_chunks, q, v_all);
    const int32_t tok_l = slot_tok[ok && lane < ki ? off + lane : 0];
    // every slot's choice (slot_argmax), 16 slots per pass
    for (int64_t sb = (int64_t)i * 16; sb < m_bs; sb += (int64_t)n_bs * 16) {
      const int64_t s = sb + jr;
      uint64_t kr;
      if (sb == (int64_t)i * 16) {
        kr = row_key(keys, s < m_bs ? s : 0, n_chunks, q, v_all);
      } else {
        uint64_t v[4];
        first_chunk_keys(keys, s < m_bs ? s : 0, n_chunks, q, v);
        kr = row_key(keys, s < m_bs ? s : 0, n_chunks, q, v);
      }
      if (q == 0 && s < m_bs) slot_argmax[s] = s < end ? key_to_index(kr) : -1;
    }

    if (!ok) {
      if (lane == 0) {
        status_or(status, DSV_STATUS_BAD_REQUEST);
        accepted[i] = -1;
        bonus[i] = -1;
        progress[i] = 0;
      }
      if (out_tokens && lane < W) out_tokens[(int64_t)i * W + lane] = -1;
    } else if (ki == 0) {
      if (lane == 0) {
        accepted[i] = 0;
        bonus[i] = -1;
        progress[i] = 0;
      }
      if (out_tokens && lane < W) out_tokens[(int64_t)i * W + lane] = -1;
    } else {
      const uint64_t kr = row_key(keys, s_own, n_chunks, q, v_own);
      // lane j holds the target's choice at slot off + j and the draft token there
      const uint64_t kj = shfl_u64(kr, 4 * (lane & 15));
      const int32_t g = lane < ki ? key_to_index(kj) : -1;
      const int32_t tok = lane < ki ? tok_l : -1;
      const int32_t g_prev = __shfl(g, lane > 0 ? lane - 1 : 0);
      const bool mismatch = lane >= 1 && lane < ki && tok != g_prev;
      const uint64_t mm = __ballot(mismatch);
      const int a = mm ? (__ffsll((long long)mm) - 1) - 1 : ki - 1;
      const int32_t b = __shfl(g, a);
      if (lane == 0) {
        accepted[i] = a;
        bonus[i] = b;
        progress[i] = 1 + a;
      }
      if (out_tokens && lane < W) {
        const int32_t next_tok = __shfl(tok, lane + 1 < kWave ? lane + 1 : lane);
        out_tokens[(int64_t)i * W + lane] = lane < a ? next_tok : (lane == a ? b : -1);
      }
    }
  }
  if (dpart) {
    for (int p = lane; p < n_pos; p += kWave) {
      const int64_t row = (int64_t)i * n_pos + p;
      Top2 r{0ull, 0u, 0u};
      for (int c = 0; c < n_chunks_d; ++c) r = top2_merge(r, dpart[row * n_chunks_d + c]);
      if (r.nan) {
        margin[row] = __uint_as_float(0x7fc00000u);
        if (draft_top1) draft_top1[row] = -1;
      } else {
        margin[row] = from_ordered_bits((uint32_t)(r.k1 >> 32)) - from_ordered_bits(r.v2);
        if (draft_top1) draft_top1[row] = (int32_t)(~(uint32_t)r.k1);
      }
    }
  }
}

// Chunking of a [rows][vocab] sweep: about 2048 workgroups (eight per CU over the launch), chunks
// of at least one 32 KB block, multiples of 1024 elements (four per lane of a 256-thread
// workgroup).
static void plan_chunks(int64_t rows, int64_t vocab, int *n_chunks, int *chunk) {
  int64_t want = rows > 0 ? (kSweepWgs + rows - 1) / rows : 1;
  int64_t cap = (vocab + kAccBlock - 1) / kAccBlock;
  if (cap < 1) cap = 1;
  int64_t n = want < 1 ? 1 : (want > cap ? cap : want);
  int64_t c = (vocab + n - 1) / n;
  c = (c + 1023) / 1024 * 1024;
  n = (vocab + c - 1) / c;
  *n_chunks = (int)(n < 1 ? 1 : n);
  *chunk = (int)c;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace dsv

extern "C" size_t dsv_accept_workspace_bytes(int32_t m_bs, int32_t vocab, int32_t n_bs,
                                             int32_t n_pos, int32_t draft_vocab) {
  size_t bytes = 0;
  int nc, ch;
  if (m_bs > 0 && vocab > 0) {
    dsv::plan_chunks(m_bs, vocab, &nc, &ch);
    bytes += dsv::align256((size_t)m_bs * nc * sizeof(uint64_t));
  }
  if (n_bs > 0 && n_pos > 0 && draft_vocab > 0) {
    dsv::plan_chunks((int64_t)n_bs * n_pos, draft_vocab, &nc, &ch);
    bytes += dsv::align256((size_t)n_bs * n_pos * nc * sizeof(dsv::Top2));
  }
  return bytes;
}

extern "C" dsv_status dsv_accept(int32_t n_bs, int32_t m_bs, int32_t W, int32_t vocab,
                                 const float *target_logits, const int32_t *slot_tok,
                                 const int32_t *offsets, const int32_t *k, int32_t *slot_argmax,
                                 int32_t *accepted, int32_t *bonus, int32_t *progress,
                                 int32_t *out_tokens, const float *draft_logits, int32_t n_pos,
                                 int32_t draft_vocab, float *margin, int32_t *draft_top1,
                                 void *workspace, size_t workspace_bytes, int32_t *status,
                                 hipStream_t stream) {
  using namespace dsv;
  if (n_bs < 0 || m_bs < 0 || W < 1 || W > DSV_MAX_W || !status) return DSV_ERR_INVALID_ARG;
  const bool tgt = target_logits != nullptr;
  const bool drf = draft_logits != nullptr;
  if (tgt && (vocab < 1 || !slot_tok || !offsets || !k || !slot_argmax || !accepted || !bonus ||
              !progress))
    return DSV_ERR_INVALID_ARG;
  if (drf && (n_pos < 1 || draft_vocab < 2 || !margin)) return DSV_ERR_INVALID_ARG;
  if (n_bs == 0 || (!tgt && !drf)) return DSV_OK;
  const size_t need = dsv_accept_workspace_bytes(tgt ? m_bs : 0, tgt ? vocab : 0, drf ? n_bs : 0,
                                                 drf ? n_pos : 0, drf ? draft_vocab : 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSV_ERR_WORKSPACE;
  {
    const int64_t mt = tgt ? m_bs : 0, nt = tgt ? n_bs : 0, nd = drf ? (int64_t)n_bs * n_pos : 0;
    const Span out[] = {{slot_argmax, span_bytes(mt, 4)}, {accepted, span_bytes(nt, 4)},
                        {bonus, span_bytes(nt, 4)},       {progress, span_bytes(nt, 4)},
                        {out_tokens, span_bytes(nt * W, 4)}, {margin, span_bytes(nd, 4)},
                        {draft_top1, span_bytes(nd, 4)},  {workspace, need},
                        {status, 4}};
    const Span in[] = {{target_logits, span_bytes(mul_sat({mt, vocab}), 4)}, {slot_tok, span_bytes(mt, 4)},
                       {offsets, span_bytes(nt + (tgt ? 1 : 0), 4)}, {k, span_bytes(nt, 4)},
                       {draft_logits, span_bytes(mul_sat({nd, drf ? draft_vocab : 0}), 4)}};
    if (outputs_alias(out, in)) return DSV_ERR_INVALID_ARG;
  }

  char *ws = static_cast<char *>(workspace);
  uint64_t *keys = nullptr;
  int nc_t = 1, ch_t = 0, nc_d = 1, ch_d = 0;
  if (tgt && m_bs > 0) plan_chunks(m_bs, vocab, &nc_t, &ch_t);
  if (drf) plan_chunks((int64_t)n_bs * n_pos, draft_vocab, &nc_d, &ch_d);
  if (!launch_fits(tgt ? (int64_t)m_bs * nc_t : 0, kAccThreads) ||
      !launch_fits(drf ? (int64_t)n_bs * n_pos * nc_d : 0, kAccThreads))
    return DSV_ERR_INVALID_ARG;
  if (tgt && m_bs > 0) {
    keys = reinterpret_cast<uint64_t *>(ws);
    ws += align256((size_t)m_bs * nc_t * sizeof(uint64_t));
    const bool vec = (vocab % 4 == 0) && ((uintptr_t)target_logits % 16 == 0);
    const int64_t grid = (int64_t)m_bs * nc_t;
    if (vec)
      hipLaunchKernelGGL(argmax_partial_kernel<true>, dim3((unsigned)grid), dim3(kAccThreads), 0,
                         stream, target_logits, (int64_t)vocab, ch_t, nc_t, m_bs, offsets, n_bs,
                         keys, status);
    else
      hipLaunchKernelGGL(argmax_partial_kernel<false>, dim3((unsigned)grid), dim3(kAccThreads), 0,
                         stream, target_logits, (int64_t)vocab, ch_t, nc_t, m_bs, offsets, n_bs,
                         keys, status);
    DSV_LAUNCH_CHECK();
  }
  Top2 *dpart = nullptr;
  if (drf) {
    const int64_t rows = (int64_t)n_bs * n_pos;
    dpart = reinterpret_cast<Top2 *>(ws);
    const bool vec = (draft_vocab % 4 == 0) && ((uintptr_t)draft_logits % 16 == 0);
    const int64_t grid = rows * nc_d;
    if (vec)
      hipLaunchKernelGGL(top2_partial_kernel<true>, dim3((unsigned)grid), dim3(kAccThreads), 0,
                         stream, draft_logits, (int64_t)draft_vocab, ch_d, nc_d, dpart, status);
    else
      hipLaunchKernelGGL(top2_partial_kernel<false>, dim3((unsigned)grid), dim3(kAccThreads), 0,
                         stream, draft_logits, (int64_t)draft_vocab, ch_d, nc_d, dpart, status);
    DSV_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(accept_finalize_kernel, dim3(n_bs), dim3(kWave), 0, stream, n_bs, m_bs, W,
                     slot_tok, offsets, k, keys, nc_t, slot_argmax, accepted, bonus, progress,
                     out_tokens, dpart, n_pos, nc_d, margin, draft_top1, status);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
