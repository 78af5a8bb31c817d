// Draft confidence features for the acceptance predictor.
//
// DScale (arXiv HTML), Sec. III-C "Acceptance predictor": every draft position contributes
// its highest logit, the 15 gaps from it to the logits of ranks 2-16, the top token's
// log-probability and the entropy of the position's distribution -- 18 values, 270 per
// request for 15 positions, in draft order.
//
// Two kernels:
//  1. feat_partial_kernel -- the HBM-bound sweep: one workgroup per (row, chunk) streams the
//     chunk (eight 16-byte non-temporal loads in flight per thread, the next block's loads
//     issued before the current block is reduced).  Each wavefront keeps the 16 largest
//     values it has seen as a sorted list spread over lanes 0-15; a value enters only if it
//     beats the list's last entry, which after the first few blocks is rare, so the common
//     cost per value is one comparison (a lane first compares the maximum of its 32 values
//     of the block).  Alongside, each lane keeps online statistics relative to its running
//     maximum m, in log2 units (z2 = z log2 e, m2 = m log2 e): S = sum 2^(z2 - m2) and
//     U = sum 2^(z2 - m2) (z2 - m2), so that each value costs one fma for its exponent.  The
//     workgroup merges its four lists and statistics into one partial record per (row, chunk).
//  2. feat_finalize_kernel -- one wavefront per row merges the chunk records and writes the
//     18 features: top = l[0], gaps fp32(l[0] - l[r - 1]), log p(top) = -ln S (S relative to
//     the top logit), entropy = ln S - U ln 2 / S.
#include "dsv_internal.h"

namespace dsv {

constexpr int kFtThreads = 256;
constexpr int kFtLoads = 8;                            // 16-byte loads in flight per thread
constexpr int kFtBlock = kFtThreads * 4 * kFtLoads;    // floats per 32 KB block
constexpr int kTopK = 16;
constexpr int kFeat = 18;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

struct FeatPart {
  float top[kTopK];  // the chunk's 16 largest values, descending (-inf where fewer)
  float m, S, U;     // statistics relative to m (the chunk maximum, log2 units); S = 0 if none is finite
  int32_t bad;       // a NaN or +inf logit
};

// Online statistics (log2 units): add the value set summarised by (m2, S2, U2) to (m, S, U).
__device__ __forceinline__ void ent_merge(float &m, float &S, float &U, float m2, float S2, float U2) {
  if (S2 == 0.f) return;
  if (S == 0.f) {
    m = m2;
    S = S2;
    U = U2;
    return;
  }
  const float mn = fmaxf(m, m2);
  const float d1 = m - mn, d2 = m2 - mn;  // <= 0
  const float r1 = __builtin_amdgcn_exp2f(d1), r2 = __builtin_amdgcn_exp2f(d2);
  U = r1 * (U + d1 * S) + r2 * (U2 + d2 * S2);
  S = r1 * S + r2 * S2;
  m = mn;
}

// A float below x (x finite or +inf): the next one down, or -FLT_MIN below zero, so that
// v > float_below(x) holds for every v >= x (a lower bound only prunes less).
__device__ __forceinline__ float float_below(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x > 0.f) return __uint_as_float(u - 1);
  if (x == 0.f) return -1.17549435e-38f;
  return __uint_as_float(u + 1);
}

// Inserts every lane's candidate x that beats the wavefront's threshold tau into the list
// (lane k < 16 holds the k-th largest value), one candidate at a time in lane order; tau is
// the list's 16th value, or `floor` while that is lower (a bound below which no value can be
// among the 16 largest).
// The candidate is broadcast with readlane and the list shifted with a DPP row shift (the
// list is one 16-lane row), so an insertion is a short chain of VALU/SALU operations.
__device__ __forceinline__ void wave_top_insert(float &l, float &tau, float x,
                                                float floor = -INFINITY) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t mask = __ballot(x > tau);
  while (mask) {
    const int src = __ffsll((long long)mask) - 1;
    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
    // prev = l of the lane below within the row (row_shr:1); lane 0 of the row gets +inf
    const float prev = __int_as_float(__builtin_amdgcn_update_dpp(
        __float_as_int(INFINITY), __float_as_int(l), 0x111, 0xf, 0xf, false));
    if (lane < kTopK) l = l >= v ? l : (prev >= v ? v : prev);
    tau = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), kTopK - 1)), floor);
    mask &= mask - 1;
    mask &= __ballot(x > tau);
  }
}

// Sorts the wavefront's 64 values (one per lane) in descending order across the lanes
// (bitonic network: lanes whose bit k is clear form descending runs, the others ascending,
// and the final stage merges one descending run).
__device__ __forceinline__ float wave_sort_desc(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const float o = __shfl_xor(v, j);
      const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
      v = keep_max ? fmaxf(v, o) : fminf(v, o);
    }
  return v;
}

__global__ __launch_bounds__(kFtThreads) void feat_partial_kernel(
    const float *__restrict__ logits, int64_t vocab, int chunk, int n_chunks, bool vec4,
    FeatPart *__restrict__ part) {
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / n_chunks;
  const int ch = (int)(bid % n_chunks);
  const int64_t lo = (int64_t)ch * chunk;
  const int64_t hi = min(vocab, lo + chunk);
  const float *x = logits + row * vocab;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  float l = -INFINITY, tau = -INFINITY;  // the wavefront's list (lanes 0-15) and its threshold
  float floor = -INFINITY;
  bool first = true;
  float m = -INFINITY, m2 = -INFINITY, S = 0.f, U = 0.f;  // m2 = m log2 e
  bool bad = false;
  // a larger maximum rescales the running sums first
  auto raise = [&](float e) __attribute__((always_inline)) {
    const float e2 = e * kLog2e;
    const float d = m2 - e2;  // <= 0 (-inf while S = 0)
    const float r = __builtin_amdgcn_exp2f(d);
    U = S > 0.f ? r * (U + d * S) : 0.f;
    S = S > 0.f ? r * S : 0.f;
    m = e;
    m2 = e2;
  };
  // one value: 2^(z2 - m2) with its exponent from one fma; a -inf logit adds nothing (its
  // weight is 0 and its exponent, clamped for the product, finite)
  auto add1 = [&](float e) __attribute__((always_inline)) {
    const float d = __builtin_fmaf(e, kLog2e, -m2);
    const float w = __builtin_amdgcn_exp2f(d);
    S += w;
    U = __builtin_fmaf(w, fmaxf(d, -128.f), U);
  };
  auto stat1 = [&](float e) __attribute__((always_inline)) {
    bad |= !(e < INFINITY) && e != -INFINITY;
    if (e > m) raise(e);
    if (e > -INFINITY) add1(e);
  };
  if (vec4) {
    constexpr int64_t kStep = 4 * kFtThreads;
    auto load = [&](f32x4 (&f)[kFtLoads], int64_t v0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kFtLoads; ++u) {
        const int64_t v = v0 + u * kStep;
        f[u] = v < hi ? gload_stream<f32x4>(x + v) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    };
    auto reduce = [&](const f32x4 (&f)[kFtLoads]) __attribute__((always_inline)) {
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < kFtLoads; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) bm = fmaxf(bm, f[u][q]);
      if (bm > m) raise(bm);
      if (m > -INFINITY) {
        // a NaN logit turns S into NaN here (its weight is NaN), caught before a later
        // maximum rescales S
#pragma unroll
        for (int u = 0; u < kFtLoads; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) add1(f[u][q]);
        bad |= S != S;
      } else {
        // no finite value yet on this lane: the block holds only -inf and NaN
#pragma unroll
        for (int u = 0; u < kFtLoads; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) bad |= f[u][q] != f[u][q];
      }
      // list: only lanes whose block maximum beats the threshold look further
      if (first) {
        // the 16th largest of the 64 lane maxima bounds the 16th largest value from below
        // (16 values reach it); sorting the maxima descending across the lanes (bitonic)
        // gives it, and values below it are never inserted
        const float v = wave_sort_desc(bm);
        const float t16 = __shfl(v, kTopK - 1);
        floor = t16 > -INFINITY ? float_below(t16) : -INFINITY;
        tau = floor;
        first = false;
      }
      if (__ballot(bm > tau)) {
#pragma unroll
        for (int u = 0; u < kFtLoads; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) wave_top_insert(l, tau, f[u][q], floor);
      }
    };
    // the block loop is uniform over the workgroup (every lane takes part in the list
    // insertions); values past the end load as -inf
    f32x4 fa[kFtLoads], fb[kFtLoads];
    int64_t b0 = lo;
    load(fa, b0 + 4 * t);
    for (; b0 < hi; b0 += 2 * kFtBlock) {
      if (b0 + kFtBlock < hi) load(fb, b0 + kFtBlock + 4 * t);
      reduce(fa);
      if (b0 + kFtBlock >= hi) break;
      if (b0 + 2 * kFtBlock < hi) load(fa, b0 + 2 * kFtBlock + 4 * t);
      reduce(fb);
    }
  } else {
    // scalar path: the wavefront steps together so that every lane takes part in the
    // list insertion (lanes past the end contribute -inf)
    for (int64_t v0 = lo; v0 < hi; v0 += kFtThreads) {
      const int64_t v = v0 + t;
      const float e = v < hi ? x[v] : -INFINITY;
      stat1(e);
      wave_top_insert(l, tau, e);
    }
  }
  bad |= m == INFINITY;
  m = m2;  // the records carry the maximum in log2 units
  // merge the lanes' statistics
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float m2 = __shfl_xor(m, d), S2 = __shfl_xor(S, d), U2 = __shfl_xor(U, d);
    ent_merge(m, S, U, m2, S2, U2);
  }
  __shared__ float sh_l[kFtThreads / kWave][kTopK];
  __shared__ float sh_s[kFtThreads / kWave][3];
  __shared__ int sh_bad;
  if (t == 0) sh_bad = 0;
  __syncthreads();
  if (bad) sh_bad = 1;
  if (lane < kTopK) sh_l[wv][lane] = l;
  if (lane == 0) {
    sh_s[wv][0] = m;
    sh_s[wv][1] = S;
    sh_s[wv][2] = U;
  }
  __syncthreads();
  if (wv == 0) {
    // wavefront 0 merges the four lists: lane j offers list j / 16, entry j % 16
    l = wave_sort_desc(sh_l[lane / kTopK][lane % kTopK]);
    FeatPart *p = part + row * n_chunks + ch;
    if (lane < kTopK) p->top[lane] = l;
    if (lane == 0) {
      float M = sh_s[0][0], SS = sh_s[0][1], UU = sh_s[0][2];
      for (int w = 1; w < kFtThreads / kWave; ++w) ent_merge(M, SS, UU, sh_s[w][0], sh_s[w][1], sh_s[w][2]);
      p->m = M;
      p->S = SS;
      p->U = UU;
      p->bad = sh_bad;
    }
  }
}

// One wavefront per row.
__global__ __launch_bounds__(kWave) void feat_finalize_kernel(int64_t rows, int n_chunks,
                                                              const FeatPart *__restrict__ part,
                                                              float *__restrict__ feat,
                                                              int32_t *status) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const FeatPart *p = part + row * n_chunks;
  // statistics: lane c takes chunks c, c + 64, ...
  float m = -INFINITY, S = 0.f, U = 0.f;
  int bad = 0;
  for (int c = lane; c < n_chunks; c += kWave) {
    ent_merge(m, S, U, p[c].m, p[c].S, p[c].U);
    bad |= p[c].bad;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float m2 = __shfl_xor(m, d), S2 = __shfl_xor(S, d), U2 = __shfl_xor(U, d);
    ent_merge(m, S, U, m2, S2, U2);
  }
  bad = __ballot(bad != 0) ? 1 : 0;
  // lists: lanes 0-15 carry the running top 16, lanes 16-63 take 48 new entries per round,
  // and a sort of the 64 keeps the largest 16 in lanes 0-15
  float l = -INFINITY;
  const int total = n_chunks * kTopK;
  for (int base = 0; base < total; base += kWave - kTopK) {
    const int j = base + lane - kTopK;
    const float cand = lane < kTopK ? l : (j < total ? p[j / kTopK].top[j % kTopK] : -INFINITY);
    l = wave_sort_desc(cand);
  }
  float *f = feat + row * kFeat;
  const float top = __shfl(l, 0);
  if (bad || !(top > -INFINITY)) {
    if (lane < kFeat) f[lane] = __uint_as_float(0x7fc00000u);
    if (lane == 0) status_or(status, DSV_STATUS_NAN);
    return;
  }
  const float lnS = __builtin_amdgcn_logf(S) * kLn2;
  if (lane == 0) f[0] = top;
  else if (lane < kTopK) f[lane] = top - l;
  else if (lane == kTopK) f[kTopK] = -lnS;
  else if (lane == kTopK + 1) f[kTopK + 1] = lnS - U * kLn2 / S;
}

// Sweep chunking: about 2048 workgroups, chunks of whole 1024-element groups (four per lane).
static void plan_feat(int64_t rows, int64_t vocab, int *n_chunks, int *chunk) {
  int64_t want = rows > 0 ? (2048 + rows - 1) / rows : 1;
  int64_t cap = (vocab + kFtBlock - 1) / kFtBlock;
  if (cap < 1) cap = 1;
  int64_t n = want < 1 ? 1 : (want > cap ? cap : want);
  int64_t c = (vocab + n - 1) / n;
  c = (c + 1023) / 1024 * 1024;
  n = (vocab + c - 1) / c;
  *n_chunks = (int)(n < 1 ? 1 : n);
  *chunk = (int)c;
}

}  // namespace dsv

extern "C" size_t dsv_draft_features_workspace_bytes(int64_t rows, int32_t vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  int nc, ch;
  dsv::plan_feat(rows, vocab, &nc, &ch);
  return ((size_t)rows * nc * sizeof(dsv::FeatPart) + 255) / 256 * 256;
}

extern "C" dsv_status dsv_draft_features(int64_t rows, int32_t vocab, const float *draft_logits,
                                         float *features, void *workspace,
                                         size_t workspace_bytes, int32_t *status,
                                         hipStream_t stream) {
  using namespace dsv;
  if (rows < 0 || vocab < kTopK || !status) return DSV_ERR_INVALID_ARG;
  if (rows == 0) return DSV_OK;
  if (!draft_logits || !features) return DSV_ERR_INVALID_ARG;
  int nc, ch;
  plan_feat(rows, vocab, &nc, &ch);
  if (!launch_fits(mul_sat({rows, nc}), kFtThreads)) return DSV_ERR_INVALID_ARG;
  const size_t need = dsv_draft_features_workspace_bytes(rows, vocab);
  if (!workspace || workspace_bytes < need) return DSV_ERR_WORKSPACE;
  {
    const Span out[] = {{features, span_bytes(rows * kFeat, 4)}, {workspace, need}, {status, 4}};
    const Span in[] = {{draft_logits, span_bytes(rows * vocab, 4)}};
    if (outputs_alias(out, in)) return DSV_ERR_INVALID_ARG;
  }
  FeatPart *part = static_cast<FeatPart *>(workspace);
  const bool vec = (vocab % 4 == 0) && ((uintptr_t)draft_logits % 16 == 0);
  hipLaunchKernelGGL(feat_partial_kernel, dim3((unsigned)(rows * nc)), dim3(kFtThreads), 0, stream,
                     draft_logits, (int64_t)vocab, ch, nc, vec, part);
  DSV_LAUNCH_CHECK();
  hipLaunchKernelGGL(feat_finalize_kernel, dim3((unsigned)rows), dim3(kWave), 0, stream, rows, nc,
                     part, features, status);
  DSV_LAUNCH_CHECK();
  return DSV_OK;
}
