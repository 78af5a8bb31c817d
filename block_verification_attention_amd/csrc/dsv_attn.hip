// Tile-routed attention for packed verification slots, plus the wide-tile prefill path.
//
// DScale (arXiv HTML), Sec. III-B "Path-aware tile router": verification rows (at most
// W = 16 per request) use a tile whose height matches the candidate width, while prefill
// keeps a wide tile so that each loaded KV row is reused by many query rows.  Sec. III-D:
// valid rows read slot offset_i + j with request-local causal masking (query j sees the whole
// committed context and candidates 0..j) and the supplied cache references (this step's
// candidate KV is written at the packed cache locations).
//
// gfx950 design
// -------------
// Verification kernel: one workgroup per (KV split, request, KV head).  Its G waves are the
// G query heads that share the KV head (grouped-query attention), each holding a 16-row
// bf16 MFMA query tile (rows j >= k_i are zero and never written).  K and V tiles of 64 rows
// are streamed once from HBM per workgroup and staged in LDS, so the KV bytes are read once
// per KV head regardless of G.  Scores are computed transposed (S^T = K Q^T, MFMA
// 16x16x32 bf16) so that the fp32 accumulator layout is directly the B operand of the
// second product (O^T = V^T P^T) after rounding P to bf16; V is transposed when it is
// written to LDS.  The softmax is online in fp32, base 2 (scale folded with log2 e).
// The pages' grid has one block per (request, head); with GQA grouping that gives only
// n_bs * hkv units (64 for 8 requests x 8 KV heads) for 256 CUs, so each request's KV range
// is split into chunks processed by separate workgroups and merged by log-sum-exp weights in
// a second, deterministic kernel.
//
// Prefill kernel: the same tile machinery with 8 waves stacked along the query rows of one
// head, giving a 128-row tile (the hardware-selected wide tile of the pages) so that every
// KV tile staged in LDS feeds 128 query rows.
//
// LDS layouts (bf16):
//   sK  [64][D]  row-major; 16-byte column slots XOR-swizzled by (row & 15) so that the 16
//                rows an MFMA operand read touches fall in distinct banks.
//   sVt [D][64]  V transposed; 8-byte slots (4 KV rows) XOR-swizzled by a function of d that
//                keeps both the transposing writes and the operand reads conflict-free.
#include <math.h>

#include "dsv_internal.h"

namespace dsv {

constexpr int kTileKV = 64;
constexpr int kPfWaves = 8;  // 8 waves x 16 rows = 128-row prefill tile
constexpr int kPfRows = kPfWaves * 16;

struct AttnParams {
  void *k_pool, *v_pool;
  int64_t pool_rows, stride_head, stride_row;
  int hq, hkv, G;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  // verification set
  int n_bs, m_bs, W;
  const int32_t *offsets, *k, *ctx_len;
  const int64_t *kv_base, *slot_cache_loc;
  const void *q, *k_new, *v_new;
  void *out;
  float *lse;
  int chunk, n_splits;
  float *ws_o, *ws_lse;  // [n_splits][m_bs][hq][D], [n_splits][m_bs][hq]
  // prefill set
  int n_pf, pf_blocks, pf_q_rows, pf_max_len;
  const int32_t *pf_q_start, *pf_q_len, *pf_ctx;
  const int64_t *pf_kv_base;
  const void *pf_q, *pf_k_new, *pf_v_new;
  void *pf_out;
  float *pf_lse;
  int32_t *status;
};

// Checks request i of the verification set; on success returns 0 and its fields.
__device__ __forceinline__ int verify_request(const AttnParams &p, int i, int &ki, int &off, int &c,
                                              int64_t &kb) {
  ki = p.k[i];
  off = p.offsets[i];
  c = p.ctx_len[i];
  kb = p.kv_base[i];
  if (ki < 0 || ki > p.W || off < 0 || (int64_t)off + ki > p.m_bs || c < 0 || kb < 0)
    return DSV_STATUS_BAD_REQUEST;
  if (kb + c + ki > p.pool_rows || (int64_t)c + ki > (int64_t)p.n_splits * p.chunk)
    return DSV_STATUS_POOL;
  return 0;
}

__device__ __forceinline__ int prefill_request(const AttnParams &p, int r, int &ql, int &qs, int &c,
                                               int64_t &kb) {
  ql = p.pf_q_len[r];
  qs = p.pf_q_start[r];
  c = p.pf_ctx[r];
  kb = p.pf_kv_base[r];
  if (ql < 0 || ql > p.pf_max_len || qs < 0 || (int64_t)qs + ql > p.pf_q_rows || c < 0 || kb < 0 ||
      kb + c + ql > p.pool_rows)
    return DSV_STATUS_PREFILL;
  return 0;
}

__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) + 2 * (d & 7)) & 15; }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Zero-fills rows [r0, r1) of a [rows][hq][D] bf16 tensor for heads [h0, h0 + nh), lse -inf.
template <int D>
__device__ void zero_rows_bf16(uint16_t *out, float *lse, int hq, int r0, int r1, int h0, int nh,
                               int tid, int nt) {
  constexpr int C = D / 8;
  const int64_t total = (int64_t)(r1 - r0) * nh * C;
  for (int64_t e = tid; e < total; e += nt) {
    int cc = (int)(e % C);
    int64_t t = e / C;
    int hh = (int)(t % nh);
    int r = r0 + (int)(t / nh);
    *reinterpret_cast<uint4 *>(out + ((int64_t)r * hq + h0 + hh) * D + cc * 8) = make_uint4(0, 0, 0, 0);
  }
  if (lse)
    for (int64_t e = tid; e < (int64_t)(r1 - r0) * nh; e += nt)
      lse[(int64_t)(r0 + e / nh) * hq + h0 + e % nh] = -INFINITY;
}

// ---------------------------------------------------------------------------
// bf16 MFMA attention kernel.  PF = false: verification (NW = G waves, one 16-row query
// tile per query head, split KV).  PF = true: prefill (NW = 8 waves along the query rows of
// one head).
// ---------------------------------------------------------------------------
template <int D, int NW, bool PF>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnParams p) {
  constexpr int NT = NW * 64;
  constexpr int KCH = D / 8;                    // 16-byte chunks per row
  constexpr int SW = KCH < 16 ? KCH : 16;       // K swizzle period
  constexpr int NKC = kTileKV * KCH;            // K chunks per tile
  constexpr int NVB = (kTileKV / 4) * KCH;      // V blocks (4 rows x 8 columns) per tile
  constexpr int KPT = (NKC + NT - 1) / NT;
  constexpr int VPT = (NVB + NT - 1) / NT;
  constexpr int DB = D / 16;
  constexpr int KS = D / 32;

  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t *sK = lds;
  uint16_t *sVt = lds + kTileKV * D;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;

  const uint16_t *kpool = static_cast<const uint16_t *>(p.k_pool);
  const uint16_t *vpool = static_cast<const uint16_t *>(p.v_pool);

  // ---- work unit ----
  int g, h, c, r_lo, r_hi, row0, nrows, split = 0, n_splits_i = 1, off = 0;
  int64_t kb, q_row0;
  const uint16_t *qsrc;
  const uint16_t *knew = nullptr, *vnew = nullptr;
  if constexpr (!PF) {
    const int bid = blockIdx.x;
    g = bid % p.hkv;
    const int t = bid / p.hkv;
    const int i = t % p.n_bs;
    split = t / p.n_bs;
    h = g * p.G + w;
    if (i == 0 && split == 0) {
      int end = p.offsets[p.n_bs];
      end = end < 0 ? 0 : (end > p.m_bs ? p.m_bs : end);
      zero_rows_bf16<D>(static_cast<uint16_t *>(p.out), p.lse, p.hq, end, p.m_bs, g * p.G, p.G,
                        tid, NT);
    }
    int ki;
    const int bad = verify_request(p, i, ki, off, c, kb);
    if (bad) {
      if (split == 0) {
        if (tid == 0 && g == 0) status_or(p.status, bad);
        if (ki >= 0 && ki <= p.W && off >= 0 && (int64_t)off + ki <= p.m_bs)
          zero_rows_bf16<D>(static_cast<uint16_t *>(p.out), p.lse, p.hq, off, off + ki, g * p.G,
                            p.G, tid, NT);
      }
      return;
    }
    const int n_vis = c + ki;
    n_splits_i = (n_vis + p.chunk - 1) / p.chunk;
    if (ki == 0 || split >= n_splits_i) return;
    r_lo = split * p.chunk;
    r_hi = min(n_vis, r_lo + p.chunk);
    row0 = 0;
    nrows = ki;
    q_row0 = off;
    qsrc = static_cast<const uint16_t *>(p.q);
    if (p.k_new) {
      knew = static_cast<const uint16_t *>(p.k_new);
      vnew = static_cast<const uint16_t *>(p.v_new);
    }
  } else {
    const int bid = blockIdx.x;
    const int per = p.n_pf * p.hq;
    const int b = p.pf_blocks - 1 - bid / per;  // longest row blocks first
    const int r = (bid % per) / p.hq;
    h = (bid % per) % p.hq;
    g = h / p.G;
    int ql, qs;
    const int bad = prefill_request(p, r, ql, qs, c, kb);
    if (bad) {
      if (tid == 0 && b == 0 && h == 0) status_or(p.status, bad);
      return;
    }
    row0 = b * kPfRows;
    if (row0 >= ql) return;
    nrows = ql;
    r_lo = 0;
    r_hi = c + min(row0 + kPfRows, ql);
    q_row0 = qs;
    qsrc = static_cast<const uint16_t *>(p.pf_q);
  }
  (void)n_splits_i;

  // ---- query fragment (B operand of S^T = K Q^T): row lq, columns 32ks + 8lg .. +7 ----
  const int my_row = PF ? row0 + w * 16 + lq : lq;  // query row index within the request
  bf16x8 qf[KS];
  {
    const bool ok = my_row < nrows;
    const uint16_t *qp = qsrc + ((q_row0 + (ok ? my_row : 0)) * p.hq + h) * (int64_t)D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = ok ? *reinterpret_cast<const uint4 *>(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  const int lim = c + my_row;  // last visible position of this lane's query row

  // ---- KV source of position pos (pool row, or this step's candidate row) ----
  auto ksrc = [&](int pos) -> const uint16_t * {
    if (knew && pos >= c)
      return knew + ((int64_t)(off + pos - c) * p.hkv + g) * D;
    return kpool + g * p.stride_head + (kb + pos) * p.stride_row;
  };
  auto vsrc = [&](int pos) -> const uint16_t * {
    if (vnew && pos >= c)
      return vnew + ((int64_t)(off + pos - c) * p.hkv + g) * D;
    return vpool + g * p.stride_head + (kb + pos) * p.stride_row;
  };
  // Candidate rows taken from k_new / v_new are also stored at their cache references.
  auto kv_dest = [&](int pos) -> int64_t {
    const int64_t loc = p.slot_cache_loc[off + pos - c];
    if (loc < 0 || loc >= p.pool_rows) {
      status_or(p.status, DSV_STATUS_POOL);
      return -1;
    }
    return g * p.stride_head + loc * p.stride_row;
  };

  uint4 kreg[KPT];
  uint4 vreg[VPT][4];
  auto load_tile = [&](int base) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ci = tid + u * NT;
      kreg[u] = make_uint4(0, 0, 0, 0);
      if (ci < NKC) {
        const int row = ci / KCH, col = ci % KCH;
        const int pos = base + row;
        if (pos < r_hi) {
          kreg[u] = *reinterpret_cast<const uint4 *>(ksrc(pos) + col * 8);
          if (knew && pos >= c) {
            const int64_t dst = kv_dest(pos);
            if (dst >= 0)
              *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.k_pool) + dst + col * 8) = kreg[u];
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int bi = tid + u * NT;
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[u][r] = make_uint4(0, 0, 0, 0);
      if (bi < NVB) {
        const int dc = bi % KCH, rg = bi / KCH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pos = base + 4 * rg + r;
          if (pos < r_hi) {
            vreg[u][r] = *reinterpret_cast<const uint4 *>(vsrc(pos) + dc * 8);
            if (vnew && pos >= c) {
              const int64_t dst = kv_dest(pos);
              if (dst >= 0)
                *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.v_pool) + dst + dc * 8) =
                    vreg[u][r];
            }
          }
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int ci = tid + u * NT;
      if (ci < NKC) {
        const int row = ci / KCH, col = ci % KCH;
        *reinterpret_cast<uint4 *>(sK + row * D + ((col ^ (row & (SW - 1))) * 8)) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int bi = tid + u * NT;
      if (bi < NVB) {
        const int dc = bi % KCH, rg = bi / KCH;
        const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&vreg[u][0]);
        const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&vreg[u][1]);
        const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&vreg[u][2]);
        const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&vreg[u][3]);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // columns d = 8dc + 2e2 (low halves) and 8dc + 2e2 + 1 (high halves)
          const int d0 = dc * 8 + 2 * e2;
          uint2 lo = make_uint2(pack_lo(r0[e2], r1[e2]), pack_lo(r2[e2], r3[e2]));
          uint2 hi = make_uint2(pack_hi(r0[e2], r1[e2]), pack_hi(r2[e2], r3[e2]));
          *reinterpret_cast<uint2 *>(sVt + d0 * kTileKV + ((rg ^ vt_swz(d0)) * 4)) = lo;
          *reinterpret_cast<uint2 *>(sVt + (d0 + 1) * kTileKV + ((rg ^ vt_swz(d0 + 1)) * 4)) = hi;
        }
      }
    }
  };

  f32x4 acc_o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (r_hi - r_lo + kTileKV - 1) / kTileKV;
  // rows of this wave: PF -> [row0 + 16w, +16); verify -> [0, 16)
  const int wave_row_lo = PF ? row0 + w * 16 : 0;
  const bool wave_live = wave_row_lo < nrows;

  load_tile(r_lo);
  for (int t = 0; t < n_tiles; ++t) {
    const int base = r_lo + t * kTileKV;
    __syncthreads();  // previous tile's LDS reads are done
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(base + kTileKV);

    // skip tiles wholly past this wave's last visible position
    if (!wave_live || base > c + wave_row_lo + 15) continue;

    // S^T blocks: acc_s[kb][e] = score of KV row base + 16kb + 4lg + e for query row lq
    f32x4 acc_s[4];
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk) {
      acc_s[kbk] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t *krow = sK + (16 * kbk + lq) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int slot = (4 * ks + lg) ^ (lq & (SW - 1));
        bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(krow + slot * 8));
        acc_s[kbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc_s[kbk], 0, 0, 0);
      }
    }
    // scale, mask, tile max
    float mt = -INFINITY;
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = base + 16 * kbk + 4 * lg + e;
        float x = acc_s[kbk][e] * p.scale_log2;
        x = (pos < r_hi && pos <= lim) ? x : -INFINITY;
        acc_s[kbk][e] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    // P rounded to bf16 is the B operand of O^T = V^T P^T; the row sum (and so the lse)
    // accumulates the fp32 values
    uint32_t pb[4][2];
    float lsum = 0.f;
#pragma unroll
    for (int kbk = 0; kbk < 4; ++kbk) {
      uint32_t bits[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(acc_s[kbk][e] - m_use);
        bits[e] = f32_to_bf16_bits(pe);
        lsum += pe;
      }
      pb[kbk][0] = bits[0] | (bits[1] << 16);
      pb[kbk][1] = bits[2] | (bits[3] << 16);
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[db] *= alpha;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 b = __builtin_bit_cast(
          bf16x8, make_uint4(pb[2 * kk][0], pb[2 * kk][1], pb[2 * kk + 1][0], pb[2 * kk + 1][1]));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + lq;
        const uint16_t *vrow = sVt + d * kTileKV;
        const int sw = vt_swz(d);
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + (((8 * kk + lg) ^ sw) * 4));
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + (((8 * kk + 4 + lg) ^ sw) * 4));
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc_o[db], 0, 0, 0);
      }
    }
  }

  if (!wave_live) return;
  // full row sum across the four lane groups holding the row
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (my_row >= nrows) return;
  const bool empty = !(l_run > 0.f);
  const float inv_l = empty ? 0.f : 1.f / l_run;
  const float lse_v = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f;
  const int64_t orow = q_row0 + my_row;
  if (PF || n_splits_i == 1) {
    uint16_t *o = static_cast<uint16_t *>(PF ? p.pf_out : p.out) + (orow * p.hq + h) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 16 * db + 4 * lg;
      uint2 v;
      v.x = f32_to_bf16_bits(acc_o[db][0] * inv_l) | (f32_to_bf16_bits(acc_o[db][1] * inv_l) << 16);
      v.y = f32_to_bf16_bits(acc_o[db][2] * inv_l) | (f32_to_bf16_bits(acc_o[db][3] * inv_l) << 16);
      *reinterpret_cast<uint2 *>(o + d) = v;
    }
    float *lse = PF ? p.pf_lse : p.lse;
    if (lse && lg == 0) lse[orow * p.hq + h] = lse_v;
  } else {
    float *o = p.ws_o + (((int64_t)split * p.m_bs + orow) * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = 16 * db + 4 * lg;
      *reinterpret_cast<float4 *>(o + d) =
          make_float4(acc_o[db][0] * inv_l, acc_o[db][1] * inv_l, acc_o[db][2] * inv_l,
                      acc_o[db][3] * inv_l);
    }
    if (lg == 0) p.ws_lse[((int64_t)split * p.m_bs + orow) * p.hq + h] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: out = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, lse = M + ln(sum),
// splits taken in increasing order (deterministic).  Half a wavefront (32 lanes x 4 floats)
// per (slot, query head) row of D = 128 (D/4 lanes in general), all of a row's split loads
// issued before they are consumed.  Requests whose KV range fits one split were written
// directly by the main kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  constexpr int LPR = D / 4;            // lanes per row
  constexpr int RPB = 256 / LPR;        // rows per workgroup
  const int sub = threadIdx.x / LPR, l4 = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + sub;  // over n_bs * W * hq
  const int h = (int)(row % p.hq);
  const int64_t t = row / p.hq;
  const int j = (int)(t % p.W), i = (int)(t / p.W);
  if (i >= p.n_bs) return;
  int ki, off, c;
  int64_t kb;
  if (verify_request(p, i, ki, off, c, kb) || j >= ki) return;
  const int S = (c + ki + p.chunk - 1) / p.chunk;
  if (S <= 1) return;
  const int64_t plane = (int64_t)p.m_bs * p.hq;
  const int64_t rh = (int64_t)(off + j) * p.hq + h;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, p.ws_lse[s * plane + rh]);
  float den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 *src = reinterpret_cast<const float4 *>(p.ws_o + rh * D) + l4;
  const int64_t step4 = plane * D / 4;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float ls = p.ws_lse[s * plane + rh];
    const float wgt = ls == -INFINITY ? 0.f : __expf(ls - M);
    const float4 o = src[s * step4];
    den += wgt;
    num.x += wgt * o.x;
    num.y += wgt * o.y;
    num.z += wgt * o.z;
    num.w += wgt * o.w;
  }
  const float inv = 1.f / den;
  uint2 v;
  v.x = f32_to_bf16_bits(num.x * inv) | (f32_to_bf16_bits(num.y * inv) << 16);
  v.y = f32_to_bf16_bits(num.z * inv) | (f32_to_bf16_bits(num.w * inv) << 16);
  *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + rh * D + 4 * l4) = v;
  if (l4 == 0 && p.lse) p.lse[rh] = M + __logf(den);
}

// ---------------------------------------------------------------------------
// fp32 path (fp32 storage and arithmetic): one workgroup per (query row, head); keys in
// blocks of 256 with an online softmax.  Used for fp32 inputs, where the bf16 matrix cores
// do not apply; it is not on the bf16 hot path.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnParams p, int prefill) {
  __shared__ float sq[D];
  __shared__ float sw[256];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int h = blockIdx.x % p.hq;
  const int unit = blockIdx.x / p.hq;
  const int g = h / p.G;
  const float *kpool = static_cast<const float *>(p.k_pool);
  const float *vpool = static_cast<const float *>(p.v_pool);
  int c, j, off = 0;
  int64_t kb, qrow;
  const float *knew = nullptr, *vnew = nullptr;
  const float *qsrc;
  float *outp;
  float *lsep;
  if (!prefill) {
    const int i = unit / p.W;
    j = unit % p.W;
    if (i == 0 && j == 0) {
      int end = p.offsets[p.n_bs];
      end = end < 0 ? 0 : (end > p.m_bs ? p.m_bs : end);
      for (int e = tid; e < (p.m_bs - end) * D; e += 256)
        static_cast<float *>(p.out)[((int64_t)(end + e / D) * p.hq + h) * D + e % D] = 0.f;
      if (p.lse)
        for (int r = end + tid; r < p.m_bs; r += 256) p.lse[(int64_t)r * p.hq + h] = -INFINITY;
    }
    int ki;
    const int bad = verify_request(p, i, ki, off, c, kb);
    if (bad) {
      if (j == 0) {
        if (tid == 0 && h == 0) status_or(p.status, bad);
        if (ki >= 0 && ki <= p.W && off >= 0 && (int64_t)off + ki <= p.m_bs) {
          for (int e = tid; e < ki * D; e += 256)
            static_cast<float *>(p.out)[((int64_t)(off + e / D) * p.hq + h) * D + e % D] = 0.f;
          if (p.lse)
            for (int r = tid; r < ki; r += 256) p.lse[(int64_t)(off + r) * p.hq + h] = -INFINITY;
        }
      }
      return;
    }
    if (j >= ki) return;
    qrow = off + j;
    qsrc = static_cast<const float *>(p.q);
    outp = static_cast<float *>(p.out);
    lsep = p.lse;
    if (p.k_new) {
      knew = static_cast<const float *>(p.k_new);
      vnew = static_cast<const float *>(p.v_new);
      // this step's KV writes: one workgroup per candidate row and KV head
      if (h % p.G == 0 && tid < D) {
        const int64_t loc = p.slot_cache_loc[off + j];
        if (loc < 0 || loc >= p.pool_rows) {
          if (tid == 0) status_or(p.status, DSV_STATUS_POOL);
        } else {
          const int64_t src = ((int64_t)(off + j) * p.hkv + g) * D + tid;
          const int64_t dst = g * p.stride_head + loc * p.stride_row + tid;
          static_cast<float *>(p.k_pool)[dst] = knew[src];
          static_cast<float *>(p.v_pool)[dst] = vnew[src];
        }
      }
    }
  } else {
    const int r = unit / p.pf_max_len;
    j = unit % p.pf_max_len;
    int ql, qs;
    const int bad = prefill_request(p, r, ql, qs, c, kb);
    if (bad) {
      if (tid == 0 && j == 0 && h == 0) status_or(p.status, bad);
      return;
    }
    if (j >= ql) return;
    qrow = qs + j;
    qsrc = static_cast<const float *>(p.pf_q);
    outp = static_cast<float *>(p.pf_out);
    lsep = p.pf_lse;
  }
  for (int e = tid; e < D; e += 256) sq[e] = qsrc[(qrow * p.hq + h) * D + e];
  __syncthreads();
  const int n = c + j + 1;
  auto krow = [&](int pos) -> const float * {
    if (knew && pos >= c) return knew + ((int64_t)(off + pos - c) * p.hkv + g) * D;
    return kpool + g * p.stride_head + (kb + pos) * p.stride_row;
  };
  auto vrow = [&](int pos) -> const float * {
    if (vnew && pos >= c) return vnew + ((int64_t)(off + pos - c) * p.hkv + g) * D;
    return vpool + g * p.stride_head + (kb + pos) * p.stride_row;
  };
  float m = -INFINITY, l = 0.f, acc = 0.f;
  for (int base = 0; base < n; base += 256) {
    const int pos = base + tid;
    float z = -INFINITY;
    if (pos < n) {
      const float *kr = krow(pos);
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(sq[e], kr[e], s);
      z = s * p.scale;
    }
    // block max
    float v = z;
    for (int msk = 32; msk >= 1; msk >>= 1) v = fmaxf(v, __shfl_xor(v, msk));
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    const float mt = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m, mt);
    const float alpha = expf(m - m_new);
    const float wgt = pos < n ? expf(z - m_new) : 0.f;
    sw[tid] = wgt;
    v = wgt;
    for (int msk = 32; msk >= 1; msk >>= 1) v += __shfl_xor(v, msk);
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    const float lt = (red[0] + red[1]) + (red[2] + red[3]);
    l = l * alpha + lt;
    if (tid < D) {
      float a = acc * alpha;
      const int cnt = min(256, n - base);
      for (int u = 0; u < cnt; ++u) a = fmaf(sw[u], vrow(base + u)[tid], a);
      acc = a;
    }
    m = m_new;
    __syncthreads();
  }
  if (tid < D) outp[(qrow * p.hq + h) * D + tid] = acc / l;
  if (lsep && tid == 0) lsep[qrow * p.hq + h] = m + logf(l);
}

// Prefill KV writes: row j of request r -> pool row pf_kv_base[r] + pf_ctx[r] + j.
template <typename T>
__global__ __launch_bounds__(256) void prefill_kv_write_kernel(AttnParams p, int d) {
  const int64_t unit = blockIdx.x;  // (r, j, g)
  const int g = (int)(unit % p.hkv);
  const int64_t t = unit / p.hkv;
  const int j = (int)(t % p.pf_max_len), r = (int)(t / p.pf_max_len);
  int ql, qs, c;
  int64_t kb;
  if (prefill_request(p, r, ql, qs, c, kb) || j >= ql) return;
  const T *kn = static_cast<const T *>(p.pf_k_new), *vn = static_cast<const T *>(p.pf_v_new);
  T *kp = static_cast<T *>(p.k_pool), *vp = static_cast<T *>(p.v_pool);
  const int64_t src = ((int64_t)(qs + j) * p.hkv + g) * d;
  const int64_t dst = g * p.stride_head + (kb + c + j) * p.stride_row;
  for (int e = threadIdx.x; e < d; e += 256) {
    kp[dst + e] = kn[src + e];
    vp[dst + e] = vn[src + e];
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct Plan {
  int chunk = 0, n_splits = 0;
  size_t ws_o = 0, ws_lse = 0;  // bytes
};

// Split plan of the verification set: KV rows per split (multiple of 64) and the number of
// splits per request the grid provides.  Auto: aim for about two workgroups per CU (512)
// when every request sits at max_ctx.
static Plan make_plan(const dsv_attn_args *a) {
  Plan pl;
  if (a->n_bs <= 0 || a->dtype != DSV_BF16) return pl;
  const int64_t rows = (int64_t)a->max_ctx + a->W;
  int64_t chunk = a->kv_chunk;
  if (chunk <= 0) {
    const int64_t units = (int64_t)a->n_bs * a->hkv;
    int64_t target = (512 + units - 1) / units;
    if (target < 1) target = 1;
    if (target > 64) target = 64;
    chunk = (rows + target - 1) / target;
    chunk = (chunk + kTileKV - 1) / kTileKV * kTileKV;
    if (chunk < kTileKV) chunk = kTileKV;
  }
  pl.chunk = (int)chunk;
  pl.n_splits = (int)((rows + chunk - 1) / chunk);
  if (pl.n_splits < 1) pl.n_splits = 1;
  if (pl.n_splits > 1) {
    pl.ws_o = align256((size_t)pl.n_splits * a->m_bs * a->hq * a->d * sizeof(float));
    pl.ws_lse = align256((size_t)pl.n_splits * a->m_bs * a->hq * sizeof(float));
  }
  return pl;
}

template <int D, int NW>
static void launch_verify(const AttnParams &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW, false>), dim3(grid), dim3(NW * 64),
                     2 * kTileKV * D * sizeof(uint16_t), s, p);
}

template <int D>
static bool launch_verify_g(const AttnParams &p, int grid, hipStream_t s) {
  switch (p.G) {
    case 1: launch_verify<D, 1>(p, grid, s); return true;
    case 2: launch_verify<D, 2>(p, grid, s); return true;
    case 3: launch_verify<D, 3>(p, grid, s); return true;
    case 4: launch_verify<D, 4>(p, grid, s); return true;
    case 5: launch_verify<D, 5>(p, grid, s); return true;
    case 6: launch_verify<D, 6>(p, grid, s); return true;
    case 7: launch_verify<D, 7>(p, grid, s); return true;
    case 8: launch_verify<D, 8>(p, grid, s); return true;
    case 9: launch_verify<D, 9>(p, grid, s); return true;
    case 10: launch_verify<D, 10>(p, grid, s); return true;
    case 11: launch_verify<D, 11>(p, grid, s); return true;
    case 12: launch_verify<D, 12>(p, grid, s); return true;
    case 13: launch_verify<D, 13>(p, grid, s); return true;
    case 14: launch_verify<D, 14>(p, grid, s); return true;
    case 15: launch_verify<D, 15>(p, grid, s); return true;
    case 16: launch_verify<D, 16>(p, grid, s); return true;
    default: return false;
  }
}

static bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace dsv

extern "C" size_t dsv_verify_attn_workspace_bytes(const dsv_attn_args *a) {
  if (!a) return 0;
  dsv::Plan pl = dsv::make_plan(a);
  return pl.ws_o + pl.ws_lse;
}

extern "C" dsv_status dsv_verify_attn(const dsv_attn_args *a, hipStream_t stream) {
  using namespace dsv;
  if (!a || !a->status) return DSV_ERR_INVALID_ARG;
  if (a->dtype != DSV_BF16 && a->dtype != DSV_F32) return DSV_ERR_UNSUPPORTED;
  if (a->d != 64 && a->d != 128 && a->d != 256) return DSV_ERR_UNSUPPORTED;
  if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv) return DSV_ERR_INVALID_ARG;
  const int G = a->hq / a->hkv;
  if (a->dtype == DSV_BF16 && G > 16) return DSV_ERR_UNSUPPORTED;
  if (!a->k_pool || !a->v_pool || a->pool_rows < 0 || a->stride_row < a->d || a->stride_head < 0)
    return DSV_ERR_INVALID_ARG;
  const int64_t salign = a->dtype == DSV_BF16 ? 8 : 4;
  if (a->stride_row % salign || a->stride_head % salign) return DSV_ERR_INVALID_ARG;
  if (a->stride_head < a->pool_rows * a->stride_row && a->hkv > 1) return DSV_ERR_INVALID_ARG;
  if (a->n_bs < 0 || a->m_bs < 0 || a->n_pf < 0) return DSV_ERR_INVALID_ARG;
  const bool verify = a->n_bs > 0;
  const bool prefill = a->n_pf > 0;
  if (verify) {
    if (a->W < 1 || a->W > DSV_MAX_W || a->max_ctx < 0) return DSV_ERR_INVALID_ARG;
    if (!a->offsets || !a->k || !a->ctx_len || !a->kv_base || !a->q || !a->out)
      return DSV_ERR_INVALID_ARG;
    if ((a->k_new == nullptr) != (a->v_new == nullptr)) return DSV_ERR_INVALID_ARG;
    if (a->k_new && !a->slot_cache_loc) return DSV_ERR_INVALID_ARG;
    if (a->kv_chunk < 0 || a->kv_chunk % kTileKV) return DSV_ERR_INVALID_ARG;
  }
  if (prefill) {
    if (!a->pf_q_start || !a->pf_q_len || !a->pf_ctx_len || !a->pf_kv_base || !a->pf_q ||
        !a->pf_out || a->pf_max_len < 1 || a->pf_q_rows < 0)
      return DSV_ERR_INVALID_ARG;
    if ((a->pf_k_new == nullptr) != (a->pf_v_new == nullptr)) return DSV_ERR_INVALID_ARG;
  }
  // 16-byte vector access for bf16 tensors
  if (a->dtype == DSV_BF16) {
    const void *ptrs[] = {a->k_pool, a->v_pool, a->q, a->k_new, a->v_new, a->out,
                          a->pf_q,   a->pf_out, a->pf_k_new, a->pf_v_new};
    for (const void *ptr : ptrs)
      if (ptr && !aligned(ptr, 16)) return DSV_ERR_INVALID_ARG;
  }
  const Plan pl = make_plan(a);
  if (pl.ws_o + pl.ws_lse > 0 && (!a->workspace || a->workspace_bytes < pl.ws_o + pl.ws_lse ||
                                  !aligned(a->workspace, 16)))
    return DSV_ERR_WORKSPACE;

  AttnParams p{};
  p.k_pool = a->k_pool;
  p.v_pool = a->v_pool;
  p.pool_rows = a->pool_rows;
  p.stride_head = a->stride_head;
  p.stride_row = a->stride_row;
  p.hq = a->hq;
  p.hkv = a->hkv;
  p.G = G;
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / sqrtf((float)a->d);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.n_bs = a->n_bs;
  p.m_bs = a->m_bs;
  p.W = a->W;
  p.offsets = a->offsets;
  p.k = a->k;
  p.ctx_len = a->ctx_len;
  p.kv_base = a->kv_base;
  p.slot_cache_loc = a->slot_cache_loc;
  p.q = a->q;
  p.k_new = a->k_new;
  p.v_new = a->v_new;
  p.out = a->out;
  p.lse = a->lse;
  p.chunk = pl.chunk;
  p.n_splits = pl.n_splits;
  p.ws_o = pl.ws_o ? static_cast<float *>(a->workspace) : nullptr;
  p.ws_lse = pl.ws_o ? reinterpret_cast<float *>(static_cast<char *>(a->workspace) + pl.ws_o) : nullptr;
  p.n_pf = a->n_pf;
  p.pf_max_len = a->pf_max_len;
  p.pf_blocks = prefill ? (a->pf_max_len + kPfRows - 1) / kPfRows : 0;
  p.pf_q_rows = a->pf_q_rows;
  p.pf_q_start = a->pf_q_start;
  p.pf_q_len = a->pf_q_len;
  p.pf_ctx = a->pf_ctx_len;
  p.pf_kv_base = a->pf_kv_base;
  p.pf_q = a->pf_q;
  p.pf_k_new = a->pf_k_new;
  p.pf_v_new = a->pf_v_new;
  p.pf_out = a->pf_out;
  p.pf_lse = a->pf_lse;
  p.status = a->status;
  if (verify && a->dtype == DSV_F32) p.n_splits = 1, p.chunk = a->max_ctx + a->W;

  const int D = a->d;
  // ---- prefill path (wide tile) ----
  if (prefill) {
    if (a->pf_k_new) {
      const int64_t grid = (int64_t)a->n_pf * a->pf_max_len * a->hkv;
      if (a->dtype == DSV_BF16)
        hipLaunchKernelGGL(prefill_kv_write_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0,
                           stream, p, D);
      else
        hipLaunchKernelGGL(prefill_kv_write_kernel<float>, dim3((unsigned)grid), dim3(256), 0,
                           stream, p, D);
      DSV_LAUNCH_CHECK();
    }
    if (a->dtype == DSV_BF16) {
      const int64_t grid = (int64_t)p.pf_blocks * a->n_pf * a->hq;
      const size_t shm = 2 * kTileKV * D * sizeof(uint16_t);
      if (D == 64)
        hipLaunchKernelGGL((attn_bf16_kernel<64, kPfWaves, true>), dim3((unsigned)grid),
                           dim3(kPfWaves * 64), shm, stream, p);
      else if (D == 128)
        hipLaunchKernelGGL((attn_bf16_kernel<128, kPfWaves, true>), dim3((unsigned)grid),
                           dim3(kPfWaves * 64), shm, stream, p);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<256, kPfWaves, true>), dim3((unsigned)grid),
                           dim3(kPfWaves * 64), shm, stream, p);
    } else {
      const int64_t grid = (int64_t)a->n_pf * a->pf_max_len * a->hq;
      if (D == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p, 1);
      else if (D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p, 1);
      else
        hipLaunchKernelGGL(attn_f32_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, p, 1);
    }
    DSV_LAUNCH_CHECK();
  }
  // ---- verification path (16-row tile) ----
  if (verify) {
    if (a->main_begin && hipEventRecord(a->main_begin, stream) != hipSuccess) return DSV_ERR_HIP;
    if (a->dtype == DSV_BF16) {
      const int64_t grid = (int64_t)pl.n_splits * a->n_bs * a->hkv;
      bool ok = D == 64 ? launch_verify_g<64>(p, (int)grid, stream)
                        : D == 128 ? launch_verify_g<128>(p, (int)grid, stream)
                                   : launch_verify_g<256>(p, (int)grid, stream);
      if (!ok) return DSV_ERR_UNSUPPORTED;
    } else {
      const int64_t grid = (int64_t)a->n_bs * a->W * a->hq;
      if (D == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p, 0);
      else if (D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p, 0);
      else
        hipLaunchKernelGGL(attn_f32_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, p, 0);
    }
    DSV_LAUNCH_CHECK();
    if (a->main_end && hipEventRecord(a->main_end, stream) != hipSuccess) return DSV_ERR_HIP;
    if (a->dtype == DSV_BF16 && pl.n_splits > 1) {
      const int64_t rows = (int64_t)a->n_bs * a->W * a->hq;
      const int64_t grid = (rows + 256 / (D / 4) - 1) / (256 / (D / 4));
      if (D == 64)
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p);
      else if (D == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL(attn_combine_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, p);
      DSV_LAUNCH_CHECK();
    }
  }
  return DSV_OK;
}
