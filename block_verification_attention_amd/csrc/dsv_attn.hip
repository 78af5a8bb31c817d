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
// Prefill kernel: the same tile machinery with its waves stacked along the query rows of one
// head, in 128-row tiles (the hardware-selected wide tile of the pages) so that every KV tile
// staged in LDS feeds at least 128 query rows: at head_dim 128 eight waves of two 16-row query
// tiles each, i.e. two 128-row tiles sharing every staged KV tile (and every K and V operand
// a wave reads from LDS feeds two MFMAs); at head_dim 64 eight waves of one.
//
// LDS layouts (bf16), one K and one V tile per stage:
//   K [TILE][D]  row-major; 16-byte column slots XOR-swizzled by (row & 15) so that the 16
//                rows an MFMA operand read touches fall in distinct banks.
//   V [TILE][D]  row-major; 32-byte column blocks XOR-swizzled by (row & 7), read with the
//                transposing LDS loads that form the P.V operand (keys along its K dimension).
#include <math.h>

#include <atomic>
#include <type_traits>

#include <hip/hip_ext.h>

#include "dsv_internal.h"

namespace dsv {

constexpr int kTileKV = 64;  // split granularity (multiple of every tile height)
constexpr int kXcds = 8;     // dispatch places block b on XCD b % 8
// Waves with at most this many 16-byte loads per tile stage two tiles in registers (more
// would push the hot shapes past the register budget of two waves per SIMD).
constexpr int kTwoSetMaxLoads = 4;
// Prefill: 8 waves per workgroup at every head_dim, two per SIMD, and 16-row query tiles per
// wave (two at head_dim 64 and 128: two 128-row tiles per workgroup; one at 256: one 128-row
// tile).  With two query tiles a wave's every K and V operand read from LDS feeds two MFMAs;
// at head_dim 256 one tile's 16 x 256 output and query fragments fill most of a wave's share
// of the register file.
constexpr int pf_qtiles(int D) { return D <= 128 ? 2 : 1; }
constexpr int pf_waves(int) { return 8; }
constexpr int pf_rows(int D) { return pf_waves(D) * 16 * pf_qtiles(D); }
// Prefill KV tile rows at head_dim 128 (the two query tiles double the score registers).
constexpr int kPfTile128 = 32;

struct AttnParams {
  void *k_pool, *v_pool;
  int64_t pool_rows, stride_head, stride_row;
  int hq, hkv, G;
  int GW, HG;        // verification: query heads per workgroup, head groups per KV head
  int xcd_sib_v;     // verification: HG sibling workgroups share an XCD (0: plain order)
  int xcd_sib_pf;    // prefill: the G query heads of a KV head share an XCD (0: plain order)
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
  uint16_t *ws_o;       // [n_splits][m_bs][hq][D] bf16 split outputs
  float *ws_lse;        // [n_splits][m_bs][hq]
  // prefill set
  int n_pf, pf_blocks, pf_q_rows, pf_max_len;
  const int32_t *pf_q_start, *pf_q_len, *pf_ctx;
  const int64_t *pf_kv_base;
  const void *pf_q, *pf_k_new, *pf_v_new;
  void *pf_out;
  float *pf_lse;
  int32_t *status;
  // token-granular cache map of the verification set (null: contiguous segments)
  const int32_t *kv_index;
  int64_t kv_index_stride;
  // packer fused into the verification launch (pk_offsets non-null): the kernel forms the
  // offsets itself and writes the packer's outputs; `offsets` then points at pk_offsets
  const int32_t *pk_tokens;
  int32_t *pk_offsets, *pk_req, *pk_tok, *pk_pos;
  int64_t *pk_loc;
};

// Checks request i of the verification set; on success returns 0 and its fields.
__device__ __forceinline__ int verify_request(const AttnParams &p, int i, int &ki, int &off, int &c,
                                              int64_t &kb) {
  ki = p.k[i];
  off = p.offsets[i];
  c = p.ctx_len[i];
  kb = p.kv_index ? 0 : p.kv_base[i];
  if (ki < 0 || ki > p.W || off < 0 || (int64_t)off + ki > p.m_bs || c < 0)
    return DSV_STATUS_BAD_REQUEST;
  if (p.kv_index) return (int64_t)c + ki > p.kv_index_stride ? DSV_STATUS_BAD_REQUEST : 0;
  if (kb < 0) return DSV_STATUS_BAD_REQUEST;
  if (kb + c + ki > p.pool_rows) return DSV_STATUS_POOL;
  return 0;
}

// Pool row of position pos of a verification request: its contiguous segment (kb + pos), or
// with a cache map (kvi = the request's row of kv_index) the mapped row; a mapped row outside
// the pool flags the status word and reads the nearest pool row instead.
__device__ __forceinline__ int64_t mapped_row(const AttnParams &p, const int32_t *kvi, int64_t kb, int pos) {
  if (!kvi) return kb + pos;
  int64_t r = gload<int32_t>(kvi + pos);
  if (r < 0 || r >= p.pool_rows) {
    status_or(p.status, DSV_STATUS_POOL);
    r = r < 0 ? 0 : p.pool_rows - 1;
  }
  return r;
}

// Splits of a verification request with n_vis visible positions: floor(n_vis / chunk) of them
// (at least one, at most the planned count); split s covers [s * chunk, (s + 1) * chunk) and
// the last one also takes the remainder, so every split has at least `chunk` rows and at most
// the last is longer.
__device__ __forceinline__ int verify_splits(const AttnParams &p, int n_vis) {
  int s = n_vis / p.chunk;
  s = s < 1 ? 1 : s;
  return s > p.n_splits ? p.n_splits : s;
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
    gstore(out + ((int64_t)r * hq + h0 + hh) * D + cc * 8, u32x4{0u, 0u, 0u, 0u});
  }
  if (lse)
    for (int64_t e = tid; e < (int64_t)(r1 - r0) * nh; e += nt)
      gstore(lse + (int64_t)(r0 + e / nh) * hq + h0 + e % nh, -INFINITY);
}

// ---------------------------------------------------------------------------
// KV staging.  Each wave loads its share of a tile from HBM into registers (16 bytes per lane,
// consecutive lanes on consecutive bytes of a row, non-temporal: the KV is streamed once) and
// later stores it to an LDS stage with the XOR swizzle applied on the LDS side.  Two register
// sets and two LDS stages keep two tiles in flight while a third is consumed; the compiler
// tracks completion of the register loads.  (Direct global->LDS loads, measured on the same
// access pattern, sustained about 12% less bandwidth than loads through registers.)
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
struct Piece {  // 16 staged bytes
  uint32_t a, b, c, d;
};

// LDS tile layouts: row-major [TILE][D] bf16 for both K and V, 16-byte column slots permuted
// per row.  K: slot ^ (row & 15) -- the 16 rows of an MFMA operand read (one slot each) land
// in distinct banks.  V: slot ^ 2*(row & 7) (a permutation of 32-byte blocks) -- the four
// rows x 32 bytes that a 16-lane group touches in a transposing read land in distinct banks.
template <int D>
__device__ __forceinline__ int k_slot(int row, int slot) {
  constexpr int SW = (D / 8) < 16 ? (D / 8) : 16;
  return slot ^ (row & (SW - 1));
}
template <int D>
__device__ __forceinline__ int v_slot(int row, int slot) {
  constexpr int VB = D / 16;  // 32-byte blocks per row
  constexpr int M = VB < 8 ? VB : 8;
  return slot ^ (2 * (row & (M - 1)));
}

typedef __attribute__((address_space(3))) uint4 lds_u4;
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Lazy reference-max threshold (log2 units): the softmax reference only moves when a tile's
// maximum exceeds it by more than this, so the probabilities stay below 2^8 and the output
// accumulators are rarely rescaled.  The result is unchanged: numerator and denominator use
// the same reference.
constexpr float kRescaleSlack = 8.0f;

// ---------------------------------------------------------------------------
// bf16 MFMA attention kernel.  PF = false: verification (NW = G waves, one 16-row query
// tile per query head, split KV).  PF = true: prefill (NW waves of QT 16-row query tiles
// along the query rows of one head).  KV tiles of TILE rows stream through an LDS ring.
// ---------------------------------------------------------------------------
template <int D, int NW, bool PF>
constexpr int waves_per_eu_hint() {
  // small workgroups get the whole register file; 3..8 waves are asked to fit 2 waves/SIMD,
  // and at head_dim 128 and 256 exactly 2 (a third wave per SIMD cannot host another
  // workgroup of this size, and tighter register budgets cost the tile loop its loads in
  // flight); head_dim-64 kernels may run more per SIMD
  return NW <= 2 ? 1 : (NW <= 8 ? 2 : 1);
}

template <int D, int NW, bool PF, int TILE, int HV, bool MAP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(waves_per_eu_hint<D, NW, PF>(), waves_per_eu_hint<D, NW, PF>() == 2 && D >= 128 ? 2 : 10))) void attn_bf16_kernel(AttnParams p) {
  constexpr int RPC = 1024 / (2 * D);        // rows per 1 KB wave load
  constexpr int NCK = TILE / RPC;            // wave loads per tensor per tile
  constexpr int NP = 2 * NCK * HV;           // wave loads per stage (HV tiles of K and V)
  constexpr int QPW = (NP + NW - 1) / NW;    // wave loads per wave per stage (at most)
  constexpr int RSETS = (!PF && QPW <= kTwoSetMaxLoads) ? 2 : 1;  // register sets (stages in flight besides LDS)
  constexpr int SUB_BYTES = 2 * TILE * D * 2;  // one tile of K and V
  constexpr int STAGE_BYTES = HV * SUB_BYTES;
  constexpr int NWH = NW / HV;               // waves per KV half
  static_assert(!PF || HV == 1, "prefill stacks its waves along the query rows");
  static_assert(!PF || !MAP, "the cache map applies to the verification set");
  static_assert(NW % HV == 0, "wave halves");
  constexpr int DB = D / 16;
  constexpr int KS = D / 32;
  constexpr int QT = PF ? pf_qtiles(D) : 1;  // 16-row query tiles per wave
  static_assert(QT == 1 || HV == 1, "two query tiles: prefill only");
  static_assert(TILE % 32 == 0 && TILE % RPC == 0, "tile shape");

  extern __shared__ __align__(16) uint16_t lds[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int lq = lane & 15, lg = lane >> 4;
  // KV half of this wave (HV = 2: waves [0, NWH) consume the even tiles of each stage pair,
  // waves [NWH, NW) the odd ones, for the same query heads) and its head within the group
  const int half = HV == 1 ? 0 : w / NWH;
  const int wh = HV == 1 ? w : w - half * NWH;  // head within the workgroup's heads

  // ---- work unit ----
  int g, h, c, r_lo, r_hi, row0, nrows, split = 0, n_splits_i = 1, off = 0, hg = 0;
  // verification: query row of this lane's column and whether its head slot exists
  int col_row = 0;
  bool col_ok = true, wave_has_heads = true;
  int64_t kb, q_row0;
  const uint16_t *qsrc;
  const uint16_t *knew = nullptr, *vnew = nullptr;
  const int32_t *kvi = nullptr;  // the request's cache-map row (verification with a cache map)
  if constexpr (!PF) {
    // Workgroups that read the same KV rows (the HG head groups of a (request, KV head,
    // split)) are consecutive blocks on one XCD, so that they run together and share its L2:
    // blocks go to XCD b % 8, so siblings are b, b + 8, ... (grid a multiple of 8 HG).
    // The KV head of unit u (u / hkv numbers the rest; the unit's XCD is u % 8 in both orders):
    // with hkv dividing 8 it moves on by one every 8 units, so that each XCD streams every KV
    // head's pool region in turn rather than one head's only (with one head per XCD, the XCDs
    // reading some heads' regions ran their tile loops up to ~12% longer).
    auto unit_kv_head = [&](int u) __attribute__((always_inline)) {
      return kXcds % p.hkv == 0 ? (u % p.hkv + u / kXcds) % p.hkv : u % p.hkv;
    };
    int bid = blockIdx.x, t0;
    if (p.xcd_sib_v) {
      const int slot = bid / kXcds;
      hg = slot % p.HG;
      const int u = (slot / p.HG) * kXcds + bid % kXcds;
      g = unit_kv_head(u);
      t0 = u / p.hkv;
    } else {
      g = unit_kv_head(bid);
      t0 = bid / p.hkv;
      hg = t0 % p.HG;  // this workgroup's query heads: [G g + GW hg, + GW)
      t0 /= p.HG;
    }
    // With fewer KV heads than XCDs a unit's XCD follows its position t0 % n_bs, and with n_bs
    // a multiple of 8 / hkv it ignores the split, so every split of a request lands on the
    // same XCD and ragged contexts leave some XCDs far more rows than others (1.7x on the
    // 32-request head_dim-256 set).  There, position t0 % n_bs of split t0 / n_bs holds
    // request (t0 + split) % n_bs: the requests rotate by one position per split.  With 8 or
    // more KV heads every XCD already serves one KV head of every (request, split).
    split = t0 / p.n_bs;
    const int i = p.hkv < kXcds ? (t0 % p.n_bs + split) % p.n_bs : t0 % p.n_bs;
    const int h0 = g * p.G + hg * p.GW;
    h = h0 + wh;
    int ki, bad, end;
    if (p.pk_offsets) {
      // Packer fused into this launch (the flat-buffer packer's rule, as dsv_pack_slots): the
      // effective lengths are k_r for well-formed requests, else 0, and all 0 when they sum
      // above m_bs; offset_i is their exclusive sum.  Every wavefront forms its request's
      // offset and the total itself (lanes over the requests, shuffle sums: no barrier), with
      // the request's own fields loaded alongside; the first workgroup of each request writes
      // that request's packer outputs, request 0's also the tail.
      c = p.ctx_len[i];
      kb = p.kv_base[i];
      const int k_i = p.k[i];
      int s_all = 0, s_before = 0;
      for (int r0 = 0; r0 < p.n_bs; r0 += kWave) {
        const int r = r0 + lane;
        const int e = r < p.n_bs ? pack_effective_length(p.k[r], p.ctx_len[r], p.kv_base[r], p.W) : 0;
        s_all += e;
        s_before += r < i ? e : 0;
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        s_all += __shfl_xor(s_all, d);
        s_before += __shfl_xor(s_before, d);
      }
      const bool drop_all = s_all > p.m_bs;
      ki = drop_all ? 0 : pack_effective_length(k_i, c, kb, p.W);
      off = drop_all ? 0 : s_before;
      end = drop_all ? 0 : s_all;
      if (split == 0 && g == 0 && hg == 0) {
        for (int j = tid; j < ki; j += NW * 64) {  // slot off + j: candidate j of request i
          p.pk_req[off + j] = i;
          p.pk_tok[off + j] = p.pk_tokens[(int64_t)i * p.W + j];
          p.pk_pos[off + j] = c + j;
          p.pk_loc[off + j] = kb + c + j;
        }
        if (tid == 0) {
          p.pk_offsets[i] = off;
          if (!pack_request_ok(k_i, c, kb, p.W)) status_or(p.status, DSV_STATUS_BAD_REQUEST);
          if (i == 0) {
            p.pk_offsets[p.n_bs] = end;
            if (drop_all) status_or(p.status, DSV_STATUS_BUDGET);
          }
        }
        if (i == 0)
          for (int sl = end + tid; sl < p.m_bs; sl += NW * 64) {
            p.pk_req[sl] = -1;
            p.pk_tok[sl] = 0;
            p.pk_pos[sl] = 0;
            p.pk_loc[sl] = -1;
          }
      }
      bad = ki > 0 && kb + c + ki > p.pool_rows ? DSV_STATUS_POOL : 0;
    } else {
      end = p.offsets[p.n_bs];
      end = end < 0 ? 0 : (end > p.m_bs ? p.m_bs : end);
      bad = verify_request(p, i, ki, off, c, kb);
    }
    if (i == 0 && split == 0)
      zero_rows_bf16<D>(static_cast<uint16_t *>(p.out), p.lse, p.hq, end, p.m_bs, h0,
                        min(p.GW, p.G - hg * p.GW), tid, NW * 64);
    if (bad) {
      if (split == 0) {
        if (tid == 0 && g == 0 && hg == 0) status_or(p.status, bad);
        if (ki >= 0 && ki <= p.W && off >= 0 && (int64_t)off + ki <= p.m_bs)
          zero_rows_bf16<D>(static_cast<uint16_t *>(p.out), p.lse, p.hq, off, off + ki, h0,
                            min(p.GW, p.G - hg * p.GW), tid, NW * 64);
      }
      return;
    }
    const int n_vis = c + ki;
    n_splits_i = verify_splits(p, n_vis);
    if (ki == 0 || split >= n_splits_i) return;
    if (MAP) kvi = p.kv_index + (int64_t)i * p.kv_index_stride;
    // the candidate block costs about one tile: the last split hands one committed tile to
    // the split before it
    const int shift = (n_splits_i >= 2 && n_vis - (n_splits_i - 1) * p.chunk >= 2 * kTileKV + ki) ? kTileKV : 0;
    r_lo = split * p.chunk + (split == n_splits_i - 1 ? shift : 0);
    r_hi = split == n_splits_i - 1 ? n_vis : r_lo + p.chunk + (split == n_splits_i - 2 ? shift : 0);
    row0 = 0;
    nrows = ki;
    q_row0 = off;
    qsrc = static_cast<const uint16_t *>(p.q);
    // Head packing: the 16 columns of a wave's tile are independent (query head, row) pairs
    // that share the K and V operands.  The request's G k_i pairs of this KV head, pair
    // p = head k_i + row, fill the columns of the workgroup's waves in order (wave w takes
    // pairs 16 w .. 16 w + 15), so that a wave's tile holds rows of several heads when k_i < 16
    // and waves past the last pair skip the tile arithmetic.  Where a KV head's query heads
    // are spread over several workgroups (HG > 1), the pairs are split as evenly as possible
    // over ceil(G k_i / (16 waves)) workgroups and the grid's other head-group workgroups of the
    // request leave, so that fewer of them stream its KV rows.  (With HG = 1 the host plan
    // gives every workgroup at least ceil(G k_i / 16) <= G waves, so all pairs fit.)
    const int pairs = p.G * ki;
    int pb = 0, pe = pairs;  // this workgroup's pairs
    if (p.HG > 1) {
      const int cap = NWH * 16;
      const int hgr = (pairs + cap - 1) / cap;
      if (hg >= hgr) return;
      const int per = (pairs + hgr - 1) / hgr;
      pb = hg * per;
      pe = min(pairs, pb + per);
    }
    const int pr = pb + wh * 16 + lq;  // this lane's pair
    col_ok = pr < pe;
    col_row = col_ok ? pr % ki : 0;
    wave_has_heads = pb + wh * 16 < pe;
    h = g * p.G + (col_ok ? pr / ki : 0);
    if (p.k_new) {
      knew = static_cast<const uint16_t *>(p.k_new);
      vnew = static_cast<const uint16_t *>(p.v_new);
    }
  } else {
    // The G query heads of a (request, KV head, row block) read the same KV tiles: with
    // xcd_sib_pf they are consecutive blocks on one XCD (grid a multiple of 8 G).
    // Block i runs on XCD i % 8.  With fewer than 8 heads per request in the order below and
    // a multiple of 8 units per row block, every row block of a request would land on the same
    // XCDs, so ragged lengths would load a few XCDs only: then request r of row block j is
    // taken by the slot of request (r - j) mod n_pf, which walks each request over the XCDs.
    int bid = blockIdx.x, b, r;
    if (p.xcd_sib_pf) {
      const int slot = bid / kXcds;
      const int hig = slot % p.G;
      const int u = (slot / p.G) * kXcds + bid % kXcds;  // (row block, request, KV head)
      const int per_u = p.n_pf * p.hkv, j = u / per_u;
      b = p.pf_blocks - 1 - j;  // longest row blocks first
      r = (u % per_u) / p.hkv;
      if (p.hkv < kXcds) r = (r + j) % p.n_pf;
      g = u % p.hkv;
      h = g * p.G + hig;
    } else {
      const int per = p.n_pf * p.hq, j = bid / per;
      b = p.pf_blocks - 1 - j;  // longest row blocks first
      r = (bid % per) / p.hq;
      if (p.hq < kXcds) r = (r + j) % p.n_pf;
      h = (bid % per) % p.hq;
      g = h / p.G;
    }
    int ql, qs;
    const int bad = prefill_request(p, r, ql, qs, c, kb);
    if (bad) {
      if (tid == 0 && b == 0 && h == 0) status_or(p.status, bad);
      return;
    }
    row0 = b * (NW * 16 * QT);
    if (row0 >= ql) return;
    nrows = ql;
    r_lo = 0;
    r_hi = c + min(row0 + NW * 16 * QT, ql);
    q_row0 = qs;
    qsrc = static_cast<const uint16_t *>(p.pf_q);
  }
  (void)n_splits_i;

  // ---- query fragment (B operand of S^T = K Q^T): row lq, columns 32ks + 8lg .. +7 ----
  // query row index within the request of this lane's column in query tile 0 (tile qt: + 16 qt)
  const int my_row0 = PF ? row0 + w * 16 * QT + lq : col_row;
  bf16x8 qf[QT][KS];
  int lim[QT];  // last visible position of this lane's query row in each tile
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int my_row = my_row0 + 16 * qt;
    const bool ok = my_row < nrows && col_ok;
    const uint16_t *qp = qsrc + ((q_row0 + (ok ? my_row : 0)) * p.hq + h) * (int64_t)D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = ok ? gload<u32x4>(qp + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
      qf[qt][ks] = __builtin_bit_cast(bf16x8, v);
    }
    lim[qt] = c + my_row;
  }

  // ---- tile loads: wave w moves pieces q = w, w + NW, ... of the 2 * NCK per tile (piece q
  // < NCK: K rows RPC q .. + RPC - 1, else the same rows of V; 16 bytes per lane) ----
  const int64_t row_elems = p.stride_row;
  const uint32_t row_bytes = (uint32_t)(row_elems * 2);
  const uint16_t *kseg = static_cast<const uint16_t *>(p.k_pool) + g * p.stride_head + kb * row_elems;
  const uint16_t *vseg = static_cast<const uint16_t *>(p.v_pool) + g * p.stride_head + kb * row_elems;
  // Verification: the tile loop covers the committed rows [r_lo, t_hi) from the pool; the
  // candidate positions [c, c + k_i) (all in the request's last split) form a separate
  // candidate block, staged with the first tile and consumed before the loop, so the split
  // that holds them runs no extra pipeline iteration.  Prefill: the loop covers everything.
  const bool has_cand = !PF && r_hi > c;
  const int t_hi = has_cand ? c : r_hi;
  // Piece q of a stage: tile q / (2 NCK) of the stage, K if q % (2 NCK) < NCK else V, rows
  // RPC (q % NCK) ..  With NCK a multiple of NW every wave moves the same pattern (which tile,
  // K or V, and no piece past the stage: decided at compile time).
  constexpr bool EVEN = NCK % NW == 0;
  auto piece_sub = [&](int u) __attribute__((always_inline)) {
    return EVEN ? u / (2 * NCK / NW) : (w + u * NW) / (2 * NCK);
  };
  auto piece_is_v = [&](int u) __attribute__((always_inline)) {
    return EVEN ? u % (2 * NCK / NW) >= NCK / NW : (w + u * NW) % (2 * NCK) >= NCK;
  };
  auto piece_exists = [&](int u) __attribute__((always_inline)) {
    return EVEN || w + u * NW < NP;
  };
  // row of piece u within its tile
  auto piece_row = [&](int u) __attribute__((always_inline)) {
    return ((w + u * NW) % NCK) * RPC + lane / (D / 8);
  };
  uint32_t goff[QPW], loff[QPW];  // byte offsets in a pool stage / in an LDS stage
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const bool isv = piece_is_v(u);
    const int sub = piece_sub(u);
    const int row = piece_row(u);
    const int slot = lane % (D / 8);
    goff[u] = (sub * TILE + row) * row_bytes + 16 * slot;
    loff[u] = sub * SUB_BYTES + (isv ? TILE * D * 2 : 0) + row * (2 * D) +
              16 * (isv ? v_slot<D>(row, slot) : k_slot<D>(row, slot));
  }
  // Each piece's address is chosen first (interior tiles: the pool segment plus a lane
  // constant; boundary tiles: per-lane rows that may come from k_new or be clamped), then one
  // load per piece; the staged data is kept as scalars so that it never forms one wide vector
  // register.
  const char *kpool_g = static_cast<const char *>(p.k_pool) + g * p.stride_head * 2;
  const char *vpool_g = static_cast<const char *>(p.v_pool) + g * p.stride_head * 2;
  // Cache map (MAP): the map entries of the next stage's rows are fetched when a stage's data
  // loads go out (stages are loaded in order), so a stage's data loads never wait for their
  // own map entries.
  int32_t map_next[MAP ? QPW : 1];
  int map_next_base = -1;
  auto fetch_map = [&](int tile_base) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      int pos = tile_base + piece_sub(u) * TILE + piece_row(u);
      pos = pos < t_hi ? pos : t_hi - 1;
      map_next[u] = gload<int32_t>(kvi + pos);
    }
    map_next_base = tile_base;
  };
  auto tile_srcs = [&](int tile_base, const char *(&src)[QPW]) __attribute__((always_inline)) {
    if constexpr (MAP) {  // cache map: every row through its mapped pool row
      if (map_next_base != tile_base) fetch_map(tile_base);
#pragma unroll
      for (int u = 0; u < QPW; ++u) {
        int64_t r = map_next[u];
        if (r < 0 || r >= p.pool_rows) {
          status_or(p.status, DSV_STATUS_POOL);
          r = r < 0 ? 0 : p.pool_rows - 1;
        }
        src[u] = (piece_is_v(u) ? vpool_g : kpool_g) + r * row_bytes + 16 * (lane % (D / 8));
      }
    } else if (tile_base + HV * TILE <= t_hi) {
      const char *kt = reinterpret_cast<const char *>(kseg) + (size_t)tile_base * row_bytes;
      const char *vt = reinterpret_cast<const char *>(vseg) + (size_t)tile_base * row_bytes;
#pragma unroll
      for (int u = 0; u < QPW; ++u) src[u] = (piece_is_v(u) ? vt : kt) + goff[u];
    } else {
#pragma unroll
      for (int u = 0; u < QPW; ++u) {
        const bool isv = piece_is_v(u);
        int pos = tile_base + piece_sub(u) * TILE + piece_row(u);
        pos = pos < t_hi ? pos : t_hi - 1;  // rows past the range re-read a visible row (masked)
        const uint16_t *r = (isv ? vseg : kseg) + (int64_t)pos * row_elems;
        src[u] = reinterpret_cast<const char *>(r + 8 * (lane % (D / 8)));
      }
    }
  };
  auto load_tile = [&](int tile_base, Piece (&x)[QPW]) __attribute__((always_inline)) {
    const char *src[QPW];
    tile_srcs(tile_base, src);
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      if (piece_exists(u)) {
        const u32x4 v = gload_stream<u32x4>(src[u]);
        x[u] = Piece{v[0], v[1], v[2], v[3]};
      }
    }
    if constexpr (MAP) {
      if (tile_base + HV * TILE < t_hi) fetch_map(tile_base + HV * TILE);
    }
  };
  auto store_tile = [&](const Piece (&x)[QPW], int stage) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < QPW; ++u)
      if (piece_exists(u))
        *(lds_u32x4 *)(uintptr_t)(lds_base + stage * STAGE_BYTES + loff[u]) =
            u32x4{x[u].a, x[u].b, x[u].c, x[u].d};
  };
  // Stores the staged tile to LDS stage `stage` and refills each piece with the next tile's
  // piece as soon as that piece is stored, so that the next tile's loads leave while the rest
  // of this tile is still arriving (the scheduling barrier keeps each store-load pair in
  // order; waits for the data are counted per piece).
  auto store_load_tile = [&](Piece (&x)[QPW], int stage, int next_base) __attribute__((always_inline)) {
    const char *src[QPW];
    tile_srcs(next_base, src);
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      if (piece_exists(u)) {
        *(lds_u32x4 *)(uintptr_t)(lds_base + stage * STAGE_BYTES + loff[u]) =
            u32x4{x[u].a, x[u].b, x[u].c, x[u].d};
        const u32x4 v = gload_stream<u32x4>(src[u]);
        x[u] = Piece{v[0], v[1], v[2], v[3]};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MAP) {
      if (next_base + HV * TILE < t_hi) fetch_map(next_base + HV * TILE);
    }
  };

  // ---- lane-constant LDS operand offsets ----
  // K (A operand of S^T): row 16kb + lq, slot 4ks + lg
  uint32_t koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    koff[ks] = lds_base + half * SUB_BYTES + lq * (2 * D) + k_slot<D>(lq, 4 * ks + lg) * 16;
  // V (transposing reads): row R + lq/4 with R = 32kk + 16half + 4lg, 8 bytes at column
  // 16db + 4(lq%4); the row term 32kk + 16half does not change the swizzle
  uint32_t voffs[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int row = 4 * lg + (lq >> 2);
    voffs[db] = lds_base + half * SUB_BYTES + TILE * D * 2 + row * (2 * D) +
                 v_slot<D>(row, 2 * db + ((lq & 3) >> 1)) * 16 + 8 * (lq & 1);
  }

  f32x4 acc_o[QT][DB];
  float m_ref[QT], l_run[QT];  // reference max (log2 units) and row-sum partial
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_o[qt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_ref[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  const int n_tiles = (t_hi - r_lo + HV * TILE - 1) / (HV * TILE);  // stages of HV tiles
  const int wave_row_lo = PF ? row0 + w * 16 * QT : 0;  // first query row of the wave
  constexpr int WROWS = 16 * QT;                        // query rows per wave
  const bool wave_live = wave_row_lo < nrows && wave_has_heads;
  const float sl2 = p.scale_log2;

  // S^T blocks of one tile from LDS stage STAGE: acc_s[qt][kb][e] = raw score of KV row
  // base + 16kb + 4lg + e for query row lq of query tile qt (KB = the tile's rows / 16); each
  // K operand read feeds the QT query tiles
  auto tile_qk = [&](auto stage_c, auto &acc_s) __attribute__((always_inline)) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr int KB = std::extent<std::remove_reference_t<decltype(acc_s)>, 1>::value;
#pragma unroll
    for (int kbk = 0; kbk < KB; ++kbk) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) acc_s[qt][kbk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t a_addr = koff[ks] + STAGE * STAGE_BYTES + 16 * kbk * (2 * D);
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(lds_u4 *)(uintptr_t)a_addr);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          acc_s[qt][kbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qt][ks], acc_s[qt][kbk], 0, 0, 0);
      }
    }
  };
  // Online softmax of those scores and P.V from the same stage.  With mask_c (a compile-time
  // constant or a wave-uniform flag), positions at or past hi or past the row's last visible
  // position are excluded; `mid` runs between the row maximum and the exponentials (the
  // prefill loop puts the next tile's Q.K products there).
  auto tile_softmax_pv = [&](int base, int hi, auto stage_c, auto mask_c, auto &acc_s, auto &&mid) __attribute__((always_inline)) {
    constexpr int STAGE = decltype(stage_c)::value;
    const bool masked = mask_c;  // a compile-time constant, or a wave-uniform flag
    constexpr int KB = std::extent<std::remove_reference_t<decltype(acc_s)>, 1>::value;
    constexpr int KK = KB / 2;  // 32-row P.V steps
    float m_use[QT];
    // transposing reads: lane j of each 16-lane group receives V[R + t][16db + j], t < 4, from
    // the 8-byte chunks that lanes j/4 + 4t point at (rows R + lq/4, columns 16db + 4(lq%4));
    // R = 32kk + 16half + 4lg.  Each V operand feeds the QT query tiles.
    auto v_operand = [&](int kk, int db) __attribute__((always_inline)) {
      const uint32_t v0 = voffs[db] + STAGE * STAGE_BYTES + (32 * kk) * (2 * D);
      const auto lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(uintptr_t)v0);
      const auto hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(uintptr_t)(v0 + 16 * (2 * D)));
      bf16x8 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = lo[e];
        a[4 + e] = hi[e];
      }
      return a;
    };
    // prefill (one 32-row step per tile) up to head_dim 128: the tile's V operands are read
    // first, so that their LDS latency runs behind the row maximum, the next tile's Q.K and
    // the exponentials.  At head_dim 256 they would take 64 more registers than two waves per
    // SIMD leave, so they are read where used.
    constexpr bool VREAD = PF && D <= 128;
    constexpr int VPRE = VREAD ? KK * DB : 1;
    bf16x8 va[VPRE];
    if constexpr (VREAD) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int db = 0; db < DB; ++db) va[kk * DB + db] = v_operand(kk, db);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if (masked) {
#pragma unroll
        for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pos = base + 16 * kbk + 4 * lg + e;
            acc_s[qt][kbk][e] = (pos < hi && pos <= lim[qt]) ? acc_s[qt][kbk][e] : -INFINITY;
          }
      }
      float mt = -INFINITY;  // this lane's maximum over its entries of the row
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk)
#pragma unroll
        for (int e = 0; e < 4; ++e) mt = fmaxf(mt, acc_s[qt][kbk][e]);
      // The reference moves only when some entry of a row exceeds it by more than the slack.
      // Whether any does is decided per lane (a ballot); the row maximum over the four lanes
      // holding the row is formed only then.
      if (__builtin_expect(__any(mt * sl2 > m_ref[qt] + kRescaleSlack), 0)) {
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mt2 = mt * sl2;  // row maximum of the tile in log2 units (-inf if masked)
        const float m_new = mt2 > m_ref[qt] + kRescaleSlack ? mt2 : m_ref[qt];
        // rows that have seen no visible key yet hold zeros: their factor is 0 (not NaN)
        const float alpha = m_ref[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[qt] - m_new);
        m_ref[qt] = m_new;
        l_run[qt] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc_o[qt][db] *= alpha;
      }
      m_use[qt] = m_ref[qt] == -INFINITY ? 0.f : m_ref[qt];
    }
    mid();
    // P (bf16) is the B operand of O^T = V^T P^T; the row sum accumulates the fp32 values
    uint32_t pb[QT][KB][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kbk = 0; kbk < KB; ++kbk) {
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc_s[qt][kbk][e], sl2, -m_use[qt]));
          l_run[qt] += pe[e];
        }
        pb[qt][kbk][0] = cvt_pk_bf16(pe[0], pe[1]);
        pb[qt][kbk][1] = cvt_pk_bf16(pe[2], pe[3]);
      }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 b[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        b[qt] = __builtin_bit_cast(bf16x8, make_uint4(pb[qt][2 * kk][0], pb[qt][2 * kk][1],
                                                      pb[qt][2 * kk + 1][0], pb[qt][2 * kk + 1][1]));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 a;
        if constexpr (VREAD)
          a = va[kk * DB + db];
        else
          a = v_operand(kk, db);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          acc_o[qt][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[qt], acc_o[qt][db], 0, 0, 0);
      }
    }
  };
  // One tile of ROWS (TILE, or 32 for the candidate block) KV rows at positions base.. from
  // LDS stage STAGE; with mask_c, positions at or past hi or past the row's last visible
  // position are excluded.
  auto compute_tile = [&](int base, int hi, auto stage_c, auto mask_c, auto rows_c) __attribute__((always_inline)) {
    f32x4 acc_s[QT][decltype(rows_c)::value / 16];
    tile_qk(stage_c, acc_s);
    tile_softmax_pv(base, hi, stage_c, mask_c, acc_s, [] {});
  };

  // rows of this wave that can see any key of tile `base`; interior tiles skip the mask
  auto consume = [&](int stage_base, auto stage_c) __attribute__((always_inline)) {
    const int base = stage_base + half * TILE;
    if (HV > 1 && base >= t_hi) return;                     // this half's tile is past the range
    if (!wave_live || base > c + wave_row_lo + WROWS - 1) return;  // past every row's last position
    using Rows = std::integral_constant<int, TILE>;
    if (base + TILE - 1 <= c + wave_row_lo && base + TILE <= t_hi)
      compute_tile(base, t_hi, stage_c, std::integral_constant<bool, false>{}, Rows{});
    else
      compute_tile(base, t_hi, stage_c, std::integral_constant<bool, true>{}, Rows{});
  };

  // Candidate block: K and V rows 0 .. k_i - 1 (from k_new, else from the pool) in the layout of
  // a 32-row tile of LDS stage 1, V rows k_i .. 31 zero (they meet zero probabilities in the
  // 32-row P.V step).  Loaded in one batch per thread, ahead of the first tile's loads, so that
  // staging them waits only for themselves (loads complete in issue order).
  constexpr int CPH = 2 * 16 * (D / 8);  // pieces of K and V rows 0..15
  constexpr int CPB = (CPH + NW * 64 - 1) / (NW * 64);
  auto load_candidates = [&](Piece (&xc)[CPB]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < CPB; ++b) {
      const int e = b * NW * 64 + tid;
      const int isv = e / (16 * (D / 8)), row = (e / (D / 8)) % 16, slot = e % (D / 8);
      xc[b] = Piece{0u, 0u, 0u, 0u};
      if (e < CPH && row < nrows) {
        const uint16_t *r =
            knew ? (isv ? vnew : knew) + ((int64_t)(off + row) * p.hkv + g) * D
                 : reinterpret_cast<const uint16_t *>((isv ? vpool_g : kpool_g) +
                                                      mapped_row(p, kvi, kb, c + row) * row_bytes);
        const u32x4 v = gload_stream<u32x4>(r + 8 * slot);
        xc[b] = Piece{v[0], v[1], v[2], v[3]};
      }
    }
  };
  auto store_candidates = [&](const Piece (&xc)[CPB]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < CPB; ++b) {
      const int e = b * NW * 64 + tid;
      const int isv = e / (16 * (D / 8)), row = (e / (D / 8)) % 16, slot = e % (D / 8);
      if (e < CPH)
        *(lds_u32x4 *)(uintptr_t)(lds_base + STAGE_BYTES + (isv ? TILE * D * 2 : 0) + row * (2 * D) +
                                  16 * (isv ? v_slot<D>(row, slot) : k_slot<D>(row, slot))) =
            u32x4{xc[b].a, xc[b].b, xc[b].c, xc[b].d};
    }
    for (int e = tid; e < 16 * (D / 8); e += NW * 64) {
      const int row = 16 + e / (D / 8), slot = e % (D / 8);
      *(lds_u32x4 *)(uintptr_t)(lds_base + STAGE_BYTES + TILE * D * 2 + row * (2 * D) +
                                16 * v_slot<D>(row, slot)) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // Tile j sits in register set j % RSETS until it is stored to LDS stage j % 2.  Iteration t
  // consumes stage t % 2, stores tile t + 1 (its loads were issued RSETS iterations ago) to the
  // other stage, which every wave finished reading before the previous barrier, and reuses the
  // freed register set for tile t + 1 + RSETS.  One barrier per tile.
  Piece xa[QPW], xb[QPW];
  if constexpr (PF) {
    // Prefill: three LDS stages, so that a wave computes tile t + 1's Q.K products and then
    // tile t's softmax and P.V (the softmax's VALU work issues while those MFMAs run) while
    // tile t + 2 is stored into the third stage; one barrier per tile.  Tile t sits in stage
    // t % 3 and its scores in buffer t % 2 (the loop is unrolled by 6).
    constexpr int KB = TILE / 16;
    f32x4 sa[QT][KB], sb[QT][KB];
    // Every wave computes every tile (a wave whose rows end before a tile sees it fully masked,
    // and waves past the request work on zero queries that are never stored), so that the
    // iteration has no branch but the mask choice before the row maximum and the rare
    // reference move: the next tile's Q.K products share one basic block with this tile's
    // exponentials and P.V, free to interleave.  The tile after the last is never consumed.
    if (n_tiles > 0) load_tile(r_lo, xa);
    if (n_tiles > 1) load_tile(r_lo + TILE, xb);
    if (n_tiles > 0) store_tile(xa, 0);
    if (n_tiles > 1) store_tile(xb, 1);
    if (n_tiles > 2) load_tile(r_lo + 2 * TILE, xa);
    __syncthreads();
    tile_qk(std::integral_constant<int, 0>{}, sa);
    auto iter = [&](int t, auto s_c, auto &cur, auto &nxt) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value;
      const int base = r_lo + t * TILE;
      // unmasked when every position of the tile is visible to every row of the wave
      const bool masked = !(base + TILE - 1 <= c + wave_row_lo && base + TILE <= t_hi);
      tile_softmax_pv(base, t_hi, s_c, masked, cur,
                      [&] { tile_qk(std::integral_constant<int, (S + 1) % 3>{}, nxt); });
      if (t + 2 < n_tiles) {
        if (t + 3 < n_tiles)
          store_load_tile(xa, (S + 2) % 3, r_lo + (t + 3) * TILE);
        else
          store_tile(xa, (S + 2) % 3);
      }
      __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int t = 0; t < n_tiles; t += 6) {
      iter(t, I0{}, sa, sb);
      if (t + 1 >= n_tiles) break;
      iter(t + 1, I1{}, sb, sa);
      if (t + 2 >= n_tiles) break;
      iter(t + 2, I2{}, sa, sb);
      if (t + 3 >= n_tiles) break;
      iter(t + 3, I0{}, sb, sa);
      if (t + 4 >= n_tiles) break;
      iter(t + 4, I1{}, sa, sb);
      if (t + 5 >= n_tiles) break;
      iter(t + 5, I2{}, sb, sa);
    }
  }
  if constexpr (!PF) {
    if (has_cand) {
      // The candidate block is staged (into stage 1, which the loop first writes after a
      // barrier) and consumed while the first tiles are still in flight; tile 0 is stored after.
      Piece xc[CPB];
      load_candidates(xc);
      if (n_tiles > 0) load_tile(r_lo, xa);
      if (RSETS == 2 && n_tiles > 1) load_tile(r_lo + (HV * TILE), xb);
      store_candidates(xc);
      __syncthreads();
      if (wave_live && half == 0)
        compute_tile(c, r_hi, std::integral_constant<int, 1>{}, std::integral_constant<bool, true>{},
                     std::integral_constant<int, 32>{});
      if (n_tiles > 0) store_tile(xa, 0);
      if (RSETS == 2) {
        if (n_tiles > 2) load_tile(r_lo + 2 * (HV * TILE), xa);
      } else {
        if (n_tiles > 1) load_tile(r_lo + (HV * TILE), xa);
      }
      __syncthreads();
    }
  }
  if (!PF && !has_cand) {
    if (n_tiles > 0) load_tile(r_lo, xa);
    if constexpr (RSETS == 2) {
      if (n_tiles > 1) load_tile(r_lo + (HV * TILE), xb);
      if (n_tiles > 0) store_tile(xa, 0);
      if (n_tiles > 2) load_tile(r_lo + 2 * (HV * TILE), xa);
    } else {
      if (n_tiles > 0) store_tile(xa, 0);
      if (n_tiles > 1) load_tile(r_lo + (HV * TILE), xa);
    }
    __syncthreads();
  }
  for (int t = 0; t < (PF ? 0 : n_tiles); t += 2) {
    consume(r_lo + t * (HV * TILE), std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) {
      if constexpr (RSETS == 2) {
        store_tile(xb, 1);
        if (t + 3 < n_tiles) load_tile(r_lo + (t + 3) * (HV * TILE), xb);
      } else {
        if (t + 2 < n_tiles)
          store_load_tile(xa, 1, r_lo + (t + 2) * (HV * TILE));
        else
          store_tile(xa, 1);
      }
    }
    __syncthreads();
    if (t + 1 >= n_tiles) break;
    consume(r_lo + (t + 1) * (HV * TILE), std::integral_constant<int, 1>{});
    if (t + 2 < n_tiles) {
      if constexpr (RSETS == 2) {
        store_tile(xa, 0);
        if (t + 4 < n_tiles) load_tile(r_lo + (t + 4) * (HV * TILE), xa);
      } else {
        if (t + 3 < n_tiles)
          store_load_tile(xa, 0, r_lo + (t + 3) * (HV * TILE));
        else
          store_tile(xa, 0);
      }
    }
    __syncthreads();
  }

  if constexpr (!PF) {
    // This step's KV writes, by split 0 of each (request, KV head) after its tile loop, so that
    // they stay off the critical path (the kernel reads candidates from k_new, not from the
    // pool): candidate j goes to pool row slot_cache_loc[off + j].
    if (knew && split == 0 && hg == 0) {
      constexpr int C16 = D / 8;
      for (int e = tid; e < nrows * C16 * 2; e += NW * 64) {
        const int isv = e / (nrows * C16);
        const int rem = e % (nrows * C16);
        const int j = rem / C16, cc = rem % C16;
        const int64_t loc = p.pk_offsets ? kb + c + j : p.slot_cache_loc[off + j];
        if (loc < 0 || loc >= p.pool_rows) {
          status_or(p.status, DSV_STATUS_POOL);
          continue;
        }
        const uint16_t *src = (isv ? vnew : knew) + ((int64_t)(off + j) * p.hkv + g) * D + cc * 8;
        uint16_t *dst = static_cast<uint16_t *>(isv ? p.v_pool : p.k_pool) + g * p.stride_head +
                        loc * p.stride_row + cc * 8;
        gstore(dst, gload<u32x4>(src));
      }
    }
  }
  if constexpr (HV == 2) {
    // The two halves hold online-softmax states over disjoint tiles of the same rows: half 1
    // hands its state to half 0 through LDS (unused after the loop's last barrier), half 0
    // merges them.  Layout [value][wave][lane], conflict-free.
    float *xs = reinterpret_cast<float *>(lds);
    auto at = [&](int k) __attribute__((always_inline)) { return (k * NWH + wh) * 64 + lane; };
    if (half == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[at(4 * db + e)] = acc_o[0][db][e];
      xs[at(4 * DB)] = m_ref[0];
      xs[at(4 * DB + 1)] = l_run[0];
    }
    __syncthreads();
    if (half == 1) return;
    const float m1 = xs[at(4 * DB)], l1 = xs[at(4 * DB + 1)];
    const float m_new = fmaxf(m_ref[0], m1);
    const float a0 = m_ref[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref[0] - m_new);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc_o[0][db][e] = acc_o[0][db][e] * a0 + xs[at(4 * db + e)] * a1;
    l_run[0] = l_run[0] * a0 + l1 * a1;
    m_ref[0] = m_new;
  }
  if (!wave_live) return;
  // full row sums across the four lane groups holding each row
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    l_run[qt] += __shfl_xor(l_run[qt], 16);
    l_run[qt] += __shfl_xor(l_run[qt], 32);
  }
  if (!col_ok) return;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int my_row = my_row0 + 16 * qt;
    if (my_row >= nrows) break;
    const bool empty = !(l_run[qt] > 0.f);
    const float inv_l = empty ? 0.f : 1.f / l_run[qt];
    const float lse_v = empty ? -INFINITY : (m_ref[qt] + __builtin_amdgcn_logf(l_run[qt])) * 0.69314718055994530942f;
    const int64_t orow = q_row0 + my_row;
    const f32x4 *ao = acc_o[qt];
    if (PF || n_splits_i == 1) {
      uint16_t *o = static_cast<uint16_t *>(PF ? p.pf_out : p.out) + (orow * p.hq + h) * (int64_t)D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + 4 * lg;
        gstore(o + d, u32x2{cvt_pk_bf16(ao[db][0] * inv_l, ao[db][1] * inv_l),
                            cvt_pk_bf16(ao[db][2] * inv_l, ao[db][3] * inv_l)});
      }
      float *lse = PF ? p.pf_lse : p.lse;
      if (lse && lg == 0) gstore(lse + orow * p.hq + h, lse_v);
    } else {
      // partials are read once, by the merge kernel: streaming (non-temporal) stores, rounded
      // to bf16 like the output itself (half the bytes of the write-back and of the merge's
      // reads; the merge weights and sums them in fp32)
      uint16_t *o = p.ws_o + (((int64_t)split * p.m_bs + orow) * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + 4 * lg;
        gstore_stream(o + d, u32x2{cvt_pk_bf16(ao[db][0] * inv_l, ao[db][1] * inv_l),
                                   cvt_pk_bf16(ao[db][2] * inv_l, ao[db][3] * inv_l)});
      }
      if (lg == 0)
        gstore_stream(p.ws_lse + ((int64_t)split * p.m_bs + orow) * p.hq + h, lse_v);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge (split outputs o_s stored in bf16, weights and sums in fp32):
// out = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M}, lse = M + ln(sum),
// splits taken in increasing order with a running maximum (deterministic).  Half a wavefront (32 lanes x 4 floats)
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
  if (p.pk_offsets) {
    // fused packer: the effective length is the difference of the offsets it wrote
    off = p.offsets[i];
    ki = p.offsets[i + 1] - off;
    c = p.ctx_len[i];
    kb = p.kv_base[i];
    if (j >= ki || kb + c + ki > p.pool_rows) return;
  } else if (verify_request(p, i, ki, off, c, kb) || j >= ki) {
    return;
  }
  const int S = verify_splits(p, c + ki);
  if (S <= 1) return;
  const int64_t plane = (int64_t)p.m_bs * p.hq;
  const int64_t rh = (int64_t)(off + j) * p.hq + h;
  // one pass with a running maximum over the splits in order; the loads of eight splits at a
  // time are all issued before any is combined
  float M = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  const u32x2 *src = reinterpret_cast<const u32x2 *>(p.ws_o + rh * D) + l4;
  const int64_t step4 = plane * D / 4;
  constexpr int kBatch = 8;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float ls[kBatch];
    f32x4 o[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + u;
      ls[u] = s < S ? gload<float>(p.ws_lse + s * plane + rh) : -INFINITY;
      const u32x2 b = s < S ? gload<u32x2>(src + s * step4) : u32x2{0u, 0u};
      o[u] = f32x4{bf16_bits_to_f32(b[0] & 0xffffu), bf16_bits_to_f32(b[0] >> 16),
                   bf16_bits_to_f32(b[1] & 0xffffu), bf16_bits_to_f32(b[1] >> 16)};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u >= S) break;
      const float m_new = fmaxf(M, ls[u]);
      const float a = m_new == -INFINITY ? 1.f : __expf(M - m_new);  // rescale of the sum so far
      const float b = ls[u] == -INFINITY ? 0.f : __expf(ls[u] - m_new);  // weight of split s
      den = den * a + b;
      num = num * a + b * o[u];
      M = m_new;
    }
  }
  const float inv = 1.f / den;
  const u32x2 v = {f32_to_bf16_bits(num[0] * inv) | (f32_to_bf16_bits(num[1] * inv) << 16),
                   f32_to_bf16_bits(num[2] * inv) | (f32_to_bf16_bits(num[3] * inv) << 16)};
  gstore(static_cast<uint16_t *>(p.out) + rh * D + 4 * l4, v);
  if (l4 == 0 && p.lse) gstore(p.lse + rh, M + __logf(den));
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
  const int32_t *kvi = nullptr;  // cache-map row of a verification request
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
    if (p.kv_index) kvi = p.kv_index + (int64_t)i * p.kv_index_stride;
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
    return kpool + g * p.stride_head + mapped_row(p, kvi, kb, pos) * p.stride_row;
  };
  auto vrow = [&](int pos) -> const float * {
    if (vnew && pos >= c) return vnew + ((int64_t)(off + pos - c) * p.hkv + g) * D;
    return vpool + g * p.stride_head + mapped_row(p, kvi, kb, pos) * p.stride_row;
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

// KV halves per verification workgroup: groups of up to 4 query heads run two halves of
// G waves each (one 8-wave workgroup per CU for G = 4), larger groups one.
static int verify_halves(int G) { return G <= 4 ? 2 : 1; }

// Longest automatic split when the units alone fill the GPU (a multiple of kTileKV).
constexpr int64_t kBalanceRows = 4096;

// Query heads per workgroup for head_dim 256: at most this many.
constexpr int kWideHeadsPerWg = 4;

// Query heads per verification workgroup.  For head_dim 256 a head's output accumulators
// take 64 registers per lane, so a KV head's query heads are spread over HG = ceil(G / GW)
// workgroups of 4 one-head waves (two per CU, 2 waves per SIMD, 64 KB of LDS each), which
// each read the KV head's rows, with at most kWideHeadsPerWg heads each.  At head_dim 128
// more than 8 one-head waves per
// workgroup would run at 3-4 waves per SIMD and spill, so larger groups are split the same
// way into workgroups of at most 8 heads.  The groups are as even as possible (the last one
// may hold fewer heads: its spare waves only move tile loads).
static int verify_heads_per_wg(int D, int G) {
  const int cap = D >= 256 ? kWideHeadsPerWg : (D >= 128 ? 8 : G);
  const int groups = (G + cap - 1) / cap;
  int gw = (G + groups - 1) / groups;
  // head_dim 128: workgroups of 2, 3 or 6 one-head waves spill and of 5 or 7 stream slowly
  // (the tile's 32 wave loads do not split evenly over them: one staged tile in registers
  // instead of two); such groups run padded to 4 or 8 heads.  At head_dim 64 groups of 5 to
  // 7 (16 wave loads per tile) run padded to 8 as well (5 heads per KV head 130 -> 121 us,
  // 7 heads 150 -> 126 us on 32 requests at contexts 4k-8k); larger groups keep one wave per
  // head (padding 9 to 15 heads to 16 waves was slower at 12)
  if (D == 128 && (gw == 2 || gw == 3)) gw = 4;
  if (D <= 128 && gw >= 5 && gw <= 7) gw = 8;
  return gw;
}
static int verify_head_groups(int D, int G) {
  const int gw = verify_heads_per_wg(D, G);
  return (G + gw - 1) / gw;
}

// Compute units of the current device, read once per device (256 on a whole MI355X; fewer
// on a partitioned one).  Without a usable device (a host-only workspace query) the plan
// assumes a whole MI355X.
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Split plan of the verification set: KV rows per split (multiple of 64) and the most splits
// per request the grid provides.  Auto: aim for two wave groups (G waves, one per query head
// of the group) in flight per SIMD -- 2 x CUs single-half or 1 x CUs two-half workgroups
// (512 or 256 on 256 CUs) -- when every request sits at max_ctx, rounding the split size down
// to whole 64-row tiles so that all splits but the last (which takes the remainder) have the
// same number of tiles.  max_ctx only shapes the plan: a longer context is still computed
// exactly, its last split being longer.
static Plan make_plan(const dsv_attn_args *a) {
  Plan pl;
  if (a->n_bs <= 0 || a->dtype != DSV_BF16) return pl;
  const int64_t rows = (int64_t)a->max_ctx + a->W;
  int64_t chunk = a->kv_chunk;
  if (chunk <= 0) {
    const int G = a->hkv > 0 ? a->hq / a->hkv : 1;
    const int GW = verify_heads_per_wg(a->d, G);
    const int64_t units = (int64_t)a->n_bs * a->hkv * verify_head_groups(a->d, G);
    // wave groups in flight: two per SIMD (512 groups of G waves, or 256 two-half ones).
    // Per-request regrouping drops at run time the head groups a request does not need (it
    // needs ceil(G k_i / 16) waves), leaving fewer workgroups than counted here, so plans with
    // head groups aim at more rounds: the wide-head workgroups (head_dim 256: 4 waves, two per
    // CU) at three -- a plan for two rounds left 1.3 of them on the 32-request head_dim-256
    // set, its sparse second round idling most CUs (197 us against 165 us for 1.7 rounds) --
    // and head_dim 128's 8-wave ones (one per CU) at twice the workgroups (9 heads per KV head
    // 324 -> 290 us, 16 heads 328 -> 314 us on 32 requests at contexts 4k-8k).  So do sets
    // with fewer KV heads than XCDs, whose units place a request's splits on few XCDs (on
    // the same 32 requests: head_dim 64 with 16/4 heads 69 -> 54 us, 4/4 90 -> 51 us; head_dim
    // 128 with 16/4 heads 116 -> 93 us, 4/4 137 -> 108 us; 8 KV heads keep their plan).
    // At head_dim 256 a KV head served by one workgroup (up to 4 query heads) with 8 or more
    // KV heads takes ten per CU: its workgroups hold one or two computing waves and many
    // units, and shorter splits balance the XCDs better (32 requests at contexts 4k-8k, 8 KV
    // heads: one query head per KV head 309 -> 284 us, two 317 -> 295 us, four 332 -> 321 us;
    // with 2 KV heads the splits get too short: four heads 93 -> 98 us, kept at six).
    const int64_t cus = device_cus();
    const bool more = verify_head_groups(a->d, G) > 1 || a->hkv < kXcds;
    const int64_t wgs = a->d >= 256 ? (more ? 6 : 10) * cus : (more ? 4 : 2) * cus / verify_halves(GW);
    int64_t target = (wgs + units - 1) / units;
    if (target < 1) target = 1;
    if (target > 64) target = 64;
    chunk = rows / target / kTileKV * kTileKV;
    if (chunk < kTileKV) chunk = kTileKV;
    // When one split per unit already fills the GPU, contexts of different lengths would
    // leave workgroups of very different lengths; splits of at most kBalanceRows rows let the
    // dispatcher hand the remaining work to whichever CU frees first (60 requests at contexts
    // 8k-32k: 1009 -> 895 us).
    if (units >= wgs && chunk > kBalanceRows) chunk = kBalanceRows;
  }
  pl.chunk = (int)chunk;
  pl.n_splits = (int)(rows / chunk);
  if (pl.n_splits < 1) pl.n_splits = 1;
  if (pl.n_splits > 1) {
    pl.ws_o = align256((size_t)pl.n_splits * a->m_bs * a->hq * a->d * sizeof(uint16_t));
    pl.ws_lse = align256((size_t)pl.n_splits * a->m_bs * a->hq * sizeof(float));
  }
  return pl;
}

// Tile rows per head_dim.  LDS: two stages of HV tiles of K and V (32 KB per tile for D = 128).
template <int D> struct TileCfg;
template <> struct TileCfg<64> { static constexpr int TILE = 64; };
template <> struct TileCfg<128> { static constexpr int TILE = 64; };
template <> struct TileCfg<256> { static constexpr int TILE = 32; };

// ev0 / ev1 (optional) are attached to the launch itself: their timestamps are the kernel's
// start and end.
template <int D, int NW, bool PF, int HV = 1, bool MAP = false>
static bool launch_attn_k(const AttnParams &p, int grid, hipStream_t s, hipEvent_t ev0 = nullptr,
                          hipEvent_t ev1 = nullptr) {
  // the two-waves-per-head verification kernel takes 64-row tiles when a tile's wave loads
  // split evenly over its waves (fewer, longer stages; otherwise the uneven piece pattern
  // spills)
  constexpr int TILE = (PF && D == 128) ? kPfTile128 : TileCfg<D>::TILE;
  constexpr size_t shm = (size_t)(PF ? 3 : 2) * HV * 2 * TILE * D * sizeof(uint16_t);
  auto kern = attn_bf16_kernel<D, NW, PF, TILE, HV, MAP>;
  // once per kernel (idempotent), so that a captured call contains launches only
  static bool lds_limit_set = false;
  if (!lds_limit_set) {
    if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) !=
        hipSuccess)
      return false;
    lds_limit_set = true;
  }
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), shm, s, ev0, ev1, 0, p);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), shm, s, p);
  return true;
}

// The cache-map variant is a separate instantiation, so that the contiguous kernel carries
// none of its registers.
template <int D, int NW, bool PF, int HV = 1>
static bool launch_attn(const AttnParams &p, int grid, hipStream_t s, hipEvent_t ev0 = nullptr,
                        hipEvent_t ev1 = nullptr) {
  if constexpr (!PF) {
    if (p.kv_index) return launch_attn_k<D, NW, PF, HV, true>(p, grid, s, ev0, ev1);
  }
  return launch_attn_k<D, NW, PF, HV, false>(p, grid, s, ev0, ev1);
}

template <int D>
static int launch_verify_g(const AttnParams &p, int grid, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  if constexpr (D >= 256) {
    // wide heads: groups of one to four heads run on 4 waves (with fewer than 64 (head, row)
    // pairs the waves past the last pair hold no heads and only move tile loads)
    switch (p.GW) {
      case 1:
      case 2:
      case 3:
      case 4: return launch_attn<D, 4, false>(p, grid, s, e0, e1);
      default: return -1;
    }
  } else if constexpr (D == 128) {
    // groups padded to 1 or 4 heads (two KV halves) or 8 heads (one half): the shapes that
    // fit two waves per SIMD without spilling and split a tile's loads evenly
    switch (p.GW) {
      case 1: return launch_attn<D, 2, false, 2>(p, grid, s, e0, e1);
      case 4: return launch_attn<D, 8, false, 2>(p, grid, s, e0, e1);
      case 8: return launch_attn<D, 8, false>(p, grid, s, e0, e1);
      default: return -1;
    }
  } else {
    // head_dim 64: every group of up to 16 heads in one workgroup; up to 4 heads in two KV
    // halves (verify_halves); groups of 5 to 7 padded to 8
    switch (p.GW) {
      case 1: return launch_attn<D, 2, false, 2>(p, grid, s, e0, e1);
      case 2: return launch_attn<D, 4, false, 2>(p, grid, s, e0, e1);
      case 3: return launch_attn<D, 6, false, 2>(p, grid, s, e0, e1);
      case 4: return launch_attn<D, 8, false, 2>(p, grid, s, e0, e1);
      case 8: return launch_attn<D, 8, false>(p, grid, s, e0, e1);
      case 9: return launch_attn<D, 9, false>(p, grid, s, e0, e1);
      case 10: return launch_attn<D, 10, false>(p, grid, s, e0, e1);
      case 11: return launch_attn<D, 11, false>(p, grid, s, e0, e1);
      case 12: return launch_attn<D, 12, false>(p, grid, s, e0, e1);
      case 13: return launch_attn<D, 13, false>(p, grid, s, e0, e1);
      case 14: return launch_attn<D, 14, false>(p, grid, s, e0, e1);
      case 15: return launch_attn<D, 15, false>(p, grid, s, e0, e1);
      case 16: return launch_attn<D, 16, false>(p, grid, s, e0, e1);
      default: return -1;
    }
  }
}

static bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

}  // namespace dsv

extern "C" size_t dsv_verify_attn_workspace_bytes(const dsv_attn_args *a) {
  if (!a) return 0;
  dsv::Plan pl = dsv::make_plan(a);
  return pl.ws_o + pl.ws_lse;
}

namespace dsv {
// Outputs of the packer when it is fused into the verification launch.
struct PackOut {
  const int32_t *block_tokens;
  int32_t *offsets, *slot_req, *slot_tok, *slot_pos;
  int64_t *slot_cache_loc;
};
}  // namespace dsv

// ---------------------------------------------------------------------------
// No-allocation variant: the split partials live in a file-scope device array instead of a
// caller workspace.  Each device holds its own copy; its address is looked up once per device
// (with that device current) and kept, and only that address is handed to the kernels.  The
// partials are written before they are read in every call, so nothing is cleared; calls that
// overlap on one device share the array and race.
// ---------------------------------------------------------------------------
namespace dsv {
constexpr size_t kScratchBytes = DSV_VERIFY_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
static std::atomic<void *> scratch_ptr[kScratchDevices];

// Device address of the current device's scratch array, or null on failure.
static void *scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  void *ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}
}  // namespace dsv

// use_scratch: the split partials go to the current device's scratch array instead of
// a->workspace (the no-allocation entry point).
static dsv_status verify_attn_impl(const dsv_attn_args *a, const dsv::PackOut *po, hipStream_t stream,
                                   bool use_scratch = false) {
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
    if ((!a->offsets && !po) || !a->k || !a->ctx_len || !a->kv_base || !a->q || !a->out)
      return DSV_ERR_INVALID_ARG;
    if ((a->k_new == nullptr) != (a->v_new == nullptr)) return DSV_ERR_INVALID_ARG;
    if (a->k_new && !a->slot_cache_loc && !po) return DSV_ERR_INVALID_ARG;
    if (a->kv_chunk < 0 || a->kv_chunk % kTileKV) return DSV_ERR_INVALID_ARG;
    if (a->kv_index && a->kv_index_stride < 1) return DSV_ERR_INVALID_ARG;
  }
  if (a->kv_index && prefill) return DSV_ERR_UNSUPPORTED;
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
  {
    // every launch of the call within the dispatch limits, checked before the first one
    // (verification workgroups counted at the widest, 16 waves)
    const bool bf16 = a->dtype == DSV_BF16;
    bool fits = true;
    if (prefill) {
      if (a->pf_k_new) fits = fits && launch_fits(mul_sat({a->n_pf, a->pf_max_len, a->hkv}), 256);
      fits = fits && (bf16 ? launch_fits(mul_sat({(a->pf_max_len + pf_rows(a->d) - 1) / pf_rows(a->d),
                                                  a->n_pf, a->hq}), 64 * pf_waves(a->d))
                           : launch_fits(mul_sat({a->n_pf, a->pf_max_len, a->hq}), 256));
    }
    if (verify) {
      fits = fits && (bf16 ? launch_fits(mul_sat({pl.n_splits, a->n_bs, a->hkv,
                                                  verify_head_groups(a->d, G)}), 16 * 64)
                           : launch_fits(mul_sat({a->n_bs, a->W, a->hq}), 256));
      if (bf16 && pl.n_splits > 1)
        fits = fits && launch_fits(mul_sat({a->n_bs, a->W, a->hq}) / (256 / (a->d / 4)) + 1, 256);
    }
    if (!fits) return DSV_ERR_INVALID_ARG;
  }
  void *ws = a->workspace;
  size_t ws_bytes = a->workspace_bytes;
  if (use_scratch) {
    ws = nullptr;
    ws_bytes = kScratchBytes;
    if (pl.ws_o + pl.ws_lse > kScratchBytes) return DSV_ERR_WORKSPACE;
    if (pl.ws_o + pl.ws_lse > 0 && !(ws = scratch_address())) return DSV_ERR_HIP;
  }
  if (pl.ws_o + pl.ws_lse > 0 && (!ws || ws_bytes < pl.ws_o + pl.ws_lse || !aligned(ws, 16)))
    return DSV_ERR_WORKSPACE;
  {
    // no output may share a byte with another output or an input; the pools (read and
    // written) with neither, though with each other (K and V interleaved by head)
    const size_t e = a->dtype == DSV_BF16 ? 2 : 4;
    const int64_t m = verify ? a->m_bs : 0, n = verify ? a->n_bs : 0;
    const int64_t pr = prefill ? a->pf_q_rows : 0, npf = prefill ? a->n_pf : 0;
    const int64_t hq = a->hq, hkv = a->hkv, d = a->d;
    const int64_t pool_elems =
        a->pool_rows > 0 ? add_sat(add_sat(mul_sat({hkv - 1, a->stride_head}),
                                           mul_sat({a->pool_rows - 1, a->stride_row})), d)
                         : 0;
    const Span out[] = {{a->out, span_bytes(mul_sat({m, hq, d}), e)},
                        {a->lse, span_bytes(mul_sat({m, hq}), 4)},
                        {a->pf_out, span_bytes(mul_sat({pr, hq, d}), e)},
                        {a->pf_lse, span_bytes(mul_sat({pr, hq}), 4)},
                        {use_scratch ? nullptr : ws, pl.ws_o + pl.ws_lse},
                        {a->status, 4},
                        {po ? po->offsets : nullptr, span_bytes(n + 1, 4)},
                        {po ? po->slot_req : nullptr, span_bytes(m, 4)},
                        {po ? po->slot_tok : nullptr, span_bytes(m, 4)},
                        {po ? po->slot_pos : nullptr, span_bytes(m, 4)},
                        {po ? po->slot_cache_loc : nullptr, span_bytes(m, 8)}};
    const Span in[] = {{a->q, span_bytes(mul_sat({m, hq, d}), e)},
                       {a->k_new, span_bytes(mul_sat({m, hkv, d}), e)},
                       {a->v_new, span_bytes(mul_sat({m, hkv, d}), e)},
                       {po ? nullptr : a->offsets, span_bytes(n + 1, 4)},
                       {a->k, span_bytes(n, 4)},
                       {a->ctx_len, span_bytes(n, 4)},
                       {a->kv_base, span_bytes(n, 8)},
                       {po ? nullptr : a->slot_cache_loc, span_bytes(m, 8)},
                       {a->kv_index, span_bytes(mul_sat({n, a->kv_index_stride}), 4)},
                       {po ? po->block_tokens : nullptr, span_bytes(mul_sat({n, a->W}), 4)},
                       {a->pf_q_start, span_bytes(npf, 4)},
                       {a->pf_q_len, span_bytes(npf, 4)},
                       {a->pf_ctx_len, span_bytes(npf, 4)},
                       {a->pf_kv_base, span_bytes(npf, 8)},
                       {a->pf_q, span_bytes(mul_sat({pr, hq, d}), e)},
                       {a->pf_k_new, span_bytes(mul_sat({pr, hkv, d}), e)},
                       {a->pf_v_new, span_bytes(mul_sat({pr, hkv, d}), e)}};
    const Span pools[] = {{a->k_pool, span_bytes(pool_elems, e)}, {a->v_pool, span_bytes(pool_elems, e)}};
    if (outputs_alias(out, in, pools)) return DSV_ERR_INVALID_ARG;
  }

  AttnParams p{};
  p.k_pool = a->k_pool;
  p.v_pool = a->v_pool;
  p.pool_rows = a->pool_rows;
  p.stride_head = a->stride_head;
  p.stride_row = a->stride_row;
  p.hq = a->hq;
  p.hkv = a->hkv;
  p.G = G;
  p.GW = verify_heads_per_wg(a->d, G);
  p.HG = verify_head_groups(a->d, G);
  p.scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / sqrtf((float)a->d);
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.n_bs = a->n_bs;
  p.m_bs = a->m_bs;
  p.W = a->W;
  p.offsets = po ? po->offsets : a->offsets;
  p.k = a->k;
  p.ctx_len = a->ctx_len;
  p.kv_base = a->kv_base;
  p.slot_cache_loc = po ? po->slot_cache_loc : a->slot_cache_loc;
  if (po) {
    p.pk_tokens = po->block_tokens;
    p.pk_offsets = po->offsets;
    p.pk_req = po->slot_req;
    p.pk_tok = po->slot_tok;
    p.pk_pos = po->slot_pos;
    p.pk_loc = po->slot_cache_loc;
  }
  p.q = a->q;
  p.k_new = a->k_new;
  p.v_new = a->v_new;
  p.out = a->out;
  p.lse = a->lse;
  p.chunk = pl.chunk;
  p.n_splits = pl.n_splits;
  p.ws_o = pl.ws_o ? static_cast<uint16_t *>(ws) : nullptr;
  p.ws_lse = pl.ws_o ? reinterpret_cast<float *>(static_cast<char *>(ws) + pl.ws_o) : nullptr;
  p.n_pf = a->n_pf;
  p.pf_max_len = a->pf_max_len;
  p.pf_blocks = prefill ? (a->pf_max_len + pf_rows(a->d) - 1) / pf_rows(a->d) : 0;
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
  p.kv_index = verify ? a->kv_index : nullptr;
  p.kv_index_stride = a->kv_index_stride;
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
      const int grid = (int)((int64_t)p.pf_blocks * a->n_pf * a->hq);
      p.xcd_sib_pf = p.G > 1 && grid % (kXcds * p.G) == 0;
      const bool ok = D == 64    ? launch_attn<64, pf_waves(64), true>(p, grid, stream)
                      : D == 128 ? launch_attn<128, pf_waves(128), true>(p, grid, stream)
                                 : launch_attn<256, pf_waves(256), true>(p, grid, stream);
      if (!ok) return DSV_ERR_HIP;
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
    if (a->dtype == DSV_BF16) {
      const int64_t grid = (int64_t)pl.n_splits * a->n_bs * a->hkv * p.HG;
      p.xcd_sib_v = p.HG > 1 && grid % (kXcds * p.HG) == 0;
      hipEvent_t e0 = a->main_begin, e1 = a->main_end;
      const int ok = D == 64    ? launch_verify_g<64>(p, (int)grid, stream, e0, e1)
                     : D == 128 ? launch_verify_g<128>(p, (int)grid, stream, e0, e1)
                                : launch_verify_g<256>(p, (int)grid, stream, e0, e1);
      if (ok < 0) return DSV_ERR_UNSUPPORTED;
      if (ok == 0) return DSV_ERR_HIP;
    } else {
      if (a->main_begin && hipEventRecord(a->main_begin, stream) != hipSuccess) return DSV_ERR_HIP;
      const int64_t grid = (int64_t)a->n_bs * a->W * a->hq;
      if (D == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p, 0);
      else if (D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, p, 0);
      else
        hipLaunchKernelGGL(attn_f32_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, p, 0);
    }
    DSV_LAUNCH_CHECK();
    if (a->dtype != DSV_BF16 && a->main_end && hipEventRecord(a->main_end, stream) != hipSuccess)
      return DSV_ERR_HIP;
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

extern "C" dsv_status dsv_verify_attn(const dsv_attn_args *a, hipStream_t stream) {
  return verify_attn_impl(a, nullptr, stream);
}


extern "C" dsv_status dsv_verify_attn_noalloc(const dsv_attn_args *a, hipStream_t stream) {
  return verify_attn_impl(a, nullptr, stream, true);
}

extern "C" dsv_status dsv_pack_verify_attn(const dsv_attn_args *a, const int32_t *block_tokens,
                                           int32_t *offsets, int32_t *slot_req, int32_t *slot_tok,
                                           int32_t *slot_pos, int64_t *slot_cache_loc,
                                           hipStream_t stream) {
  // the verification set in bf16 over contiguous segments, with the packer's outputs given
  if (!a || a->dtype != DSV_BF16 || a->n_bs < 1 || a->kv_index) return a ? DSV_ERR_UNSUPPORTED : DSV_ERR_INVALID_ARG;
  if (!block_tokens || !offsets || !slot_req || !slot_tok || !slot_pos || !slot_cache_loc)
    return DSV_ERR_INVALID_ARG;
  if (a->m_bs < 0 || a->W < 1 || a->W > DSV_MAX_W) return DSV_ERR_INVALID_ARG;
  const dsv::PackOut po{block_tokens, offsets, slot_req, slot_tok, slot_pos, slot_cache_loc};
  return verify_attn_impl(a, &po, stream);
}
