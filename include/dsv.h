/*
 * dsv.h -- C ABI of libdsv: packed block verification for block-diffusion
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * The library implements the target-side verification step described in
 * "DScale: Scaling Block-Diffusion Speculative Decoding with Adaptive
 * Verification" (arXiv HTML): each request brings one known anchor token
 * followed by draft candidates (Sec. II-A/II-B); the candidate prefixes of all
 * requests share one flat slot buffer (Sec. III-C, Flat-buffer packer);
 * attention runs on a short verification tile matched to the candidate width,
 * with a separate wide tile for prefill (Sec. III-B, Path-aware tile router);
 * the prefix verifier accepts the longest exact-match prefix and takes the
 * successor from row offset_i + a_i (Sec. III-D, Prefix verifier).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Ownership: every pointer argument is device memory owned by the caller
 *   (unless documented as host).  The library never allocates or frees and
 *   keeps no state between calls; workspaces are caller-owned buffers sized by
 *   the *_workspace_bytes queries and may be reused at a fixed address from
 *   call to call (Sec. III-D, fixed-address workspace).
 * - Execution: work is enqueued on `stream` and returns without waiting.
 *   DSV_OK means "validated and enqueued".  There is no host synchronisation
 *   and no device-to-host readback inside any call (Sec. II-C: no per-step
 *   host readback for slice reconstruction).
 * - Host-detectable errors (null required pointer, sizes out of range,
 *   unsupported head configuration, workspace too small) return a non-zero
 *   dsv_status before anything is enqueued.  So does aliasing: an output
 *   (the status word and the workspace included) that shares a byte with
 *   another output or with an input, over the extents the call's sizes give,
 *   is refused with DSV_ERR_INVALID_ARG.  Inputs may share bytes; the KV
 *   pools, read and written, may share an allocation with each other (for
 *   example K and V interleaved by head) but with no other argument.  Sizes
 *   whose launches would exceed a dispatch's 2^32 - 1 work-items are refused
 *   with DSV_ERR_INVALID_ARG as well (before the call's first launch).
 * - Data-dependent errors are reported in the caller's device word `status`
 *   (int32, OR-ed with the DSV_STATUS_* bits below; the library never clears
 *   it) and the affected outputs take the defined values stated per call.
 * - Calls are re-entrant; calls that share output or workspace buffers must
 *   be ordered by the caller (same stream).  No C++ exception crosses the ABI.
 */
#ifndef DSV_H
#define DSV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsv_status {
  DSV_OK = 0,
  DSV_ERR_INVALID_ARG = 1, /* null required pointer, size or layout out of range, aliasing */
  DSV_ERR_UNSUPPORTED = 2, /* head_dim / grouping / dtype the kernels do not cover */
  DSV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query reports */
  DSV_ERR_HIP = 4          /* a HIP launch failed */
} dsv_status;

typedef enum dsv_dtype {
  DSV_BF16 = 0, /* bfloat16 storage, fp32 arithmetic */
  DSV_F32 = 1   /* float32 storage and arithmetic */
} dsv_dtype;

/* Bits of the device status word. */
#define DSV_STATUS_BAD_REQUEST 1 /* k_i outside [0, W], negative context/base, offsets out of range */
#define DSV_STATUS_BUDGET 2      /* sum of k_i exceeds the slot capacity m_bs */
#define DSV_STATUS_NAN 4         /* a NaN logit */
#define DSV_STATUS_POOL 8        /* a visible KV row or a candidate write outside the pool */
#define DSV_STATUS_PREFILL 16    /* a prefill request outside its declared bounds */

/* Largest candidate block width (anchor included) the verification tile covers. */
#define DSV_MAX_W 16

/* Human-readable name of a status code (static string). */
const char *dsv_status_string(dsv_status s);

/* ABI version of this header; bumps on any change of a struct or signature. */
#define DSV_ABI_VERSION 1
int dsv_abi_version(void);

/* ------------------------------------------------------------------------ */
/* dsv_pack_slots -- flat-buffer packer                                      */
/*                                                                            */
/* DScale Sec. III-C ("Flat-buffer packer", Fig. 6) and Sec. II-C            */
/* (Challenge 3): prefixes of lengths k_i share one buffer of capacity m_bs  */
/* using exclusive prefix-sum offsets, and tokens, positions and cache       */
/* references are packed with identical row mappings.                        */
/*                                                                            */
/* Inputs  k[n_bs] (0 = inactive request), ctx_len[n_bs] (committed context), */
/*         kv_base[n_bs] (first pool row of the request's contiguous KV      */
/*         segment), block_tokens[n_bs][W] (row-major; column 0 = anchor).   */
/* Outputs offsets[n_bs + 1]: offsets[i] = sum_{j<i} k_j, offsets[n_bs] = end */
/*         boundary S.  For slot s = offsets[i] + j (j < k_i):               */
/*           slot_req[s] = i, slot_tok[s] = block_tokens[i][j],              */
/*           slot_pos[s] = ctx_len[i] + j,                                    */
/*           slot_cache_loc[s] = kv_base[i] + ctx_len[i] + j.                */
/*         Tail slots s in [S, m_bs): req -1, tok 0, pos 0, cache_loc -1.    */
/* Sizes   0 <= n_bs <= 1048576, 1 <= W <= DSV_MAX_W, 0 <= m_bs < 2^31.     */
/* Errors  (device) a request with k_i outside [0, W] or negative ctx/base   */
/*         sets DSV_STATUS_BAD_REQUEST and is packed as inactive (k_i = 0);  */
/*         if the remaining lengths sum above m_bs, DSV_STATUS_BUDGET is set */
/*         and every request is packed as inactive (all offsets 0, every     */
/*         slot a tail placeholder).                                         */
/* One kernel launch (a single workgroup).                                   */
/* ------------------------------------------------------------------------ */
dsv_status dsv_pack_slots(int32_t n_bs, int32_t W, int32_t m_bs, const int32_t *k,
                          const int32_t *ctx_len, const int64_t *kv_base,
                          const int32_t *block_tokens, int32_t *offsets, int32_t *slot_req,
                          int32_t *slot_tok, int32_t *slot_pos, int64_t *slot_cache_loc,
                          int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_allocate_pack -- budget allocator fused with the flat-buffer packer   */
/*                                                                            */
/* DScale Sec. III-C ("Acceptance predictor" from the sigmoid scores on,     */
/* "Budget allocator", "Flat-buffer packer", Fig. 6).  For each live request */
/* i < n_live, scores[i][0 .. W-2] are the acceptance scores of draft        */
/* positions 1 .. W-1 (sigmoid outputs of a predictor, which is not part of  */
/* the library).  Prefix scores: q[i][0] = 1 (anchor), q[i][j] =             */
/* min(q[i][j-1], scores[i][j-1]); a NaN score counts as 0 and sets          */
/* DSV_STATUS_NAN.  Seed: k0_i = the fp32 sum q[i][1] + ... + q[i][W-1]      */
/* (added in that order) rounded to nearest, ties to even, clipped to        */
/* [1, W].  The seeds are then adjusted until sum k = m_live: slots are      */
/* added, one at a time, to the request whose next slot q[i][k_i] scores     */
/* highest, or removed from the request whose last slot q[i][k_i - 1]        */
/* scores lowest (the anchor is never removed; k_i <= W; ties go to the      */
/* lowest request index).  If every request reaches W (or 1) first, the      */
/* adjustment stops there.  Requests n_live .. n_bs-1 get k = 0.  The        */
/* adjusted lengths are then packed exactly as by dsv_pack_slots.            */
/*                                                                            */
/* Inputs  scores[n_bs][W-1] fp32 (rows >= n_live unread), ctx_len, kv_base, */
/*         block_tokens as for dsv_pack_slots.                               */
/* Outputs k[n_bs] adjusted lengths, k0[n_bs] seeds (nullable), offsets and  */
/*         slot arrays as for dsv_pack_slots.                                */
/* Sizes   0 <= n_live <= n_bs <= 1024, 1 <= W <= DSV_MAX_W,                 */
/*         0 <= m_live <= m_bs.                                              */
/* Errors  host: DSV_ERR_INVALID_ARG for sizes outside these bounds or a     */
/*         missing pointer; device: DSV_STATUS_NAN as above.                 */
/* One kernel launch (a single workgroup), no host synchronisation.         */
/* ------------------------------------------------------------------------ */
dsv_status dsv_allocate_pack(int32_t n_live, int32_t n_bs, int32_t W, int32_t m_live, int32_t m_bs,
                             const float *scores, const int32_t *ctx_len, const int64_t *kv_base,
                             const int32_t *block_tokens, int32_t *k, int32_t *k0, int32_t *offsets,
                             int32_t *slot_req, int32_t *slot_tok, int32_t *slot_pos,
                             int64_t *slot_cache_loc, int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_verify_attn -- tile-routed attention over packed slots                */
/*                                                                            */
/* DScale Sec. III-B (Path-aware tile router: verification rows, at most     */
/* W = 16 per request, use a 16-row tile; prefill keeps a wide tile for KV   */
/* reuse) and Sec. III-D (valid rows read offset_i + j with request-local    */
/* causal masking and the supplied cache references).                        */
/*                                                                            */
/* Verification set.  Request i has k_i query rows at slots offsets[i] + j.  */
/* Its key sequence is ctx_len[i] committed rows (pool rows kv_base[i] + p)  */
/* followed by its k_i candidates (anchor first).  Query row j, for every    */
/* query head h, attends to positions 0 .. ctx_len[i] + j with KV head       */
/* h / (hq / hkv):                                                            */
/*   out = softmax(scale * q K^T) V,  lse = ln sum exp(scale * q K^T).       */
/* If k_new/v_new are given they hold the candidates' keys and values (row   */
/* offsets[i] + j); they are used for the candidate positions and written   */
/* to pool rows slot_cache_loc[offsets[i] + j] (this step's KV writes).  If  */
/* they are null the candidates are read from pool rows kv_base[i] +         */
/* ctx_len[i] + j.  A cache reference must not be a row that some request    */
/* of the same call reads from the pool (its committed context): such reads  */
/* would race with the write.                                                */
/*                                                                            */
/* Prefill set (optional, n_pf > 0).  Request r has pf_q_len[r] query rows   */
/* at rows pf_q_start[r] + j of pf_q at positions pf_ctx_len[r] + j; every   */
/* key/value row (pool rows pf_kv_base[r] + p) must already be in the pool,  */
/* or be given in pf_k_new/pf_v_new rows pf_q_start[r] + j, which are then   */
/* written to pool rows pf_kv_base[r] + pf_ctx_len[r] + j first.  Row j      */
/* attends to positions 0 .. pf_ctx_len[r] + j.                              */
/*                                                                            */
/* Layouts (row-major, contiguous unless strided):                           */
/*   k_pool, v_pool [hkv][pool_rows][d] addressed as                         */
/*     g * stride_head + row * stride_row + c   (elements; stride_row >= d,  */
/*     both strides multiples of 8 for bf16 and of 4 for fp32)               */
/*   q, out [m_bs][hq][d]; k_new, v_new [m_bs][hkv][d]; lse [m_bs][hq] f32   */
/*   pf_q, pf_out [pf_q_rows][hq][d]; pf_k_new, pf_v_new [pf_q_rows][hkv][d] */
/*   All of q/out/pool/k_new/v_new/pf_* have element type `dtype`.          */
/* Outputs: rows of valid requests are written; tail rows                    */
/*   [offsets[n_bs], m_bs) are zero-filled (lse -inf); any other row is not   */
/*   touched.  The pool is written only at the candidate (and pf_k_new) rows. */
/* Supported: d in {64, 128, 256}; hq % hkv == 0; hq / hkv <= 16 (bf16);     */
/*   W <= DSV_MAX_W.                                                         */
/* Errors (device): invalid request (k_i outside [0, W], negative ctx/base,  */
/*   offsets[i] + k_i > m_bs, segment past pool_rows):                      */
/*   DSV_STATUS_BAD_REQUEST or DSV_STATUS_POOL, its rows are zero-filled     */
/*   when its offsets are in range; a candidate write outside the pool is    */
/*   skipped with DSV_STATUS_POOL; invalid prefill request:                  */
/*   DSV_STATUS_PREFILL, nothing computed for it.                            */
/* ------------------------------------------------------------------------ */
typedef struct dsv_attn_args {
  dsv_dtype dtype;
  int32_t hq, hkv, d;
  float softmax_scale; /* 0 => 1 / sqrt(d) */
  int32_t kv_chunk;    /* KV rows per split of a verification request (multiple of 64); 0 => auto */
  int32_t max_ctx;     /* host-known typical/upper context length of the verification set: sizes
                          the split plan and the workspace; a longer ctx_len[i] is still
                          computed exactly (its last split is longer) */

  /* KV pool (written at candidate rows) */
  void *k_pool, *v_pool;
  int64_t pool_rows, stride_head, stride_row;

  /* verification set (packed by dsv_pack_slots) */
  int32_t n_bs, m_bs, W;
  const int32_t *offsets;        /* [n_bs + 1] */
  const int32_t *k;              /* [n_bs] */
  const int32_t *ctx_len;        /* [n_bs] */
  const int64_t *kv_base;        /* [n_bs] */
  const int64_t *slot_cache_loc; /* [m_bs], required when k_new is given */
  const void *q;                 /* [m_bs][hq][d] */
  const void *k_new, *v_new;     /* [m_bs][hkv][d] or null */
  void *out;                     /* [m_bs][hq][d] */
  float *lse;                    /* [m_bs][hq] or null */

  /* prefill set (n_pf = 0 to omit) */
  int32_t n_pf, pf_max_len, pf_q_rows;
  const int32_t *pf_q_start, *pf_q_len, *pf_ctx_len; /* [n_pf] */
  const int64_t *pf_kv_base;                         /* [n_pf] */
  const void *pf_q;
  const void *pf_k_new, *pf_v_new; /* or null */
  void *pf_out;
  float *pf_lse; /* or null */

  void *workspace;
  size_t workspace_bytes;
  int32_t *status;

  /* Optional instrumentation: when non-null, these events time the
     verification attention kernel itself.  For bf16 they are the start and
     stop events of its launch (hipExtLaunchKernel), so their elapsed time is
     the kernel's duration; for fp32 they are recorded on `stream` right
     before and after it.  The split-KV merge, if any, is not included.  Do
     not pass them while `stream` is being captured into a graph. */
  hipEvent_t main_begin, main_end;

  /* Optional token-granular cache map of the verification set (the pages'
     cacheMap / historyKV gather, DScale Sec. III-D): when non-null, position
     p of request i (0 <= p < ctx_len[i] + k[i]) is pool row
     kv_index[i * kv_index_stride + p] instead of kv_base[i] + p.  Rows are
     read for the context and, when k_new is null, for the candidates; a
     row outside [0, pool_rows) sets DSV_STATUS_POOL and reads row 0 or the
     last row instead; ctx_len[i] + k[i] > kv_index_stride makes request i
     invalid (DSV_STATUS_BAD_REQUEST).  kv_base is then unused by this call.
     Not supported together with a prefill set or with DSV_F32 prefill. */
  const int32_t *kv_index;  /* [n_bs][kv_index_stride] or null */
  int64_t kv_index_stride;
} dsv_attn_args;

/* sizeof(dsv_attn_args) as compiled into the library (binding check). */
size_t dsv_attn_args_size(void);

/* Workspace bytes dsv_verify_attn needs for these arguments (sizes only are
   read; pointers may be null).  Returns 0 when none is needed. */
size_t dsv_verify_attn_workspace_bytes(const dsv_attn_args *args);

dsv_status dsv_verify_attn(const dsv_attn_args *args, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_verify_attn_noalloc -- dsv_verify_attn without a caller workspace     */
/*                                                                            */
/* For callers that cannot allocate device memory (code under HIP graph      */
/* capture, tight serving loops, harnesses that forbid hipMalloc): the same */
/* computation, kernels and results as dsv_verify_attn(args), with the      */
/* split-KV partials kept in a fixed device array inside the library        */
/* (DSV_VERIFY_SCRATCH_BYTES per GPU, held from the library's first use on  */
/* that GPU until the process ends) instead of args->workspace, which is    */
/* ignored.  No hipMalloc, hipFree or other allocating call is made.        */
/* Limit: calls whose dsv_verify_attn_workspace_bytes(args) exceeds          */
/* DSV_VERIFY_SCRATCH_BYTES return DSV_ERR_WORKSPACE before anything is      */
/* enqueued (pass a larger kv_chunk, or use dsv_verify_attn).  Calls on one  */
/* GPU share that GPU's array: calls that may overlap in time on the same   */
/* GPU (different streams without ordering) race and must not be issued.    */
/* Other errors: as dsv_verify_attn; DSV_ERR_HIP if the array's device      */
/* address cannot be obtained.                                               */
/* ------------------------------------------------------------------------ */
#define DSV_VERIFY_SCRATCH_BYTES ((size_t)32 << 20)
dsv_status dsv_verify_attn_noalloc(const dsv_attn_args *args, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_pack_verify_attn -- the packer fused into the verification launch    */
/*                                                                            */
/* DScale Sec. III-C (Flat-buffer packer, Fig. 6) and Sec. III-D (verification */
/* over the packed slots) in one kernel launch (plus the split merge): the    */
/* same results as dsv_pack_slots(a->n_bs, a->W, a->m_bs, a->k, a->ctx_len,   */
/* a->kv_base, block_tokens, offsets, slot_req, slot_tok, slot_pos,           */
/* slot_cache_loc, a->status) followed by dsv_verify_attn(a) with those       */
/* offsets and cache references, for well-formed requests, without the       */
/* packer's separate launch: every verification workgroup forms its          */
/* request's offset from the effective lengths itself (each reads the        */
/* lengths of all n_bs requests, so the call suits batches of up to a few    */
/* thousand requests; larger ones are better served by the separate calls).  */
/*                                                                            */
/* a: as for dsv_verify_attn; a->offsets and a->slot_cache_loc are ignored    */
/*   (the packer's outputs below take their place); bf16, contiguous          */
/*   segments (a->kv_index null), at least one request.  The packer's         */
/*   outputs: as dsv_pack_slots (offsets [n_bs + 1], slot fields [m_bs]).     */
/* Requests that are malformed (k outside [0, W], a negative context or base) */
/*   or all requests when their lengths sum above m_bs take no slots and get  */
/*   no attention rows (DSV_STATUS_BAD_REQUEST / DSV_STATUS_BUDGET); rows     */
/*   past offsets[n_bs] are zero, their lse -inf.                             */
/* Errors  host: as dsv_verify_attn, DSV_ERR_UNSUPPORTED (fp32, a cache map,  */
/*   no verification set), DSV_ERR_INVALID_ARG (a missing packer output).     */
/* ------------------------------------------------------------------------ */
dsv_status dsv_pack_verify_attn(const dsv_attn_args *args, const int32_t *block_tokens,
                                int32_t *offsets, int32_t *slot_req, int32_t *slot_tok,
                                int32_t *slot_pos, int64_t *slot_cache_loc, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_accept -- greedy prefix verifier, output builder and draft margin     */
/*                                                                            */
/* DScale Sec. III-D (Prefix verifier, greedy: a deterministic top-1 draft   */
/* is accepted when it equals the target's choice; after a_i accepted        */
/* candidates, row offset_i + a_i supplies the successor; the output is the  */
/* accepted candidates followed by the successor), Sec. II-B (progress = one */
/* anchor plus accepted drafts; the Top1-Top2 draft logit gap, Fig. 4) and   */
/* DFlash-Mini-Lab (the anchor is not drafted; accept the exact prefix; the  */
/* top-1/top-2 draft margin of DFlash7-ACT).                                 */
/*                                                                            */
/* Target part (target_logits non-null), logits [m_bs][vocab] f32:          */
/*   slot_argmax[s] = first index of the maximum of row s for s < S =        */
/*     offsets[n_bs] (-0.0 == +0.0), -1 for s >= S.                          */
/*   For request i with k_i > 0: a_i = largest a <= k_i - 1 such that        */
/*     slot_tok[off_i + j] == slot_argmax[off_i + j - 1] for all 1 <= j <= a; */
/*     accepted[i] = a_i, bonus[i] = slot_argmax[off_i + a_i],               */
/*     progress[i] = 1 + a_i, out_tokens[i] = the a_i accepted drafts, then  */
/*     bonus, then -1 up to W.  k_i = 0: accepted 0, bonus -1, progress 0,   */
/*     out_tokens all -1.                                                     */
/* Draft part (draft_logits non-null), draft_logits [n_bs][n_pos][draft_vocab] */
/*   f32: margin[i][p] = fp32(top1 - top2) where top2 is the second element */
/*   of the row sorted descending as a multiset; draft_top1[i][p] = first    */
/*   index of top1 (draft_top1 may be null).                                 */
/* Sizes: 1 <= W <= DSV_MAX_W, vocab >= 1, draft_vocab >= 2, n_pos >= 1.     */
/* Errors (device): invalid k_i/offsets: DSV_STATUS_BAD_REQUEST, accepted -1, */
/*   bonus -1, progress 0, out_tokens -1; a NaN in a row: DSV_STATUS_NAN,    */
/*   that row's argmax / draft_top1 = -1 and its margin NaN.                 */
/* ------------------------------------------------------------------------ */
size_t dsv_accept_workspace_bytes(int32_t m_bs, int32_t vocab, int32_t n_bs, int32_t n_pos,
                                  int32_t draft_vocab);

dsv_status dsv_accept(int32_t n_bs, int32_t m_bs, int32_t W, int32_t vocab,
                      const float *target_logits, const int32_t *slot_tok, const int32_t *offsets,
                      const int32_t *k, int32_t *slot_argmax, int32_t *accepted, int32_t *bonus,
                      int32_t *progress, int32_t *out_tokens, const float *draft_logits,
                      int32_t n_pos, int32_t draft_vocab, float *margin, int32_t *draft_top1,
                      void *workspace, size_t workspace_bytes, int32_t *status,
                      hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_accept_sample -- sampling-mode prefix verifier and output builder     */
/*                                                                            */
/* DScale Sec. III-D (Prefix verifier: with P the target's next-token        */
/* distribution, a deterministic top-1 draft x is accepted with probability  */
/* P(x); at the first rejection the successor is drawn from P with x removed */
/* and the rest renormalised; when every candidate passes, from the          */
/* unmodified P; row offset_i + a_i supplies the successor).                 */
/*                                                                            */
/* target_logits [m_bs][vocab] f32; P_s = softmax(target_logits[s] / T),    */
/*   0 < temperature < inf.  Candidate j >= 1 of request i (x =              */
/*   slot_tok[off_i + j]) is tested by row s = off_i + j - 1 and passes when  */
/*   u_accept[s] < P_s(x) (P_s in fp32; a token outside [0, vocab) has       */
/*   P = 0).  a_i = passes before the first failure.  The successor is drawn */
/*   from row off_i + a_i with weights w_v = exp((l_v - max l) / T) in fp64, */
/*   w_x = 0 after a failure, by the inverse CDF at u_draw[i]: the smallest  */
/*   v whose cumulative weight in index order exceeds u_draw[i] * sum(w)      */
/*   (the last v with w_v > 0 if rounding leaves none).  Uniforms are the    */
/*   caller's, in [0, 1): u_accept [m_bs], u_draw [n_bs].                     */
/* Outputs as dsv_accept: accepted, bonus (successor), progress = 1 + a_i,   */
/*   out_tokens [n_bs][W] (may be null) = accepted drafts, successor, -1.    */
/*   p_cand [m_bs] (may be null): P_s(x) for each row that tests a           */
/*   candidate, -1 for a request's last row, other rows unchanged.           */
/*   k_i = 0: accepted 0, bonus -1, progress 0, out_tokens -1.                */
/* Workspace: dsv_accept_sample_workspace_bytes(n_bs, m_bs, vocab) bytes,    */
/*   256-byte aligned device memory, no initialisation needed.               */
/* Errors  host: DSV_ERR_INVALID_ARG (sizes, W outside [1, DSV_MAX_W], a      */
/*   temperature that is not finite and positive, a missing pointer),        */
/*   DSV_ERR_WORKSPACE.  Device: invalid k_i/offsets: DSV_STATUS_BAD_REQUEST; */
/*   a NaN or +inf logit, or no finite logit, in a row of request i:         */
/*   DSV_STATUS_NAN; both give accepted -1, bonus -1, progress 0 and         */
/*   out_tokens -1 for that request.                                          */
/* ------------------------------------------------------------------------ */
size_t dsv_accept_sample_workspace_bytes(int32_t n_bs, int32_t m_bs, int32_t vocab);

dsv_status dsv_accept_sample(int32_t n_bs, int32_t m_bs, int32_t W, int32_t vocab,
                             const float *target_logits, float temperature,
                             const int32_t *slot_tok, const int32_t *offsets, const int32_t *k,
                             const float *u_accept, const float *u_draw, int32_t *accepted,
                             int32_t *bonus, int32_t *progress, int32_t *out_tokens,
                             float *p_cand, void *workspace, size_t workspace_bytes,
                             int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_draft_features -- per-position confidence features of the drafts      */
/*                                                                            */
/* DScale Sec. III-C (Acceptance predictor: every draft position contributes */
/* its highest logit, the gaps from it to ranks 2-16, the top token's        */
/* log-probability and the distribution's entropy, 18 values in that order). */
/*                                                                            */
/* draft_logits [rows][vocab] f32 (rows = requests x draft positions, in     */
/*   draft order), vocab >= 16.  features [rows][18] f32: with the row       */
/*   sorted descending as a multiset, f[0] = sorted[0], f[r - 1] =           */
/*   fp32(sorted[0] - sorted[r - 1]) for r = 2..16 (exact: the rounded      */
/*   difference), f[16] = ln softmax(row)[top] = -ln sum_v e^(z_v - top),   */
/*   f[17] = -sum_v p_v ln p_v (fp32 accumulation; -inf logits have p = 0). */
/*   For 15 positions a request's 270 features are features[15 i .. 15 i +  */
/*   14], flattened.                                                          */
/* Workspace: dsv_draft_features_workspace_bytes(rows, vocab) bytes of       */
/*   256-byte aligned device memory, no initialisation needed.               */
/* Errors  host: DSV_ERR_INVALID_ARG (rows < 0, vocab < 16, a missing        */
/*   pointer, more than 2^31 workgroups), DSV_ERR_WORKSPACE.  Device: a NaN  */
/*   or +inf logit, or a row without a finite logit, sets DSV_STATUS_NAN and */
/*   that row's 18 features are NaN.                                          */
/* ------------------------------------------------------------------------ */
size_t dsv_draft_features_workspace_bytes(int64_t rows, int32_t vocab);

dsv_status dsv_draft_features(int64_t rows, int32_t vocab, const float *draft_logits,
                              float *features, void *workspace, size_t workspace_bytes,
                              int32_t *status, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_philox_uniforms -- counter-based uniforms for the sampling verifier   */
/*                                                                            */
/* DScale Sec. III-D (Prefix verifier, sampling mode: the accept test and    */
/* the successor draw each take a uniform), generated on the device with     */
/* Philox4x64-10 as defined by Salmon et al., "Parallel random numbers: as   */
/* easy as 1, 2, 3" (SC 2011), so that a serving loop (or a captured graph)  */
/* can refill u_accept / u_draw of dsv_accept_sample without the host.       */
/*                                                                            */
/* out[i] (f32, device) = (w_i >> 40) * 2^-24, w_i = 64-bit word i % 4 of    */
/*   the Philox4x64-10 block at the 128-bit counter                           */
/*   (counter_hi:counter_lo) + i / 4 (carried into counter_hi, the sum taken */
/*   modulo 2^128; the two high counter words are 0) under the key           */
/*   (key1:key0).  Values are multiples of 2^-24 in [0, 1).  A stream of n   */
/*   values consumes ceil(n / 4) counter values, so consecutive calls can    */
/*   advance the counter by that much.                                       */
/* Errors  host: DSV_ERR_INVALID_ARG (n < 0, out null with n > 0, more than  */
/*   2^31 workgroups), DSV_ERR_HIP.  n = 0 enqueues nothing.                  */
/* ------------------------------------------------------------------------ */
dsv_status dsv_philox_uniforms(uint64_t key0, uint64_t key1, uint64_t counter_lo,
                               uint64_t counter_hi, int64_t n, float *out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* dsv_probe_stream_read -- measurement helper (not part of the method)      */
/*                                                                            */
/* Reads `bytes` (rounded down to 16) of device memory at `buf` (16-byte     */
/* aligned) with non-temporal loads in the verification kernel's access      */
/* pattern (two workgroups per CU, each streaming one contiguous range in    */
/* 32 KB blocks), so that a caller can time the practical HBM read ceiling   */
/* that the verification kernel's bandwidth is compared with.  `sink` is a   */
/* device float that is written only in a pathological case (it keeps the    */
/* loads alive).  Enqueued on the current device's `stream`.  Errors:        */
/* DSV_ERR_INVALID_ARG (null, unaligned or shorter than 16 bytes),           */
/* DSV_ERR_HIP (device query or launch failed).                              */
/* ------------------------------------------------------------------------ */
dsv_status dsv_probe_stream_read(const void *buf, size_t bytes, float *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSV_H */
