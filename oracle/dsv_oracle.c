/*
 * dsv_oracle.c -- CPU oracle for packed block verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with
 * the HIP library.
 *
 * Every function is the plain definition of what the method computes,
 * written for a reader to check by eye against the pages:
 *
 *   "DScale: Scaling Block-Diffusion Speculative Decoding with Adaptive
 *    Verification" (arXiv HTML), Sec. III-C (Flat-buffer packer, Fig. 6),
 *    Sec. III-D (fixed-address workspace, request-local causal row mask,
 *    Prefix verifier), Sec. II-A/II-B (anchor + draft prefixes, Fig. 2-4).
 *   "DFlash-Mini-Lab" README (anchor semantics, exact-prefix acceptance,
 *    top-1/top-2 draft margin used by DFlash7-ACT).
 *
 * Floating point: attention is evaluated in IEEE double from the exact
 * input values (bf16 bit patterns or fp32).  Acceptance is integer work
 * driven by float comparisons only.  The margin is the correctly rounded
 * fp32 value of top1 - top2 (the double difference of two floats, rounded
 * once to float; double has 53 >= 2*24+2 bits, so the double rounding is
 * innocuous -- Figueroa, "When is double rounding innocuous?", 1995).
 *
 * Parallelism: OpenMP over independent (request, KV head) or row units; each
 * output element is computed by exactly one thread in a fixed order, so the
 * results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_F32 1

#define OR_OK 0
#define OR_ERR_ARG 1      /* malformed sizes / pointers */
#define OR_ERR_K 2        /* a prefix length outside [0, W] or a bad context */
#define OR_ERR_BUDGET 3   /* sum of prefix lengths exceeds the slot capacity */
#define OR_ERR_NAN 4      /* a NaN logit */
#define OR_ERR_POOL 5     /* a visible KV row outside the pool */

/* Exact value of input element i (bf16 bits are the top half of an fp32). */
static double elem(const void *base, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float *)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Flat-buffer packer (DScale Sec. III-C, "Flat-buffer packer", Fig. 6).     */
/*                                                                            */
/* offset_i is the exclusive prefix sum of the allocated lengths k_i in      */
/* request order; slot offset_i + j carries request i's candidate j (j = 0   */
/* is the anchor).  Tokens, positions and cache references are written with  */
/* the same row mapping.  Position of candidate j is ctx_i + j (the anchor   */
/* sits right after the committed context); its cache reference is the pool */
/* row kv_base_i + ctx_i + j of the request's contiguous segment.  Slots at  */
/* and beyond the end boundary sum(k) are tail placeholders:                 */
/* req -1, token 0, position 0, cache reference -1.                          */
/* ------------------------------------------------------------------------ */
int oracle_pack(int n_bs, int W, int m_bs, const int32_t *k, const int32_t *ctx_len,
                const int64_t *kv_base, const int32_t *block_tokens, int32_t *offsets,
                int32_t *slot_req, int32_t *slot_tok, int32_t *slot_pos, int64_t *slot_cache_loc) {
  if (n_bs < 0 || W < 1 || m_bs < 0) return OR_ERR_ARG;
  for (int i = 0; i < n_bs; ++i) {
    if (k[i] < 0 || k[i] > W) return OR_ERR_K;
    if (ctx_len[i] < 0 || kv_base[i] < 0) return OR_ERR_K;
  }
  int64_t run = 0;
  offsets[0] = 0;
  for (int i = 0; i < n_bs; ++i) {
    run += k[i];
    if (run > m_bs) return OR_ERR_BUDGET;
    offsets[i + 1] = (int32_t)run;
  }
  for (int s = 0; s < m_bs; ++s) {
    slot_req[s] = -1;
    slot_tok[s] = 0;
    slot_pos[s] = 0;
    slot_cache_loc[s] = -1;
  }
  for (int i = 0; i < n_bs; ++i) {
    for (int j = 0; j < k[i]; ++j) {
      int s = offsets[i] + j;
      slot_req[s] = i;
      slot_tok[s] = block_tokens[(int64_t)i * W + j];
      slot_pos[s] = ctx_len[i] + j;
      slot_cache_loc[s] = kv_base[i] + ctx_len[i] + j;
    }
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Budget allocator (DScale Sec. III-C, "Acceptance predictor" and "Budget   */
/* allocator", Algorithm 1 steps from the sigmoid scores on, Fig. 6).        */
/*                                                                            */
/* Input: per live request i < n_live, W - 1 draft acceptance scores         */
/* (sigmoid outputs of the predictor; the predictor itself needs trained     */
/* weights and is not part of this function).                               */
/*   prefix scores: q[i][0] = 1 (the known anchor), q[i][j] = min(q[i][j-1], */
/*     score[i][j-1]) -- acceptance needs accepted predecessors;             */
/*   estimate: l_i = q[i][1] + ... + q[i][W-1] (fp32, added in that order);  */
/*   seed: k0_i = l_i rounded to nearest (ties to even), clipped to [1, W];  */
/*   gap: delta = m_live - sum_i k0_i;                                       */
/*   while delta > 0: the request with the largest next-slot score           */
/*     q[i][k_i] (k_i < W; ties: lowest i) grows by one;                     */
/*   while delta < 0: the request with the smallest last-slot score          */
/*     q[i][k_i - 1] (k_i > 1, the anchor stays; ties: lowest i) shrinks.    */
/* Requests n_live .. n_bs - 1 are inactive: k = 0.  A NaN score counts as   */
/* 0.  If no request can move, the loop stops (the caller sees sum k !=     */
/* m_live).  Writes k[n_bs] and k0[n_bs]; returns OR_ERR_ARG on bad sizes.   */
/* ------------------------------------------------------------------------ */
int oracle_allocate(int n_live, int n_bs, int W, int m_live, const float *score, int32_t *k0,
                    int32_t *k) {
  if (n_live < 0 || n_bs < n_live || W < 1 || W > 64 || m_live < 0) return OR_ERR_ARG;
  float *q = (float *)malloc(sizeof(float) * (size_t)(n_live > 0 ? n_live : 1) * (size_t)W);
  if (!q) return OR_ERR_ARG;
  int64_t total = 0;
  for (int i = 0; i < n_live; ++i) {
    float *qi = q + (size_t)i * W;
    qi[0] = 1.0f;
    float l = 0.0f;
    for (int j = 1; j < W; ++j) {
      float x = score[(size_t)i * (W - 1) + (j - 1)];
      if (x != x) x = 0.0f;
      qi[j] = x < qi[j - 1] ? x : qi[j - 1];
      l = l + qi[j];
    }
    float r = rintf(l);
    int ki = r < 1.0f ? 1 : (r > (float)W ? W : (int)r);
    k0[i] = ki;
    k[i] = ki;
    total += ki;
  }
  for (int i = n_live; i < n_bs; ++i) k0[i] = k[i] = 0;
  int64_t delta = (int64_t)m_live - total;
  while (delta > 0) {
    int best = -1;
    for (int i = 0; i < n_live; ++i)
      if (k[i] < W && (best < 0 || q[(size_t)i * W + k[i]] > q[(size_t)best * W + k[best]])) best = i;
    if (best < 0) break;
    k[best] += 1;
    delta -= 1;
  }
  while (delta < 0) {
    int best = -1;
    for (int i = 0; i < n_live; ++i)
      if (k[i] > 1 && (best < 0 || q[(size_t)i * W + k[i] - 1] < q[(size_t)best * W + k[best] - 1])) best = i;
    if (best < 0) break;
    k[best] -= 1;
    delta += 1;
  }
  free(q);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention for one query row: keys/values are the first n rows of K and V */
/* (row-major [n, d], already in double).                                    */
/*   z_p = scale * sum_c q_c K[p][c];  m = max_p z_p;  w_p = exp(z_p - m);   */
/*   l = sum_p w_p;  o_c = sum_p w_p V[p][c] / l;  lse = m + ln l.           */
/* z is caller scratch of length n.                                          */
/* ------------------------------------------------------------------------ */
static void attend_row(int d, double scale, const double *q, const double *K, const double *V,
                       int64_t n, double *z, double *o, double *lse) {
  double m = -INFINITY;
  for (int64_t p = 0; p < n; ++p) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += q[c] * K[p * d + c];
    z[p] = scale * acc;
    if (z[p] > m) m = z[p];
  }
  double l = 0.0;
  for (int64_t p = 0; p < n; ++p) {
    z[p] = exp(z[p] - m);
    l += z[p];
  }
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int64_t p = 0; p < n; ++p) acc += z[p] * V[p * d + c];
    o[c] = acc / l;
  }
  *lse = m + log(l);
}

/* ------------------------------------------------------------------------ */
/* Packed verification attention (DScale Sec. III-B tile routing; Sec.       */
/* III-D row mask: "valid rows read offset_i + j with request-local causal   */
/* masking and the supplied cache references").                              */
/*                                                                            */
/* Request i's key sequence has ctx_i committed rows followed by its k_i     */
/* candidates (anchor + drafts).  Position p < ctx_i is pool row             */
/* kv_base_i + p.  Candidate position ctx_i + j comes from k_new/v_new row   */
/* offset_i + j when those are given (this step's new KV), else from pool    */
/* row kv_base_i + ctx_i + j.  Query slot offset_i + j sees positions        */
/* 0 .. ctx_i + j (full over the context, causal inside the block).  Query   */
/* head h uses KV head h / (hq / hkv).                                       */
/*                                                                            */
/* Pools are [hkv, pool_rows, d] addressed by element strides.  q is         */
/* [m_bs, hq, d]; k_new, v_new are [m_bs, hkv, d].  out is [m_bs, hq, d] and */
/* lse [m_bs, hq] in double.  Rows s with s >= offsets[n_bs] are the tail:   */
/* out 0, lse -inf.  Other rows not owned by any request are not written.    */
/* slot_mask (nullable, [m_bs]) restricts the computed slots (sampling).     */
/* ------------------------------------------------------------------------ */
/* Pool row of position p of request i: the contiguous segment kv_base_i + p, or, with a     */
/* token-granular cache map (the pages' cacheMap/historyKV gather, Sec. III-D), the row       */
/* kv_index[i * kv_index_stride + p].                                                          */
static int64_t pool_row(const int64_t *kv_base, const int32_t *kv_index, int64_t kv_index_stride,
                        int i, int64_t p) {
  return kv_index ? (int64_t)kv_index[(int64_t)i * kv_index_stride + p] : kv_base[i] + p;
}

int oracle_verify_attn(int dtype, int hq, int hkv, int d, double scale, const void *k_pool,
                       const void *v_pool, int64_t pool_rows, int64_t stride_head,
                       int64_t stride_row, int n_bs, int m_bs, const int32_t *offsets,
                       const int32_t *k, const int32_t *ctx_len, const int64_t *kv_base,
                       const int32_t *kv_index, int64_t kv_index_stride,
                       const void *q, const void *k_new, const void *v_new,
                       const uint8_t *slot_mask, double *out, double *lse) {
  if (hkv <= 0 || hq % hkv != 0 || d <= 0 || n_bs < 0) return OR_ERR_ARG;
  const int G = hq / hkv;
  for (int i = 0; i < n_bs; ++i) {
    if (k[i] < 0 || ctx_len[i] < 0 || kv_base[i] < 0) return OR_ERR_K;
    if (offsets[i] < 0 || offsets[i] + k[i] > m_bs) return OR_ERR_K;
    if (kv_index) {
      if ((int64_t)ctx_len[i] + k[i] > kv_index_stride) return OR_ERR_K;
      /* rows read from the pool: the context, and the candidates when k_new is absent */
      int64_t n_read = (int64_t)ctx_len[i] + (k_new ? 0 : k[i]);
      for (int64_t p = 0; p < n_read; ++p) {
        int64_t r = pool_row(kv_base, kv_index, kv_index_stride, i, p);
        if (r < 0 || r >= pool_rows) return OR_ERR_POOL;
      }
    } else if (kv_base[i] + ctx_len[i] + k[i] > pool_rows) {
      return OR_ERR_POOL;
    }
  }
  int end = offsets[n_bs];
  if (end < 0 || end > m_bs) return OR_ERR_ARG;
  for (int s = end; s < m_bs; ++s) {
    if (slot_mask && !slot_mask[s]) continue;
    for (int h = 0; h < hq; ++h) {
      for (int c = 0; c < d; ++c) out[((int64_t)s * hq + h) * d + c] = 0.0;
      lse[(int64_t)s * hq + h] = -INFINITY;
    }
  }
  int err = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int unit = 0; unit < n_bs * hkv; ++unit) {
    int i = unit / hkv, g = unit % hkv;
    if (k[i] == 0) continue;
    int64_t n = (int64_t)ctx_len[i] + k[i];
    double *K = malloc(sizeof(double) * n * d);
    double *V = malloc(sizeof(double) * n * d);
    double *z = malloc(sizeof(double) * n);
    double *qv = malloc(sizeof(double) * d);
    if (!K || !V || !z || !qv) {
#pragma omp atomic write
      err = OR_ERR_ARG;
      free(K); free(V); free(z); free(qv);
      continue;
    }
    for (int64_t p = 0; p < n; ++p) {
      for (int c = 0; c < d; ++c) {
        if (p >= ctx_len[i] && k_new) {
          int64_t s = offsets[i] + (p - ctx_len[i]);
          K[p * d + c] = elem(k_new, dtype, (s * hkv + g) * d + c);
          V[p * d + c] = elem(v_new, dtype, (s * hkv + g) * d + c);
        } else {
          int64_t idx = g * stride_head + pool_row(kv_base, kv_index, kv_index_stride, i, p) * stride_row + c;
          K[p * d + c] = elem(k_pool, dtype, idx);
          V[p * d + c] = elem(v_pool, dtype, idx);
        }
      }
    }
    for (int j = 0; j < k[i]; ++j) {
      int64_t s = offsets[i] + j;
      if (slot_mask && !slot_mask[s]) continue;
      for (int h = g * G; h < (g + 1) * G; ++h) {
        for (int c = 0; c < d; ++c) qv[c] = elem(q, dtype, (s * hq + h) * d + c);
        attend_row(d, scale, qv, K, V, (int64_t)ctx_len[i] + j + 1, z,
                   out + (s * hq + h) * d, lse + s * hq + h);
      }
    }
    free(K); free(V); free(z); free(qv);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* One request on its own (the unpacked formulation): q_req [k_req, hq, d],  */
/* K_seq / V_seq [hkv, n_seq, d] hold the request's whole key sequence in    */
/* position order (context then candidates).  Query row j sees positions     */
/* 0 .. ctx + j.  out_req [k_req, hq, d], lse_req [k_req, hq].               */
/* ------------------------------------------------------------------------ */
int oracle_attn_one_request(int dtype, int hq, int hkv, int d, double scale, int ctx, int k_req,
                            int64_t n_seq, const void *q_req, const void *K_seq,
                            const void *V_seq, double *out_req, double *lse_req) {
  if (hkv <= 0 || hq % hkv != 0 || ctx < 0 || k_req < 0) return OR_ERR_ARG;
  if ((int64_t)ctx + k_req > n_seq) return OR_ERR_POOL;
  const int G = hq / hkv;
  int64_t n = (int64_t)ctx + k_req;
  double *K = malloc(sizeof(double) * (n ? n : 1) * d);
  double *V = malloc(sizeof(double) * (n ? n : 1) * d);
  double *z = malloc(sizeof(double) * (n ? n : 1));
  double *qv = malloc(sizeof(double) * d);
  if (!K || !V || !z || !qv) { free(K); free(V); free(z); free(qv); return OR_ERR_ARG; }
  for (int g = 0; g < hkv; ++g) {
    for (int64_t p = 0; p < n; ++p)
      for (int c = 0; c < d; ++c) {
        K[p * d + c] = elem(K_seq, dtype, ((int64_t)g * n_seq + p) * d + c);
        V[p * d + c] = elem(V_seq, dtype, ((int64_t)g * n_seq + p) * d + c);
      }
    for (int j = 0; j < k_req; ++j)
      for (int h = g * G; h < (g + 1) * G; ++h) {
        for (int c = 0; c < d; ++c) qv[c] = elem(q_req, dtype, ((int64_t)j * hq + h) * d + c);
        attend_row(d, scale, qv, K, V, (int64_t)ctx + j + 1, z, out_req + ((int64_t)j * hq + h) * d,
                   lse_req + (int64_t)j * hq + h);
      }
  }
  free(K); free(V); free(z); free(qv);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Padded-and-masked formulation (the layout DScale replaces: every request  */
/* reserves W rows, Sec. II-B "N x 16 candidate slots").  q_pad             */
/* [n_req, W, hq, d]; K_pad / V_pad [n_req, hkv, L, d] zero-padded key       */
/* sequences; mask [n_req, W, L] (1 = visible), materialised by the caller.  */
/* Masked scores are -inf, so they contribute exact zeros.  All n_req * W    */
/* rows are computed, including the padding rows the caller discards.       */
/* A row with no visible key is written as 0 with lse -inf.                  */
/* ------------------------------------------------------------------------ */
int oracle_attn_padded_masked(int dtype, int n_req, int W, int hq, int hkv, int d, double scale,
                              int64_t L, const void *q_pad, const void *K_pad, const void *V_pad,
                              const uint8_t *mask, double *out_pad, double *lse_pad) {
  if (hkv <= 0 || hq % hkv != 0 || L <= 0) return OR_ERR_ARG;
  const int G = hq / hkv;
  double *z = malloc(sizeof(double) * L);
  if (!z) return OR_ERR_ARG;
  for (int r = 0; r < n_req; ++r)
    for (int j = 0; j < W; ++j)
      for (int h = 0; h < hq; ++h) {
        int g = h / G;
        const uint8_t *mrow = mask + ((int64_t)r * W + j) * L;
        int64_t qoff = (((int64_t)r * W + j) * hq + h) * d;
        int64_t kvoff = ((int64_t)r * hkv + g) * L * d;
        double m = -INFINITY;
        for (int64_t p = 0; p < L; ++p) {
          if (!mrow[p]) { z[p] = -INFINITY; continue; }
          double acc = 0.0;
          for (int c = 0; c < d; ++c)
            acc += elem(q_pad, dtype, qoff + c) * elem(K_pad, dtype, kvoff + p * d + c);
          z[p] = scale * acc;
          if (z[p] > m) m = z[p];
        }
        double *o = out_pad + qoff;
        if (m == -INFINITY) {
          for (int c = 0; c < d; ++c) o[c] = 0.0;
          lse_pad[((int64_t)r * W + j) * hq + h] = -INFINITY;
          continue;
        }
        double l = 0.0;
        for (int64_t p = 0; p < L; ++p) {
          z[p] = exp(z[p] - m);
          l += z[p];
        }
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t p = 0; p < L; ++p) acc += z[p] * elem(V_pad, dtype, kvoff + p * d + c);
          o[c] = acc / l;
        }
        lse_pad[((int64_t)r * W + j) * hq + h] = m + log(l);
      }
  free(z);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Softmax weights of one query row (materialised P for tiny cases).         */
/* ------------------------------------------------------------------------ */
int oracle_softmax_probs(int dtype, int d, double scale, const void *q, const void *K, int64_t n,
                         double *p_out) {
  double m = -INFINITY;
  for (int64_t p = 0; p < n; ++p) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += elem(q, dtype, c) * elem(K, dtype, p * d + c);
    p_out[p] = scale * acc;
    if (p_out[p] > m) m = p_out[p];
  }
  double l = 0.0;
  for (int64_t p = 0; p < n; ++p) {
    p_out[p] = exp(p_out[p] - m);
    l += p_out[p];
  }
  for (int64_t p = 0; p < n; ++p) p_out[p] /= l;
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Prefill attention (the wide-tile path of DScale Sec. III-B: prefill keeps */
/* the hardware tile for KV reuse).  Request r has q_len_r query rows at     */
/* positions ctx_r .. ctx_r + q_len_r - 1, stored at rows q_start_r + j of   */
/* pf_q [rows, hq, d].  Keys/values of position p are pool row kv_base_r + p */
/* (the new rows already written).  Row j sees positions 0 .. ctx_r + j.     */
/* Only the (request, j) pairs listed in sel_req / sel_j are computed;       */
/* out / lse are indexed by the selection: out [n_sel, hq, d], lse [n_sel,   */
/* hq].                                                                       */
/* ------------------------------------------------------------------------ */
int oracle_prefill_attn(int dtype, int hq, int hkv, int d, double scale, const void *k_pool,
                        const void *v_pool, int64_t pool_rows, int64_t stride_head,
                        int64_t stride_row, int n_pf, const int32_t *q_start, const int32_t *q_len,
                        const int32_t *ctx_len, const int64_t *kv_base, const void *pf_q,
                        int n_sel, const int32_t *sel_req, const int32_t *sel_j, double *out,
                        double *lse) {
  if (hkv <= 0 || hq % hkv != 0) return OR_ERR_ARG;
  const int G = hq / hkv;
  for (int t = 0; t < n_sel; ++t) {
    int r = sel_req[t];
    if (r < 0 || r >= n_pf || sel_j[t] < 0 || sel_j[t] >= q_len[r]) return OR_ERR_ARG;
    if (kv_base[r] + ctx_len[r] + q_len[r] > pool_rows) return OR_ERR_POOL;
  }
  int err = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < n_sel; ++t) {
    int r = sel_req[t], j = sel_j[t];
    int64_t n = (int64_t)ctx_len[r] + j + 1;
    double *K = malloc(sizeof(double) * n * d), *V = malloc(sizeof(double) * n * d);
    double *z = malloc(sizeof(double) * n), *qv = malloc(sizeof(double) * d);
    if (!K || !V || !z || !qv) {
#pragma omp atomic write
      err = OR_ERR_ARG;
      free(K); free(V); free(z); free(qv);
      continue;
    }
    for (int h = 0; h < hq; ++h) {
      int g = h / G;
      if (h % G == 0)
        for (int64_t p = 0; p < n; ++p)
          for (int c = 0; c < d; ++c) {
            int64_t idx = g * stride_head + (kv_base[r] + p) * stride_row + c;
            K[p * d + c] = elem(k_pool, dtype, idx);
            V[p * d + c] = elem(v_pool, dtype, idx);
          }
      int64_t row = (int64_t)q_start[r] + j;
      for (int c = 0; c < d; ++c) qv[c] = elem(pf_q, dtype, (row * hq + h) * d + c);
      attend_row(d, scale, qv, K, V, n, z, out + ((int64_t)t * hq + h) * d, lse + (int64_t)t * hq + h);
    }
    free(K); free(V); free(z); free(qv);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Greedy target choice per slot: the first index of the row maximum        */
/* (numerical comparisons, so -0.0 equals +0.0).  A NaN is an error.         */
/* ------------------------------------------------------------------------ */
int oracle_argmax_rows(int64_t rows, int64_t vocab, const float *logits, int32_t *out) {
  if (vocab <= 0) return OR_ERR_ARG;
  int err = OR_OK;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float *x = logits + r * vocab;
    int64_t best = 0;
    for (int64_t v = 0; v < vocab; ++v) {
      if (isnan(x[v])) {
#pragma omp atomic write
        err = OR_ERR_NAN;
      }
      if (x[v] > x[best]) best = v;
    }
    out[r] = (int32_t)best;
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Greedy prefix verifier + output builder (DScale Sec. III-D "Prefix        */
/* verifier"; DFlash-Mini-Lab: accept the exact prefix, the anchor is not    */
/* drafted).                                                                  */
/*                                                                            */
/* Slot s = offset_i + j holds candidate j of request i; the target row s    */
/* predicts the token that follows it, g_s = slot_argmax[s].  Draft j >= 1   */
/* is accepted while every draft 1..j equals the target's choice at the      */
/* previous slot: tok[offset_i + j] == g[offset_i + j - 1].  a_i is the      */
/* number of accepted drafts (<= k_i - 1); row offset_i + a_i supplies the   */
/* successor (bonus) token; progress = 1 + a_i (the anchor plus accepted     */
/* drafts, also the number of tokens emitted).  Output tokens: the accepted  */
/* drafts followed by the successor, -1 padded to W.  Inactive (k_i = 0):    */
/* accepted 0, bonus -1, progress 0, all -1.                                 */
/* ------------------------------------------------------------------------ */
int oracle_accept(int n_bs, int m_bs, int W, const int32_t *offsets, const int32_t *k,
                  const int32_t *slot_tok, const int32_t *slot_argmax, int32_t *accepted,
                  int32_t *bonus, int32_t *progress, int32_t *out_tokens) {
  for (int i = 0; i < n_bs; ++i) {
    if (k[i] < 0 || k[i] > W || offsets[i] < 0 || offsets[i] + k[i] > m_bs) return OR_ERR_K;
  }
  for (int i = 0; i < n_bs; ++i) {
    for (int t = 0; t < W; ++t) out_tokens[(int64_t)i * W + t] = -1;
    if (k[i] == 0) {
      accepted[i] = 0;
      bonus[i] = -1;
      progress[i] = 0;
      continue;
    }
    int off = offsets[i];
    int a = 0;
    while (a + 1 < k[i] && slot_tok[off + a + 1] == slot_argmax[off + a]) ++a;
    accepted[i] = a;
    bonus[i] = slot_argmax[off + a];
    progress[i] = 1 + a;
    for (int t = 0; t < a; ++t) out_tokens[(int64_t)i * W + t] = slot_tok[off + 1 + t];
    out_tokens[(int64_t)i * W + a] = bonus[i];
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Sampling-mode prefix verifier (DScale Sec. III-D "Prefix verifier": a     */
/* deterministic top-1 draft x is accepted with probability P(x); at the     */
/* first rejection the successor is drawn from P with x removed and the      */
/* remaining mass renormalised; when every candidate passes it is drawn from */
/* the unmodified P; row offset_i + a_i supplies the successor).             */
/*                                                                            */
/* P_s = softmax(logits[s] / T), evaluated in double as                       */
/* exp((l_v - max l) / T) / sum_u exp((l_u - max l) / T).  Candidate j >= 1   */
/* of request i (x = slot_tok[off + j]) is tested by row s = off + j - 1 and  */
/* passes when u_accept[s] < P_s(x).  a_i = number of passes before the      */
/* first failure.  The successor is drawn from row off + a_i with weights    */
/* w_v = P(v), w_x = 0 on a rejection, by the inverse CDF at u_draw[i]: the  */
/* smallest y with u * S < w_0 + ... + w_y (S = sum of w, index order); if   */
/* rounding leaves no such y, the last y with w_y > 0.  Outputs as in the    */
/* greedy verifier.  p_cand[s] = P_s(x) for rows that test a candidate, -1   */
/* for other rows of the request.  Diagnostics for the tests: acc_margin[s]  */
/* = |u_accept[s] - P_s(x)| for every test taken (NaN otherwise) and         */
/* draw_margin[i] = the distance of u * S to the nearer boundary of the      */
/* drawn token's interval, divided by S.  A candidate token outside         */
/* [0, vocab) has probability 0.  A NaN or +inf in a row of an active        */
/* request, or a row with no finite entry, is an error.                       */
/* ------------------------------------------------------------------------ */
static int softmax_row(const float *x, int64_t vocab, double T, double *p) {
  double m = -INFINITY;
  for (int64_t v = 0; v < vocab; ++v) {
    if (isnan(x[v]) || x[v] == INFINITY) return OR_ERR_NAN;
    if ((double)x[v] > m) m = (double)x[v];
  }
  if (m == -INFINITY) return OR_ERR_NAN;
  double z = 0.0;
  for (int64_t v = 0; v < vocab; ++v) {
    p[v] = exp(((double)x[v] - m) / T);
    z += p[v];
  }
  for (int64_t v = 0; v < vocab; ++v) p[v] /= z;
  return OR_OK;
}

int oracle_accept_sample(int n_bs, int m_bs, int W, int64_t vocab, const float *logits,
                         double T, const int32_t *offsets, const int32_t *k,
                         const int32_t *slot_tok, const float *u_accept, const float *u_draw,
                         int32_t *accepted, int32_t *bonus, int32_t *progress,
                         int32_t *out_tokens, double *p_cand, double *acc_margin,
                         double *draw_margin) {
  if (vocab < 1 || !(T > 0.0) || isinf(T)) return OR_ERR_ARG;
  for (int i = 0; i < n_bs; ++i)
    if (k[i] < 0 || k[i] > W || offsets[i] < 0 || offsets[i] + k[i] > m_bs) return OR_ERR_K;
  for (int64_t s = 0; s < m_bs; ++s) acc_margin[s] = NAN;
  int err = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_bs; ++i) {
    for (int t = 0; t < W; ++t) out_tokens[(int64_t)i * W + t] = -1;
    draw_margin[i] = NAN;
    accepted[i] = 0;
    bonus[i] = -1;
    progress[i] = 0;
    if (k[i] == 0) continue;
    const int off = offsets[i];
    double *p = malloc((size_t)vocab * sizeof(double));
    double *prow = malloc((size_t)k[i] * sizeof(double));
    int bad = 0;
    /* P_s(x) for every row that tests a candidate */
    for (int j = 0; j < k[i] && !bad; ++j) {
      const int s = off + j;
      bad = softmax_row(logits + (int64_t)s * vocab, vocab, T, p);
      if (bad) break;
      if (j + 1 < k[i]) {
        const int32_t x = slot_tok[s + 1];
        prow[j] = x >= 0 && x < vocab ? p[x] : 0.0;
      } else {
        prow[j] = -1.0;
      }
      p_cand[s] = prow[j];
    }
    if (bad) {
#pragma omp atomic write
      err = bad;
      free(p);
      free(prow);
      continue;
    }
    int a = 0;
    int rejected = 0;
    while (a + 1 < k[i]) {
      const int s = off + a;
      acc_margin[s] = fabs((double)u_accept[s] - prow[a]);
      if ((double)u_accept[s] < prow[a]) {
        ++a;
      } else {
        rejected = 1;
        break;
      }
    }
    /* successor from row off + a, the rejected draft removed */
    const int s = off + a;
    softmax_row(logits + (int64_t)s * vocab, vocab, T, p);
    if (rejected && slot_tok[s + 1] >= 0 && slot_tok[s + 1] < vocab) p[slot_tok[s + 1]] = 0.0;
    double S = 0.0;
    for (int64_t v = 0; v < vocab; ++v) S += p[v];
    const double target = (double)u_draw[i] * S;
    int64_t y = -1, last = -1;
    double below = 0.0, cum = 0.0;
    for (int64_t v = 0; v < vocab; ++v) {
      if (p[v] > 0.0) last = v;
      below = cum;
      cum += p[v];
      if (target < cum) {
        y = v;
        break;
      }
    }
    if (y < 0) {
      y = last;
      draw_margin[i] = 0.0;
    } else {
      const double d0 = target - below, d1 = cum - target;
      draw_margin[i] = (d0 < d1 ? d0 : d1) / S;
    }
    accepted[i] = a;
    bonus[i] = (int32_t)y;
    progress[i] = 1 + a;
    for (int t = 0; t < a; ++t) out_tokens[(int64_t)i * W + t] = slot_tok[off + 1 + t];
    out_tokens[(int64_t)i * W + a] = (int32_t)y;
    free(p);
    free(prow);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Draft top-1 / top-2 margin (DScale Sec. II-B, Fig. 4: "mean Top1-Top2     */
/* logit gap"; DFlash-Mini-Lab DFlash7-ACT margin).  For each row, top1 is   */
/* the largest value and top2 the second element of the row sorted in       */
/* descending order as a multiset (a repeated maximum gives margin 0).       */
/* margin = fp32(top1 - top2); top1_idx = first index holding top1.  A NaN   */
/* is an error.                                                               */
/* ------------------------------------------------------------------------ */
int oracle_top2_margin(int64_t rows, int64_t vocab, const float *logits, float *margin,
                       int32_t *top1_idx) {
  if (vocab < 2) return OR_ERR_ARG;
  int err = OR_OK;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float *x = logits + r * vocab;
    int64_t best = 0;
    for (int64_t v = 0; v < vocab; ++v) {
      if (isnan(x[v])) {
#pragma omp atomic write
        err = OR_ERR_NAN;
      }
      if (x[v] > x[best]) best = v;
    }
    /* second element of the descending multiset: the maximum over all
       positions other than the first occurrence of the top value */
    double second = -INFINITY;
    for (int64_t v = 0; v < vocab; ++v)
      if (v != best && (double)x[v] > second) second = (double)x[v];
    margin[r] = (float)((double)x[best] - second);
    top1_idx[r] = (int32_t)best;
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Draft confidence features (DScale Sec. III-C "Acceptance predictor": per  */
/* draft position, the highest logit, its gaps to ranks 2-16, the top        */
/* token's log-probability and the entropy of the distribution; 18 values    */
/* per position, in this order).                                              */
/*                                                                            */
/* For a row z of vocab >= 16 logits: sorted = z in descending order (as a   */
/* multiset); f[0] = sorted[0]; f[r - 1] = fp32(sorted[0] - sorted[r - 1])   */
/* for r = 2..16 (the double difference of two floats rounded once to       */
/* float); with p = softmax(z) in double, f[16] = log p(top) and f[17] =     */
/* -sum_{p_v > 0} p_v log p_v, each rounded to float.  A NaN or +inf logit,  */
/* or a row with no finite logit, is an error.                                */
/* ------------------------------------------------------------------------ */
static int cmp_desc(const void *a, const void *b) {
  const float x = *(const float *)a, y = *(const float *)b;
  return x < y ? 1 : (x > y ? -1 : 0);
}

int oracle_draft_features(int64_t rows, int64_t vocab, const float *logits, float *feat) {
  if (vocab < 16) return OR_ERR_ARG;
  int err = OR_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    const float *z = logits + r * vocab;
    float *f = feat + r * 18;
    int bad = 0;
    for (int64_t v = 0; v < vocab; ++v)
      if (isnan(z[v]) || z[v] == INFINITY) bad = 1;
    float *sorted = malloc((size_t)vocab * sizeof(float));
    memcpy(sorted, z, (size_t)vocab * sizeof(float));
    if (!bad) qsort(sorted, (size_t)vocab, sizeof(float), cmp_desc);
    if (bad || sorted[0] == -INFINITY) {
#pragma omp atomic write
      err = OR_ERR_NAN;
      for (int c = 0; c < 18; ++c) f[c] = NAN;
      free(sorted);
      continue;
    }
    const double top = (double)sorted[0];
    f[0] = sorted[0];
    for (int rank = 2; rank <= 16; ++rank) f[rank - 1] = (float)(top - (double)sorted[rank - 1]);
    double Z = 0.0;
    for (int64_t v = 0; v < vocab; ++v) Z += exp((double)z[v] - top);
    double H = 0.0;
    for (int64_t v = 0; v < vocab; ++v) {
      const double p = exp((double)z[v] - top) / Z;
      if (p > 0.0) H -= p * log(p);
    }
    f[16] = (float)log(1.0 / Z);
    f[17] = (float)H;
    free(sorted);
  }
  return err;
}

/* ------------------------------------------------------------------------ */
/* Counter-based uniforms for the sampling verifier's draws.                  */
/*                                                                            */
/* Philox4x64-10 as defined by Salmon, Moraes, Dror and Shaw, "Parallel       */
/* random numbers: as easy as 1, 2, 3" (SC 2011): a 256-bit counter block     */
/* (x0, x1, x2, x3) and a 128-bit key (k0, k1) go through ten rounds; a round */
/* multiplies x0 and x2 by the two round multipliers into 128-bit products    */
/* and produces (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1,         */
/* lo(M0 x0)); between rounds the key is bumped by the two Weyl constants.    */
/* Output i of a stream is word i % 4 of the block at counter c + i / 4       */
/* (c a 128-bit base held in the two low counter words, carried); its         */
/* uniform is the top 24 bits times 2^-24, exactly representable in fp32 and  */
/* in [0, 1).                                                                 */
/* ------------------------------------------------------------------------ */
static void philox4x64_10(uint64_t x[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  for (int r = 0; r < 10; ++r) {
    const unsigned __int128 p0 = (unsigned __int128)M0 * x[0];
    const unsigned __int128 p1 = (unsigned __int128)M1 * x[2];
    const uint64_t y0 = (uint64_t)(p1 >> 64) ^ x[1] ^ k0;
    const uint64_t y1 = (uint64_t)p1;
    const uint64_t y2 = (uint64_t)(p0 >> 64) ^ x[3] ^ k1;
    const uint64_t y3 = (uint64_t)p0;
    x[0] = y0;
    x[1] = y1;
    x[2] = y2;
    x[3] = y3;
    k0 += W0;
    k1 += W1;
  }
}

/* Raw 64-bit words: out[i] = word i % 4 of the block at counter (ctr_lo, ctr_hi) + i / 4. */
int oracle_philox_raw(uint64_t key0, uint64_t key1, uint64_t ctr_lo, uint64_t ctr_hi, int64_t n,
                      uint64_t *out) {
  if (n < 0) return OR_ERR_ARG;
  for (int64_t b = 0; 4 * b < n; ++b) {
    const uint64_t lo = ctr_lo + (uint64_t)b;
    uint64_t x[4] = {lo, ctr_hi + (lo < ctr_lo ? 1u : 0u), 0, 0};
    philox4x64_10(x, key0, key1);
    for (int j = 0; j < 4 && 4 * b + j < n; ++j) out[4 * b + j] = x[j];
  }
  return OR_OK;
}

/* Uniforms: out[i] = (word i >> 40) * 2^-24. */
int oracle_philox_uniforms(uint64_t key0, uint64_t key1, uint64_t ctr_lo, uint64_t ctr_hi,
                           int64_t n, float *out) {
  if (n < 0) return OR_ERR_ARG;
  uint64_t *raw = malloc((size_t)(n > 0 ? n : 1) * sizeof(uint64_t));
  if (!raw) return OR_ERR_ARG;
  oracle_philox_raw(key0, key1, ctr_lo, ctr_hi, n, raw);
  for (int64_t i = 0; i < n; ++i) out[i] = (float)ldexp((double)(raw[i] >> 40), -24);
  free(raw);
  return OR_OK;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Number of threads the OpenMP loops above will use. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the following calls (timing at a chosen thread count; results do not depend
   on it).  Returns the count now in effect. */
int oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}
