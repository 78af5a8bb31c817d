"""Seeded synthetic inputs for packed block verification.

This module only draws inputs: shapes, value distributions and planted
answers.  It holds none of the method's arithmetic (no packing, attention,
argmax or prefix matching) and is shared by the oracle side and the HIP side
of every test, so both receive the same bits.

Distributions follow the pages' workload statistics:

* W = 16 slots per block including the anchor (DScale Sec. II-A/III-C).
* Mean progress 6.09 with a tail to 16 (DScale Sec. II-B, Fig. 2): drafts
  accepted ~ min(Poisson(5.09), 15), so E[progress] = 1 + E[a] ~ 6.09.
* Geometric-tailed prefix lengths rescaled to a shared 8N budget (DScale
  Sec. III-C, "8N live slots").
* Qwen3 vocabulary 151,936 (DFlash-Mini-Lab configuration list); 24 query /
  2 KV heads, head_dim 256, vocabulary 248,320 (PixelML DFlash drafter card,
  architecture table); 8k serving context (same card, measured serving
  protocol).

Seeds: ``numpy.random.default_rng(1000 * c + t)`` for configuration c and a
fixed per-tensor index t.  Floating inputs are drawn in fp32 and, for bf16
cases, rounded to bf16 with round-to-nearest-even; the bit patterns (uint16)
go to both sides unchanged.

Target logits are planted so that every answer is known by construction: each
row gets a unique maximum (row max + 1) at a chosen token, drafts that should
be accepted equal the planted maximum of the previous slot, and the first
draft that should be rejected differs from it.  Logits rows are laid out
request after request (the order in which the target's LM head emits them for
a packed batch), followed by tail rows.
"""
from __future__ import annotations

import numpy as np

W_BLOCK = 16
N_DRAFT_POS = 15


def rng(config: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(1000 * config + tensor)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


def normal(g: np.random.Generator, shape, scale: float, dtype: str, chunk: int = 1 << 26):
    """N(0, scale^2) values as bf16 bits (uint16) or float32, drawn in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[lo:hi] = to_bf16_bits(x) if dtype == "bf16" else x
    return out.reshape(shape)


def lengths_geometric_rescaled(g, n: int, budget: int, W: int = W_BLOCK) -> np.ndarray:
    """Prefix lengths 1 + min(G, W-1) with P(G >= t) = 0.845^t (mean ~6, long tail),
    rescaled to sum exactly to `budget`: round(k0 * budget / sum k0) clipped to [1, W], then
    +-1 in request order until the sum matches."""
    k0 = 1 + np.minimum(g.geometric(0.155, size=n) - 1, W - 1)
    k = np.clip(np.rint(k0 * budget / k0.sum()), 1, W).astype(np.int64)
    i = 0
    guard = 0
    while k.sum() != budget:
        if k.sum() < budget and k[i] < W:
            k[i] += 1
        elif k.sum() > budget and k[i] > 1:
            k[i] -= 1
        i = (i + 1) % n
        guard += 1
        assert guard < 100 * n * W, "budget not reachable"
    return k.astype(np.int32)


def segments(ctx_len, capacity_extra: int):
    """Contiguous pool segments: request i owns rows [kv_base_i, kv_base_i + ctx_i + extra)."""
    cap = np.asarray(ctx_len, np.int64) + capacity_extra
    kv_base = np.zeros(len(cap), np.int64)
    if len(cap) > 1:
        kv_base[1:] = np.cumsum(cap)[:-1]
    return kv_base, int(cap.sum())


def planted_logits(g, k, vocab: int, m_bs: int, accepted, block_tokens, W: int = W_BLOCK):
    """Target logits [m_bs, vocab] ~ N(0,1) with a unique planted maximum in every row, and
    block tokens rewritten so that request i accepts exactly accepted[i] drafts.

    Returns (logits, block_tokens, planted_argmax [n, W] (-1 where unused))."""
    n = len(k)
    blocks = []
    planted = np.full((n, W), -1, np.int64)
    bt = np.array(block_tokens, np.int64, copy=True)
    for i in range(n):
        rows = g.standard_normal((int(k[i]), vocab), dtype=np.float32)
        for j in range(int(k[i])):
            t = int(g.integers(vocab))
            rows[j, t] = rows[j].max() + np.float32(1.0)
            planted[i, j] = t
        a = int(accepted[i])
        for j in range(1, int(k[i])):
            if j <= a:
                bt[i, j] = planted[i, j - 1]
            elif j == a + 1:
                t = int(g.integers(vocab - 1))
                bt[i, j] = t if t < planted[i, j - 1] else t + 1
        blocks.append(rows)
    used = int(sum(int(x) for x in k))
    tail = g.standard_normal((m_bs - used, vocab), dtype=np.float32)
    logits = np.concatenate(blocks + [tail], axis=0) if n else tail
    return np.ascontiguousarray(logits), bt.astype(np.int32), planted.astype(np.int32)


def sampling_logits(g, k, vocab: int, m_bs: int, block_tokens, boost=(4.0, 12.0),
                    p_random: float = 0.2, W: int = W_BLOCK):
    """Target logits [m_bs, vocab] ~ N(0,1) for sampling-mode verification, and block tokens
    whose drafts are the target's likely picks: for draft j >= 1 of request i, with probability
    1 - p_random a random token t gets the logit (row max + U(boost)) in the row that predicts
    it (row j - 1 of the request) and becomes the draft; otherwise the draft is a random token
    with no boost.  The boost range sets how much of the row's mass the draft carries (the
    defaults spread it over (0, 1) at a 151,936-token vocabulary and unit temperature).

    Returns (logits, block_tokens)."""
    n = len(k)
    blocks = []
    bt = np.array(block_tokens, np.int64, copy=True)
    for i in range(n):
        rows = g.standard_normal((int(k[i]), vocab), dtype=np.float32)
        for j in range(1, int(k[i])):
            t = int(g.integers(vocab))
            if g.random() >= p_random:
                rows[j - 1, t] = rows[j - 1].max() + np.float32(g.uniform(*boost))
            bt[i, j] = t
        blocks.append(rows)
    used = int(sum(int(x) for x in k))
    tail = g.standard_normal((m_bs - used, vocab), dtype=np.float32)
    logits = np.concatenate(blocks + [tail], axis=0) if n else tail
    return np.ascontiguousarray(logits), bt.astype(np.int32)


def uniforms(g, n: int) -> np.ndarray:
    """n fp32 uniforms in [0, 1) (24-bit resolution)."""
    return g.random(n, dtype=np.float32)


def draft_logits(seed_config: int, n: int, vocab: int) -> np.ndarray:
    """Draft logits [n, 15, vocab] ~ N(0,1) fp32 (one row per new draft position)."""
    return rng(seed_config, 8).standard_normal((n, N_DRAFT_POS, vocab), dtype=np.float32)


def make_case(
    seed_config: int,
    *,
    dtype: str,
    hq: int,
    hkv: int,
    d: int,
    k,
    ctx_len,
    m_bs: int,
    W: int = W_BLOCK,
    qkv_scale: float = 1.0,
    vocab: int | None = None,
    accepted=None,
    draft_vocab: int | None = None,
    capacity_extra: int | None = None,
) -> dict:
    """A verification batch: pool, packed queries, candidate KV, block tokens, logits."""
    k = np.asarray(k, np.int32)
    ctx_len = np.asarray(ctx_len, np.int32)
    n = len(k)
    kv_base, pool_rows = segments(ctx_len, W if capacity_extra is None else capacity_extra)
    c = dict(
        name=f"cfg{seed_config}",
        dtype=dtype, W=W, hq=hq, hkv=hkv, d=d, n_bs=n, m_bs=m_bs,
        k=k, ctx_len=ctx_len, kv_base=kv_base, pool_rows=pool_rows,
    )
    c["k_pool"] = normal(rng(seed_config, 1), (hkv, pool_rows, d), qkv_scale, dtype)
    c["v_pool"] = normal(rng(seed_config, 2), (hkv, pool_rows, d), qkv_scale, dtype)
    c["q"] = normal(rng(seed_config, 3), (m_bs, hq, d), qkv_scale, dtype)
    c["k_new"] = normal(rng(seed_config, 4), (m_bs, hkv, d), qkv_scale, dtype)
    c["v_new"] = normal(rng(seed_config, 5), (m_bs, hkv, d), qkv_scale, dtype)
    g = rng(seed_config, 6)
    tok_vocab = vocab if vocab else 32000
    c["block_tokens"] = g.integers(0, tok_vocab, size=(n, W)).astype(np.int32)
    c["vocab"] = vocab
    if vocab:
        if accepted is None:
            accepted = np.array([g.integers(0, max(1, int(x))) for x in k], np.int32)
        accepted = np.minimum(np.asarray(accepted, np.int32), np.maximum(k - 1, 0))
        logits, bt, planted = planted_logits(rng(seed_config, 7), k, vocab, m_bs, accepted,
                                             c["block_tokens"], W)
        c["logits"], c["block_tokens"], c["planted_argmax"] = logits, bt, planted
        c["planted_accepted"] = np.where(k > 0, accepted, 0).astype(np.int32)
    else:
        c["logits"] = None
    if draft_vocab:
        c["draft_logits"] = draft_logits(seed_config, n, draft_vocab)
    else:
        c["draft_logits"] = None
    c["prefill"] = None
    return c


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------
def config1() -> dict:
    """Tiny fp32 case: 2 requests, 2 query heads / 1 KV head, head_dim 64, contexts 32 and
    48, prefixes [3, 4] in 7 slots; logits [7, 1000]; the first two drafts of each request
    equal the target's choice, the next one does not."""
    return make_case(1, dtype="f32", hq=2, hkv=1, d=64, k=[3, 4], ctx_len=[32, 48], m_bs=7,
                     vocab=1000, accepted=[2, 2])


def config2() -> tuple[dict, dict]:
    """Layout shift, bf16: 3 requests, 32/8 heads, head_dim 128, contexts U[1024, 2048].
    Step 1 prefixes [4, 12, 8], step 2 [10, 8, 6] (24 slots each).  Step 2's contexts are the
    step-1 contexts advanced by the planted progress (anchor + accepted drafts committed);
    both steps share one pool whose segments hold ctx + 2W rows."""
    g = rng(2, 0)
    ctx1 = g.integers(1024, 2049, size=3).astype(np.int32)
    s1 = make_case(2, dtype="bf16", hq=32, hkv=8, d=128, k=[4, 12, 8], ctx_len=ctx1, m_bs=24,
                   qkv_scale=0.5, vocab=32000, capacity_extra=2 * W_BLOCK)
    ctx2 = (ctx1 + 1 + s1["planted_accepted"]).astype(np.int32)
    s2 = make_case(20, dtype="bf16", hq=32, hkv=8, d=128, k=[10, 8, 6], ctx_len=ctx2, m_bs=24,
                   qkv_scale=0.5, vocab=32000, capacity_extra=2 * W_BLOCK)
    # step 2 continues in step 1's pool: same segment bases, same pool tensors
    s2["kv_base"] = s1["kv_base"].copy()
    s2["pool_rows"] = s1["pool_rows"]
    s2["k_pool"], s2["v_pool"] = s1["k_pool"], s1["v_pool"]
    s1["name"], s2["name"] = "cfg2-step1", "cfg2-step2"
    return s1, s2


def config3(with_logits: bool = True) -> dict:
    """Full-width verify, bf16: 8 requests x 16 slots, 32/8 heads, head_dim 128, context 8192;
    logits [128, 151936] with accepted drafts ~ min(Poisson(5.09), 15)."""
    g = rng(3, 0)
    acc = np.minimum(g.poisson(5.09, size=8), 15).astype(np.int32)
    return make_case(3, dtype="bf16", hq=32, hkv=8, d=128, k=[16] * 8, ctx_len=[8192] * 8,
                     m_bs=128, qkv_scale=0.5, vocab=151936 if with_logits else None, accepted=acc)


def config4(with_draft_logits: bool = True) -> dict:
    """Reduced 8N budget, bf16: 32 requests sharing 256 slots (lengths 1..16, mean ~6, long
    tail), 24/2 heads, head_dim 256, contexts U[4096, 8192]; draft logits [32, 15, 248320]."""
    g = rng(4, 0)
    k = lengths_geometric_rescaled(g, 32, 256)
    ctx = g.integers(4096, 8193, size=32).astype(np.int32)
    return make_case(4, dtype="bf16", hq=24, hkv=2, d=256, k=k, ctx_len=ctx, m_bs=256,
                     qkv_scale=0.5, draft_vocab=248320 if with_draft_logits else None)


def config5(draw: bool = True) -> dict:
    """Mixed launch, bf16: 4 prefill requests x 4096 causal rows (fresh, context 0) plus 60
    verification requests with ragged prefixes in a 480-slot budget and contexts
    U[8192, 32768]; 32/8 heads, head_dim 128.  The prefill rows' K/V are already in the pool,
    in segments after the verification segments.  draw=False gives the layout only (lengths,
    segments, tokens), without the ~5 GB of pool, query and candidate tensors."""
    g = rng(5, 0)
    k = lengths_geometric_rescaled(g, 60, 480)
    ctx = g.integers(8192, 32769, size=60).astype(np.int32)
    return make_mixed_case(5, hq=32, hkv=8, d=128, k=k, ctx_len=ctx, m_bs=480,
                           pf_q_len=[4096] * 4, pf_ctx=[0] * 4, qkv_scale=0.5, draw=draw)


def make_mixed_case(seed_config: int, *, hq, hkv, d, k, ctx_len, m_bs, pf_q_len, pf_ctx,
                    qkv_scale=0.5, dtype="bf16", draw: bool = True) -> dict:
    """Verification batch plus prefill requests sharing one pool.  Prefill request r has
    pf_q_len[r] query rows at positions pf_ctx[r] .. pf_ctx[r] + len - 1; its segment holds
    pf_ctx[r] + pf_q_len[r] rows, all already in the pool.  draw=False leaves the pool, query
    and candidate tensors out (None)."""
    k = np.asarray(k, np.int32)
    ctx_len = np.asarray(ctx_len, np.int32)
    pf_q_len = np.asarray(pf_q_len, np.int32)
    pf_ctx = np.asarray(pf_ctx, np.int32)
    kv_base, v_rows = segments(ctx_len, W_BLOCK)
    pf_base, pf_rows = segments(pf_ctx + pf_q_len, 0)
    pf_base = pf_base + v_rows
    pool_rows = v_rows + pf_rows
    n = len(k)
    c = dict(name=f"cfg{seed_config}", dtype=dtype, W=W_BLOCK, hq=hq, hkv=hkv, d=d, n_bs=n,
             m_bs=m_bs, k=k, ctx_len=ctx_len, kv_base=kv_base, pool_rows=pool_rows)
    for key, t, shape in (("k_pool", 1, (hkv, pool_rows, d)), ("v_pool", 2, (hkv, pool_rows, d)),
                          ("q", 3, (m_bs, hq, d)), ("k_new", 4, (m_bs, hkv, d)), ("v_new", 5, (m_bs, hkv, d))):
        c[key] = normal(rng(seed_config, t), shape, qkv_scale, dtype) if draw else None
    c["block_tokens"] = rng(seed_config, 6).integers(0, 32000, size=(n, W_BLOCK)).astype(np.int32)
    c["vocab"] = None
    c["logits"] = None
    c["draft_logits"] = None
    q_start = np.zeros(len(pf_q_len), np.int32)
    if len(pf_q_len) > 1:
        q_start[1:] = np.cumsum(pf_q_len)[:-1]
    c["prefill"] = dict(
        n_pf=len(pf_q_len), q_start=q_start, q_len=pf_q_len, ctx_len=pf_ctx, kv_base=pf_base,
        q=normal(rng(seed_config, 9), (int(pf_q_len.sum()), hq, d), qkv_scale, dtype) if draw else None,
        max_len=int(pf_q_len.max()) if len(pf_q_len) else 0,
    )
    return c


def sentinel_variant(case: dict) -> dict:
    """Leak detector: candidate V rows x100 (a causal leak changes outputs by O(1)), and
    every pool row at or past ctx_i poisoned with NaN (any read of a row the request must not
    see from the pool turns its outputs into NaN).  The candidate rows then come only from
    k_new / v_new."""
    assert case["dtype"] == "bf16"
    c = dict(case)
    c["name"] = case["name"] + "-sentinel"
    vn = bf16_bits_to_f32(case["v_new"]) * np.float32(100.0)
    c["v_new"] = to_bf16_bits(vn)
    kp = case["k_pool"].copy()
    vp = case["v_pool"].copy()
    for i in range(case["n_bs"]):
        b, cx = int(case["kv_base"][i]), int(case["ctx_len"][i])
        end = int(case["kv_base"][i + 1]) if i + 1 < case["n_bs"] else case["pool_rows"]
        kp[:, b + cx:end, :] = BF16_NAN
        vp[:, b + cx:end, :] = BF16_NAN
    c["k_pool"], c["v_pool"] = kp, vp
    return c


def sharp_variant(case: dict) -> dict:
    """Queries x8: peaked softmax, so a wrong key or a wrong scale moves outputs visibly."""
    c = dict(case)
    c["name"] = case["name"] + "-sharp"
    if case["dtype"] == "bf16":
        c["q"] = to_bf16_bits(bf16_bits_to_f32(case["q"]) * np.float32(8.0))
    else:
        c["q"] = case["q"] * np.float32(8.0)
    return c
