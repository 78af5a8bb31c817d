"""Pins for the oracle's verification and prefill attention.

The attention the method computes is ordinary masked softmax attention; packing and tile
routing only reorganise it (DScale Sec. III-B/III-D).  The oracle is pinned to:
  * the three formulations agreeing exactly (packed / one request at a time / padded with a
    materialised mask),
  * softmax rows summing to one,
  * closed forms (constant V, all-zero K, one dominant key),
  * torch's fp64 CPU scaled_dot_product_attention on the special cases that reduce to it
    (single-query decode, textbook causal prefill), with an explicit boolean mask,
  * brute force on the tiny fp32 workload (materialised mask and probabilities).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _small_case(seed=11, dtype="bf16", hq=4, hkv=2, d=32, k=(3, 16, 1, 0, 7), ctx=(5, 40, 0, 9, 70),
                extra_tail=3):
    k = np.asarray(k, np.int32)
    return wl.make_case(seed, dtype=dtype, hq=hq, hkv=hkv, d=d, k=k, ctx_len=ctx,
                        m_bs=int(k.sum()) + extra_tail, qkv_scale=0.7)


def _offsets(c):
    return oracle.pack(c["k"], c["ctx_len"], c["kv_base"], c["block_tokens"], c["W"], c["m_bs"])["offsets"]


def _f64(a):
    if a.dtype == np.uint16:
        return wl.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _run3(c, use_new=True):
    off = _offsets(c)
    kn = c["k_new"] if use_new else None
    vn = c["v_new"] if use_new else None
    args = (c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"], c["kv_base"])
    p = oracle.verify_attn(*args, k_new=kn, v_new=vn)
    r = oracle.attn_per_request(*args, k_new=kn, v_new=vn)
    pad = oracle.attn_padded(*args, c["W"], k_new=kn, v_new=vn)
    return off, p, r, pad


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("use_new", [True, False])
def test_three_formulations_agree(dtype, use_new):
    c = _small_case(dtype=dtype)
    off, (po, pl), (ro, rl), (ao, al) = _run3(c, use_new)
    end = int(off[-1])
    assert np.array_equal(po[:end], ro[:end]) and np.array_equal(pl[:end], rl[:end])
    assert np.array_equal(po[:end], ao[:end]) and np.array_equal(pl[:end], al[:end])
    assert np.all(po[end:] == 0) and np.all(np.isneginf(pl[end:]))
    assert np.all(np.isfinite(po[:end]))


def test_softmax_rows_sum_to_one():
    r = np.random.default_rng(5)
    for n in (1, 2, 17, 300):
        q = wl.to_bf16_bits(r.standard_normal(64).astype(np.float32) * 3)
        K = wl.to_bf16_bits(r.standard_normal((n, 64)).astype(np.float32))
        p = oracle.softmax_probs(q, K)
        assert abs(p.sum() - 1.0) <= 1e-12 and np.all(p >= 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_probs_match_scipy(dtype):
    """The materialised weights equal scipy's softmax of scale * K q (a library routine
    independent of the oracle), for the default scale 1/sqrt(d) and for a given one, on
    random rows and on a row where one planted key dominates."""
    from scipy.special import softmax

    r = np.random.default_rng(6)
    conv = wl.to_bf16_bits if dtype == "bf16" else (lambda a: a.astype(np.float32))
    for n, d, scale in ((1, 16, 0.0), (7, 32, 0.0), (40, 64, 0.37), (300, 128, 1.9)):
        q = conv(r.standard_normal(d).astype(np.float32))
        K = conv(r.standard_normal((n, d)).astype(np.float32))
        p = oracle.softmax_probs(q, K, scale)
        s = scale if scale > 0 else 1.0 / np.sqrt(d)
        want = softmax(s * (_f64(K) @ _f64(q)))
        assert np.allclose(p, want, rtol=1e-12, atol=1e-300), (n, d, scale)
    # one key aligned with q and scaled up takes (almost) all the weight, at its own index
    d, n, hot = 32, 50, 37
    q = conv(np.ones(d, np.float32))
    K = np.zeros((n, d), np.float32)
    K[hot] = 1.0
    p = oracle.softmax_probs(q, conv(K), 0.5)
    assert int(np.argmax(p)) == hot and p[hot] > 1 - 1e-5
    assert np.allclose(p[np.arange(n) != hot], np.exp(-16.0) / (np.exp(-16.0) * (n - 1) + 1.0), rtol=1e-12)


def test_scatter_candidates_hand_built():
    """Candidate K/V rows land exactly at their cache references, in every KV head; a -1
    reference writes nothing; every other pool row and the inputs are unchanged.  Expected
    pools are written out by hand."""
    hkv, rows, d = 2, 6, 3
    k_pool = np.arange(hkv * rows * d, dtype=np.float32).reshape(hkv, rows, d)  # value = index
    v_pool = -k_pool
    k_in, v_in = k_pool.copy(), v_pool.copy()
    # three slots: slot 0 -> row 4, slot 1 -> tail placeholder (-1), slot 2 -> row 0
    k_new = np.array([[[100, 101, 102], [110, 111, 112]],
                      [[200, 201, 202], [210, 211, 212]],
                      [[300, 301, 302], [310, 311, 312]]], np.float32)
    v_new = k_new + 0.5
    kp, vp = oracle.scatter_candidates(k_pool, v_pool, k_new, v_new, np.array([4, -1, 0], np.int64))
    want_k = np.array([[[300, 301, 302], [3, 4, 5], [6, 7, 8], [9, 10, 11], [100, 101, 102], [15, 16, 17]],
                       [[310, 311, 312], [21, 22, 23], [24, 25, 26], [27, 28, 29], [110, 111, 112], [33, 34, 35]]],
                      np.float32)
    want_v = np.array([[[300.5, 301.5, 302.5], [-3, -4, -5], [-6, -7, -8], [-9, -10, -11],
                        [100.5, 101.5, 102.5], [-15, -16, -17]],
                       [[310.5, 311.5, 312.5], [-21, -22, -23], [-24, -25, -26], [-27, -28, -29],
                        [110.5, 111.5, 112.5], [-33, -34, -35]]], np.float32)
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)
    assert np.array_equal(k_pool, k_in) and np.array_equal(v_pool, v_in)  # copies, not in place


def _sequence(c, i, off):
    """Request i's key/value sequence in position order (context rows, then k_new)."""
    b, cx, kk = int(c["kv_base"][i]), int(c["ctx_len"][i]), int(c["k"][i])
    K = _f64(c["k_pool"][:, b:b + cx + kk]).copy()
    V = _f64(c["v_pool"][:, b:b + cx + kk]).copy()
    K[:, cx:cx + kk] = np.transpose(_f64(c["k_new"][off[i]:off[i] + kk]), (1, 0, 2))
    V[:, cx:cx + kk] = np.transpose(_f64(c["v_new"][off[i]:off[i] + kk]), (1, 0, 2))
    return K, V


def test_closed_forms():
    c = _small_case(seed=12, dtype="f32", hq=2, hkv=1, d=16, k=(4, 2), ctx=(10, 3))
    off = _offsets(c)
    # constant V -> output equals that constant row
    const = np.linspace(-2, 2, 16).astype(np.float32)
    c1 = dict(c, v_pool=np.broadcast_to(const, c["v_pool"].shape).copy(),
              v_new=np.broadcast_to(const, c["v_new"].shape).copy())
    o, _ = oracle.verify_attn(c1["q"], c1["k_pool"], c1["v_pool"], off, c1["k"], c1["ctx_len"],
                              c1["kv_base"], c1["k_new"], c1["v_new"])
    assert np.allclose(o[: off[-1]], const, atol=1e-12)
    # all-zero K -> uniform weights: output is the mean of the visible V rows, lse = ln(n)
    c2 = dict(c, k_pool=np.zeros_like(c["k_pool"]), k_new=np.zeros_like(c["k_new"]))
    o, l = oracle.verify_attn(c2["q"], c2["k_pool"], c2["v_pool"], off, c2["k"], c2["ctx_len"],
                              c2["kv_base"], c2["k_new"], c2["v_new"])
    for i in range(c["n_bs"]):
        _, V = _sequence(c2, i, off)
        for j in range(int(c["k"][i])):
            n = int(c["ctx_len"][i]) + j + 1
            s = off[i] + j
            assert np.allclose(o[s, 0], V[0, :n].mean(axis=0), atol=1e-12)
            assert abs(l[s, 0] - np.log(n)) < 1e-12
    # one dominant key -> output is (almost exactly) that key's V row
    c3 = dict(c, k_pool=np.zeros_like(c["k_pool"]), k_new=np.zeros_like(c["k_new"]))
    q = np.zeros_like(c["q"])
    q[:, :, 0] = 1.0
    kp = c3["k_pool"].copy()
    b = int(c["kv_base"][0])
    kp[0, b + 5, 0] = 60.0  # position 5 of request 0 dominates by e^15
    o, _ = oracle.verify_attn(q, kp, c3["v_pool"], off, c3["k"], c3["ctx_len"], c3["kv_base"],
                              c3["k_new"], c3["v_new"])
    assert np.allclose(o[0, 0], c3["v_pool"][0, b + 5], atol=1e-4)


def _sdpa(qrows, K, V, mask, scale):
    """torch fp64 CPU SDPA with an explicit boolean mask: qrows [n_q, d], K/V [n_k, d]."""
    q = torch.from_numpy(qrows)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    m = torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0, 0].numpy()


def test_single_query_decode_matches_sdpa():
    """k_i = 1 (anchor only) is plain single-query decode attention over ctx + 1 keys."""
    c = _small_case(seed=13, dtype="bf16", hq=4, hkv=2, d=32, k=(1, 1, 1), ctx=(0, 31, 200), extra_tail=0)
    off = _offsets(c)
    o, l = oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"],
                              c["kv_base"], c["k_new"], c["v_new"])
    q64 = _f64(c["q"])
    for i in range(3):
        K, V = _sequence(c, i, off)
        for h in range(4):
            g = h // 2
            n = K.shape[1]
            ref = _sdpa(q64[off[i], h][None], K[g], V[g], np.ones((1, n), bool), 1 / np.sqrt(32))
            assert np.allclose(o[off[i], h], ref[0], rtol=1e-12, atol=1e-12)
            z = (K[g] @ q64[off[i], h]) / np.sqrt(32)
            assert abs(l[off[i], h] - torch.logsumexp(torch.from_numpy(z), 0).item()) < 1e-12


def test_verify_block_matches_sdpa_with_mask():
    """A full 16-slot block over a context: rows see the whole context and a causal prefix of
    the block (DScale Sec. III-D request-local causal mask)."""
    c = _small_case(seed=14, dtype="f32", hq=6, hkv=2, d=16, k=(16, 5), ctx=(23, 0), extra_tail=2)
    off = _offsets(c)
    o, _ = oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"],
                              c["kv_base"], c["k_new"], c["v_new"])
    q64 = _f64(c["q"])
    for i in range(2):
        K, V = _sequence(c, i, off)
        kk, cx = int(c["k"][i]), int(c["ctx_len"][i])
        mask = np.zeros((kk, cx + kk), bool)
        for j in range(kk):
            mask[j, : cx + j + 1] = True
        for h in range(6):
            ref = _sdpa(q64[off[i]:off[i] + kk, h], K[h // 3], V[h // 3], mask, 0.25)
            assert np.allclose(o[off[i]:off[i] + kk, h], ref, rtol=1e-12, atol=1e-12)


def test_prefill_matches_textbook_causal():
    """Fresh prefill (context 0) is textbook causal attention (is_causal=True in SDPA)."""
    r = wl.rng(99, 0)
    hq, hkv, d, L = 4, 1, 32, 70
    pool_k = wl.normal(r, (hkv, 200, d), 0.8, "bf16")
    pool_v = wl.normal(r, (hkv, 200, d), 0.8, "bf16")
    q = wl.normal(r, (L + 30, hq, d), 0.8, "bf16")
    # request 0: rows 0..L-1 at pool rows 100.., request 1: 30 rows after a 12-row context
    q_start, q_len, ctx, base = [0, L], [L, 30], [0, 12], [100, 40]
    sel_req = [0] * L + [1] * 30
    sel_j = list(range(L)) + list(range(30))
    o, l = oracle.prefill_attn(q, pool_k, pool_v, q_start, q_len, ctx, base, sel_req, sel_j)
    qq = torch.from_numpy(_f64(q[:L]).transpose(1, 0, 2))[None]
    kk = torch.from_numpy(_f64(pool_k[:, 100:100 + L]))[None].expand(1, hq, L, d)
    vv = torch.from_numpy(_f64(pool_v[:, 100:100 + L]))[None].expand(1, hq, L, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True)[0].numpy()
    assert np.allclose(o[:L], ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)
    # request 1 with context: explicit mask over 12 + 30 keys
    K = _f64(pool_k[0, 40:40 + 42])
    V = _f64(pool_v[0, 40:40 + 42])
    mask = np.zeros((30, 42), bool)
    for j in range(30):
        mask[j, : 12 + j + 1] = True
    for h in range(hq):
        ref = _sdpa(_f64(q[L:L + 30, h]), K, V, mask, 1 / np.sqrt(d))
        assert np.allclose(o[L:, h], ref, rtol=1e-12, atol=1e-12)


def test_prefill_equals_verify_on_short_rows():
    """A prefill request with <= W rows is the same computation as a verification request
    whose candidates already sit in the pool (different oracle entry points)."""
    c = _small_case(seed=15, dtype="bf16", hq=4, hkv=2, d=32, k=(6, 9), ctx=(17, 4), extra_tail=0)
    off = _offsets(c)
    o_v, l_v = oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"], c["kv_base"])
    sel_req = [0] * 6 + [1] * 9
    sel_j = list(range(6)) + list(range(9))
    o_p, l_p = oracle.prefill_attn(c["q"], c["k_pool"], c["v_pool"], off[:-1], c["k"], c["ctx_len"],
                                   c["kv_base"], sel_req, sel_j)
    assert np.array_equal(o_v, o_p) and np.array_equal(l_v, l_p)


def test_config1_bruteforce():
    """Tiny fp32 workload: brute force with a materialised mask and probabilities."""
    c = wl.config1()
    off = _offsets(c)
    o, l = oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"],
                              c["kv_base"], c["k_new"], c["v_new"])
    q64 = _f64(c["q"])
    for i in range(2):
        K, V = _sequence(c, i, off)
        n_all = K.shape[1]
        for j in range(int(c["k"][i])):
            visible = np.arange(n_all) <= int(c["ctx_len"][i]) + j
            for h in range(2):
                z = np.where(visible, K[0] @ q64[off[i] + j, h] / 8.0, -np.inf)
                p = np.exp(z - z.max())
                p /= p.sum()
                assert np.allclose(o[off[i] + j, h], p @ V[0], rtol=1e-12, atol=1e-13)
                assert abs(l[off[i] + j, h] - (z.max() + np.log(np.exp(z - z.max()).sum()))) < 1e-12


def test_errors():
    c = _small_case(seed=16)
    off = _offsets(c)
    bad = c["kv_base"].copy()
    bad[-1] = c["pool_rows"]  # segment past the pool
    with pytest.raises(oracle.OracleError):
        oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"], bad)


def _scatter_pool(c, seed, share=False):
    """The same case with every pool row moved to a random place and a token-granular cache
    map [n_bs, ctx + W] pointing at it (DScale Sec. III-D: historyKV gathered through
    cacheMap).  With share=True request 1's first context rows alias request 0's (a shared
    prefix)."""
    rng = np.random.default_rng(seed)
    hkv, rows, d = c["k_pool"].shape
    perm = rng.permutation(rows)  # row r moves to perm[r]
    kp = np.empty_like(c["k_pool"])
    vp = np.empty_like(c["v_pool"])
    kp[:, perm] = c["k_pool"]
    vp[:, perm] = c["v_pool"]
    n_bs = len(c["k"])
    stride = int((c["ctx_len"] + c["W"]).max())
    idx = np.full((n_bs, stride), -1, np.int32)
    for i in range(n_bs):
        n = int(c["ctx_len"][i] + c["k"][i])
        idx[i, :n] = perm[int(c["kv_base"][i]) + np.arange(n)]
    if share:
        n = int(min(c["ctx_len"][0], c["ctx_len"][1]))
        idx[1, :n] = idx[0, :n]
    return kp, vp, idx


@pytest.mark.parametrize("use_new", [True, False])
def test_cache_map_equals_contiguous_segments(use_new):
    """Reading rows through a token-granular cache map of a permuted pool gives exactly the
    contiguous-segment result (the gather is an addressing change only)."""
    c = _small_case(seed=21, dtype="bf16")
    off = _offsets(c)
    kn = c["k_new"] if use_new else None
    vn = c["v_new"] if use_new else None
    base = oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], off, c["k"], c["ctx_len"], c["kv_base"], kn, vn)
    kp, vp, idx = _scatter_pool(c, 5)
    mapped = oracle.verify_attn(c["q"], kp, vp, off, c["k"], c["ctx_len"], c["kv_base"], kn, vn, kv_index=idx)
    end = int(off[-1])
    assert np.array_equal(base[0][:end], mapped[0][:end]) and np.array_equal(base[1][:end], mapped[1][:end])


def test_cache_map_shared_prefix_matches_sdpa():
    """A cache map whose requests share context rows: every row equals fp64 SDPA over the
    gathered keys with the request-local causal mask."""
    c = _small_case(seed=22, dtype="f32", hq=4, hkv=2, d=16, k=(5, 9), ctx=(30, 20), extra_tail=0)
    off = _offsets(c)
    kp, vp, idx = _scatter_pool(c, 6, share=True)
    o, _ = oracle.verify_attn(c["q"], kp, vp, off, c["k"], c["ctx_len"], c["kv_base"], c["k_new"],
                              c["v_new"], kv_index=idx)
    q64 = _f64(c["q"])
    for i in range(2):
        kk, cx = int(c["k"][i]), int(c["ctx_len"][i])
        rows = idx[i, :cx]
        for h in range(4):
            g = h // 2
            K = np.concatenate([_f64(kp[g, rows]), _f64(c["k_new"][off[i]:off[i] + kk, g])])
            V = np.concatenate([_f64(vp[g, rows]), _f64(c["v_new"][off[i]:off[i] + kk, g])])
            mask = np.zeros((kk, cx + kk), bool)
            for j in range(kk):
                mask[j, : cx + j + 1] = True
            ref = _sdpa(q64[off[i]:off[i] + kk, h], K, V, mask, 1 / np.sqrt(16))
            assert np.allclose(o[off[i]:off[i] + kk, h], ref, rtol=1e-12, atol=1e-12)


def test_cache_map_errors():
    c = _small_case(seed=23, dtype="bf16")
    off = _offsets(c)
    kp, vp, idx = _scatter_pool(c, 7)
    bad = idx.copy()
    bad[0, 0] = kp.shape[1]  # a row past the pool
    with pytest.raises(oracle.OracleError):
        oracle.verify_attn(c["q"], kp, vp, off, c["k"], c["ctx_len"], c["kv_base"], c["k_new"], c["v_new"],
                           kv_index=bad)
    short = idx[:, :3]  # fewer entries than a request's visible positions
    with pytest.raises(oracle.OracleError):
        oracle.verify_attn(c["q"], kp, vp, off, c["k"], c["ctx_len"], c["kv_base"], c["k_new"], c["v_new"],
                           kv_index=short)
