"""GPU parity of dsv_accept_sample (sampling-mode prefix verifier) against the oracle on the
same logits and uniforms: accepted lengths, successors, progress and output tokens
bit-exact, P(x) per tested row within fp32 rounding.

The decisions are floating-point comparisons (u < P(x), and u * S against the cumulative
weights), which the kernels take in fp32 (P) and fp64 (the draw) and the oracle in fp64.
Every fixture asserts, from the oracle's decision margins, that no decision lies within the
kernels' rounding error of its threshold (1e-5 for u - P, whose fp32 error is ~1e-6; 1e-9
of the total weight for the draw), so both sides must agree exactly."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import DEV, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402

ACC_MARGIN = 1e-5
DRAW_MARGIN = 1e-9


def _gpu_sample(logits, slot_tok, offsets, k, W, T, u_acc, u_draw, logits_dev=None):
    st = dsv.new_status(DEV)
    o = dsv.accept_sample(
        n_bs=len(k), W=W, status=st,
        target_logits=logits_dev if logits_dev is not None else to_dev(np.ascontiguousarray(logits, np.float32)),
        temperature=T, slot_tok=to_dev(np.asarray(slot_tok, np.int32)),
        offsets=to_dev(np.asarray(offsets, np.int32)), k=to_dev(np.asarray(k, np.int32)),
        u_accept=to_dev(np.asarray(u_acc, np.float32)), u_draw=to_dev(np.asarray(u_draw, np.float32)))
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in o.items()}, int(st.item())


def _case(seed, n_bs, W, vocab, *, tail=0, boost=(4.0, 12.0), p_random=0.2, k=None):
    g = np.random.default_rng(seed)
    if k is None:
        k = g.integers(0, W + 1, n_bs).astype(np.int32)
    k = np.asarray(k, np.int32)
    m_bs = int(k.sum()) + tail
    bt = g.integers(0, vocab, (len(k), W)).astype(np.int32)
    logits, bt = wl.sampling_logits(g, k, vocab, m_bs, bt, boost=boost, p_random=p_random, W=W)
    p = oracle.pack(k, np.zeros(len(k), np.int32), np.zeros(len(k), np.int64), bt, W, m_bs)
    return dict(logits=logits, slot_tok=p["slot_tok"], offsets=p["offsets"], k=k, W=W,
                u_acc=wl.uniforms(g, m_bs), u_draw=wl.uniforms(g, len(k)))


def _check(c, T, tag, logits_dev=None):
    ref = oracle.accept_sample(c["logits"], c["slot_tok"], c["offsets"], c["k"], c["W"], T,
                               c["u_acc"], c["u_draw"])
    am = ref["acc_margin"][~np.isnan(ref["acc_margin"])]
    dm = ref["draw_margin"][~np.isnan(ref["draw_margin"])]
    assert am.size == 0 or am.min() > ACC_MARGIN, f"{tag}: fixture has an accept decision at its threshold"
    assert dm.size == 0 or dm.min() > DRAW_MARGIN, f"{tag}: fixture has a draw at a boundary"
    got, st = _gpu_sample(c["logits"], c["slot_tok"], c["offsets"], c["k"], c["W"], T,
                          c["u_acc"], c["u_draw"], logits_dev=logits_dev)
    assert st == 0, f"{tag}: status {st}"
    for key in ("accepted", "bonus", "progress", "out_tokens"):
        assert np.array_equal(got[key], ref[key]), f"{tag}: {key}\n{got[key]}\n{ref[key]}"
    rows = ~np.isnan(ref["p_cand"])
    pc_ref, pc = ref["p_cand"][rows], got["p_cand"][rows].astype(np.float64)
    assert np.all(np.abs(pc - pc_ref) <= 1e-6 + 1e-5 * np.abs(pc_ref)), f"{tag}: p_cand"
    return got, ref


@pytest.mark.parametrize("vocab", [1, 2, 7, 1000, 4099, 32768])
@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_sample_parity_small(vocab, T):
    boost = (0.0, 8.0) if vocab >= 1000 else (0.0, 3.0)
    for trial in range(3):
        seed = 100 * vocab + 10 * trial + int(T * 10)
        g = np.random.default_rng(seed)
        n_bs, W = int(g.integers(1, 21)), int(g.integers(1, 17))
        c = _case(seed, n_bs, W, vocab, tail=int(g.integers(0, 5)), boost=boost)
        if c["logits"].shape[0] == 0:
            continue
        _check(c, T, f"vocab {vocab} T {T} trial {trial}")


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_sample_parity_full_width(T):
    # the full-width verification batch: 8 requests x 16 slots over the 151,936-token vocabulary
    c = _case(3000 + int(T * 10), 8, 16, 151936, k=[16] * 8)
    got, ref = _check(c, T, f"full width T {T}")
    # the fixture exercises both outcomes
    assert 0 < ref["accepted"].sum() < 8 * 15


def test_sample_many_requests():
    # more requests than chunks: one draw chunk per request, and many chunks per row
    c = _case(77, 200, 16, 50000, tail=3, boost=(2.0, 12.0))
    _check(c, 1.0, "200 requests")
    c = _case(78, 3, 16, 300000, boost=(6.0, 14.0))
    _check(c, 0.9, "300k vocabulary")


def test_sample_bad_nan_and_inactive():
    c = _case(5, 5, 16, 3000, k=[4, 3, 0, 5, 2], tail=2)
    lg = c["logits"].copy()
    off = c["offsets"]
    lg[off[0] + 1, 10] = np.nan          # request 0: NaN
    lg[off[1] + 2, 20] = np.inf          # request 1: +inf
    lg[off[3]:off[3] + 1] = -np.inf      # request 3: a row with no finite entry
    got, st = _gpu_sample(lg, c["slot_tok"], off, c["k"], 16, 1.0, c["u_acc"], c["u_draw"])
    assert st & dsv.STATUS_NAN and not st & dsv.STATUS_BAD_REQUEST
    for i in (0, 1, 3):
        assert got["accepted"][i] == -1 and got["bonus"][i] == -1 and got["progress"][i] == 0
        assert np.all(got["out_tokens"][i] == -1)
    assert got["accepted"][2] == 0 and got["bonus"][2] == -1 and got["progress"][2] == 0
    # request 4 is untouched by the others' bad rows: it matches the oracle run on it alone
    s4 = slice(off[4], off[4] + 2)
    ref = oracle.accept_sample(c["logits"][s4], c["slot_tok"][s4], [0, 2], [2], 16, 1.0,
                               c["u_acc"][s4], c["u_draw"][4:5])
    for key in ("accepted", "bonus", "progress", "out_tokens"):
        assert np.array_equal(got[key][4], ref[key][0]), key
    # malformed requests: k > W (request 3) and a prefix running past offsets[n_bs] (request 4)
    got, st = _gpu_sample(c["logits"], c["slot_tok"], [0, 4, 7, 7, 15, 16], [4, 3, 0, 17, 2], 16,
                          1.0, c["u_acc"], c["u_draw"])
    assert st & dsv.STATUS_BAD_REQUEST
    for i in (3, 4):
        assert got["accepted"][i] == -1 and got["progress"][i] == 0


def test_sample_marginals():
    # the device sampler on its own: two candidates, 32768 requests with seeded uniforms; every
    # emitted sequence has the probability of drawing its tokens from the rows that predict them
    g = np.random.default_rng(21)
    N, V = 32768, 6
    rows = np.array([[0.5, 1.0, -0.3, 0.0, 0.2, -1.0],
                     [-1.0, 0.4, 0.9, 0.1, 0.0, 0.3],
                     [0.0, -0.7, 0.3, 1.2, -0.2, 0.4]], np.float32)
    x1, x2 = 1, 2
    P = np.exp(rows.astype(np.float64))
    P /= P.sum(axis=1, keepdims=True)
    logits = np.tile(rows, (N, 1))
    slot_tok = np.tile(np.array([4, x1, x2], np.int32), N)
    offsets = np.arange(N + 1, dtype=np.int32) * 3
    got, st = _gpu_sample(logits, slot_tok, offsets, np.full(N, 3, np.int32), 16, 1.0,
                          wl.uniforms(g, 3 * N), wl.uniforms(g, N))
    assert st == 0
    expect = {}
    for y in range(V):
        if y != x1:
            expect[(y,)] = P[0][y]
        if y != x2:
            expect[(x1, y)] = P[0][x1] * P[1][y]
        expect[(x1, x2, y)] = P[0][x1] * P[1][x2] * P[2][y]
    counts = {}
    for t, p in zip(got["out_tokens"], got["progress"]):
        sq = tuple(int(v) for v in t[:p])
        counts[sq] = counts.get(sq, 0) + 1
    assert set(counts) <= set(expect)
    for sq, p in expect.items():
        f = counts.get(sq, 0) / N
        assert abs(f - p) <= 5 * np.sqrt(p * (1 - p) / N) + 1.0 / N, (sq, f, p)


def test_sample_host_errors():
    st = dsv.new_status(DEV)
    lg = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=DEV)  # noqa: E731
    u = torch.zeros(4, dtype=torch.float32, device=DEV)
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(dsv.DsvError):
            dsv.accept_sample(n_bs=1, W=16, status=st, target_logits=lg, temperature=T,
                              slot_tok=i32([0, 1, 2, 3]), offsets=i32([0, 4]), k=i32([4]),
                              u_accept=u, u_draw=u)
    with pytest.raises(dsv.DsvError):
        dsv.accept_sample(n_bs=1, W=17, status=st, target_logits=lg, temperature=1.0,
                          slot_tok=i32([0, 1, 2, 3]), offsets=i32([0, 4]), k=i32([4]),
                          u_accept=u, u_draw=u)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
