"""Pins for the oracle's greedy prefix verifier, argmax and draft margin.

DScale Sec. III-D (Prefix verifier: after a_i accepted candidates, row offset_i + a_i
supplies the successor; progress = one anchor plus accepted drafts, Sec. II-B) and
DFlash-Mini-Lab (the anchor is never drafted; accept the exact prefix; top-1/top-2 draft
margin).  Pinned to planted answers, numpy's documented first-occurrence argmax, brute force
over the accepted length, and numpy sorting for the margin."""
import numpy as np
import pytest

import oracle
import workloads as wl


def test_argmax_matches_numpy_first_occurrence():
    r = np.random.default_rng(0)
    x = r.standard_normal((50, 777)).astype(np.float32)
    x[3, 10] = x[3, 500] = 9.0           # tie -> lowest index
    x[4, :] = 0.0                         # all equal -> index 0
    x[5, 7] = -0.0
    x[5, :] = -1.0
    x[5, 7] = -0.0
    x[5, 2] = 0.0                         # -0.0 == +0.0: first index (2) wins
    x[6, :] = -np.inf
    x[6, 600] = -1e30
    got = oracle.argmax_rows(x)
    assert np.array_equal(got, np.argmax(x, axis=1))
    assert got[3] == 10 and got[4] == 0 and got[5] == 2 and got[6] == 600


def test_argmax_nan_is_error():
    x = np.zeros((2, 5), np.float32)
    x[1, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.argmax_rows(x)


def _bruteforce_accept(slot_tok, g, off, k):
    """Largest a <= k-1 such that drafts 1..a all equal the target choice one slot earlier."""
    best = 0
    for a in range(k):
        if all(slot_tok[off + j] == g[off + j - 1] for j in range(1, a + 1)):
            best = a
    return best


@pytest.mark.parametrize("cfg", [1, 2])
def test_planted_acceptance(cfg):
    c = wl.config1() if cfg == 1 else wl.config2()[0]
    p = oracle.pack(c["k"], c["ctx_len"], c["kv_base"], c["block_tokens"], c["W"], c["m_bs"])
    out = oracle.accept(c["logits"], p["slot_tok"], p["offsets"], c["k"], c["W"])
    assert np.array_equal(out["accepted"], c["planted_accepted"])
    assert np.array_equal(out["progress"], np.where(c["k"] > 0, 1 + c["planted_accepted"], 0))
    end = int(p["offsets"][-1])
    for i in range(c["n_bs"]):
        for j in range(int(c["k"][i])):
            assert out["slot_argmax"][p["offsets"][i] + j] == c["planted_argmax"][i, j]
    assert np.all(out["slot_argmax"][end:] == -1)
    if cfg == 1:
        assert list(out["accepted"]) == [2, 2] and list(out["progress"]) == [3, 3]


def test_accept_bruteforce_random():
    r = np.random.default_rng(7)
    for trial in range(200):
        W = int(r.integers(1, 17))
        n = int(r.integers(1, 6))
        k = r.integers(0, W + 1, size=n).astype(np.int32)
        m_bs = int(k.sum()) + int(r.integers(0, 3))
        vocab = int(r.integers(2, 6))  # tiny vocab: matches happen often
        logits = r.standard_normal((max(m_bs, 1), vocab)).astype(np.float32)[:m_bs]
        tokens = r.integers(0, vocab, size=(n, W)).astype(np.int32)
        p = oracle.pack(k, np.zeros(n, np.int32), np.zeros(n, np.int64), tokens, W, m_bs)
        out = oracle.accept(logits, p["slot_tok"], p["offsets"], k, W)
        g = np.argmax(logits, axis=1) if m_bs else np.zeros(0, int)
        for i in range(n):
            off = int(p["offsets"][i])
            if k[i] == 0:
                assert (out["accepted"][i], out["bonus"][i], out["progress"][i]) == (0, -1, 0)
                assert np.all(out["out_tokens"][i] == -1)
                continue
            a = _bruteforce_accept(p["slot_tok"], g, off, int(k[i]))
            assert out["accepted"][i] == a
            assert out["bonus"][i] == g[off + a]
            assert 1 <= out["progress"][i] == 1 + a <= k[i] <= W
            expect = [int(p["slot_tok"][off + 1 + t]) for t in range(a)] + [int(g[off + a])]
            assert list(out["out_tokens"][i][: a + 1]) == expect
            assert np.all(out["out_tokens"][i][a + 1:] == -1)


def test_anchor_is_never_checked():
    """The anchor (j = 0) is the known token; only drafts are compared (DFlash-Mini-Lab)."""
    logits = np.zeros((3, 4), np.float32)
    logits[:, 2] = 1.0  # every row predicts token 2
    k = np.array([3], np.int32)
    tokens = np.array([[3, 2, 2]], np.int32)  # anchor 3 differs from anything; drafts match
    p = oracle.pack(k, [0], [0], tokens, 3, 3)
    out = oracle.accept(logits, p["slot_tok"], p["offsets"], k, 3)
    assert out["accepted"][0] == 2 and out["bonus"][0] == 2 and out["progress"][0] == 3


def test_margin_matches_numpy_sort():
    r = np.random.default_rng(3)
    x = r.standard_normal((4, 15, 301)).astype(np.float32)
    x[0, 0, 5] = x[0, 0, 9] = 7.0   # duplicated maximum -> margin 0, top1 = first index
    x[1, 3, :] = 2.5                # constant row
    m, t = oracle.top2_margin(x)
    s = -np.sort(-x, axis=-1)
    assert np.array_equal(m, (s[..., 0] - s[..., 1]).astype(np.float32))  # fp32 subtraction
    assert np.array_equal(t, np.argmax(x, axis=-1))
    assert m[0, 0] == 0.0 and t[0, 0] == 5 and m[1, 3] == 0.0 and t[1, 3] == 0


def test_margin_is_correctly_rounded():
    """Cases where the exact difference needs more than 24 bits."""
    x = np.array([[1.0, np.float32(1e-8), -3.0], [np.float32(16777216.0), 1.0, 0.0],
                  [np.float32(3.0000002), np.float32(-1.1754944e-38), 0.5]], np.float32)
    m, _ = oracle.top2_margin(x)
    exact = [np.float32(np.float64(1.0) - np.float64(np.float32(1e-8))),
             np.float32(np.float64(16777216.0) - 1.0),
             np.float32(np.float64(np.float32(3.0000002)) - 0.5)]
    assert np.array_equal(m, np.array(exact, np.float32))
    assert np.array_equal(m, x.max(1) - np.sort(x, 1)[:, -2])
