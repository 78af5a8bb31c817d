"""Pins of the sampling-mode prefix verifier of the oracle (DScale Sec. III-D "Prefix
verifier": accept the top-1 draft x with probability P(x); at the first rejection draw the
successor from P with x removed and renormalised; after all candidates pass, draw from the
unmodified P).  The identity that makes the rule exact -- every emitted token is distributed
as the target's P at its position -- is checked on stratified grids (exact up to the grid
resolution) and with seeded uniforms (binomial bounds); closed forms pin the inverse-CDF draw
and the temperature."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle

W = 16


def _batch(rows, n_req, tokens):
    """n_req identical requests of len(rows) slots each: logits, slot_tok, offsets, k."""
    k = len(rows)
    logits = np.tile(np.asarray(rows, np.float32), (n_req, 1))
    slot_tok = np.tile(np.asarray(tokens, np.int32), n_req)
    offsets = np.arange(n_req + 1, dtype=np.int32) * k
    return logits, slot_tok, offsets, np.full(n_req, k, np.int32)


def test_uniform_row_draw_is_floor():
    # equal logits: P is uniform over V, so the inverse CDF at u is floor(u * V) (dyadic u:
    # every value below is exact); u on a boundary belongs to the upper token
    V = 8
    us = np.array([0.0, 0.0625, 0.125, 0.3, 0.5, 0.74, 0.875, 0.999], np.float32)
    logits, slot_tok, offsets, k = _batch([[0.0] * V], len(us), [5])
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1.0, np.zeros(len(us)), us)
    assert np.array_equal(r["bonus"], np.floor(us.astype(np.float64) * V).astype(np.int32))
    assert np.array_equal(r["accepted"], np.zeros(len(us)))
    assert np.array_equal(r["progress"], np.ones(len(us)))


def test_rejection_removes_the_draft():
    # uniform over 4 tokens, draft x = 0 has P = 1/4: u = 1/4 fails (strict test), the next
    # float below passes; after the failure the draw is uniform over {1, 2, 3}
    V, x = 4, 0
    u_acc = np.array([0.25, np.nextafter(np.float32(0.25), np.float32(0)), 0.25, 0.25, 0.9], np.float32)
    u_draw = np.array([0.5, 0.5, 0.0, 0.999, 0.34], np.float32)
    n = len(u_acc)
    logits, slot_tok, offsets, k = _batch([[0.0] * V, [0.0] * V], n, [7, x])
    ua = np.zeros(2 * n, np.float32)
    ua[0::2] = u_acc
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1.0, ua, u_draw)
    assert r["accepted"].tolist() == [0, 1, 0, 0, 0]
    # request 1 passed: successor from the unmodified second row, floor(0.5 * 4) = 2
    # rejected: token index floor(u * 3) among {1, 2, 3}
    assert r["bonus"].tolist() == [2, 2, 1, 3, 2]
    assert r["out_tokens"][1, :3].tolist() == [x, 2, -1]
    assert np.allclose(r["p_cand"][0::2], 0.25) and np.all(r["p_cand"][1::2] == -1.0)


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_first_token_marginal_equals_target_on_a_grid(T):
    # one candidate; u_accept and u_draw run over the midpoints of an n x n grid, so each
    # frequency equals its probability up to 1/n per coordinate
    n = 512
    row0 = np.array([1.0, 0.2, -0.5, 0.7, -2.0, 0.0], np.float32)
    row1 = np.array([0.3, 0.1, 0.0, -1.0, 2.0, 0.5], np.float32)
    x = 3
    P = softmax(row0.astype(np.float64) / T)
    g = (np.arange(n) + 0.5) / n
    ua, ud = np.meshgrid(g, g, indexing="ij")
    logits, slot_tok, offsets, k = _batch([row0, row1], n * n, [9, x])
    u_acc = np.zeros(2 * n * n, np.float32)
    u_acc[0::2] = ua.ravel()
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, T, u_acc, ud.ravel().astype(np.float32))
    first = r["out_tokens"][:, 0]
    freq = np.bincount(first, minlength=len(P)) / first.size
    assert np.abs(freq - P).max() <= 2.0 / n
    # the rejected draft never comes back as the successor
    rej = r["accepted"] == 0
    assert not np.any(r["bonus"][rej] == x)


def test_sequence_distribution_three_slots():
    # two candidates: every emitted sequence has the probability of drawing its tokens one by
    # one from the rows that predict them (P0, then P1 after x1, then P2 after x2)
    rng = np.random.default_rng(7)
    N, V = 200_000, 5
    rows = [np.array([0.5, 1.0, -0.3, 0.0, 0.2], np.float32),
            np.array([-1.0, 0.4, 0.9, 0.1, 0.0], np.float32),
            np.array([0.0, -0.7, 0.3, 1.2, -0.2], np.float32)]
    x1, x2 = 1, 2
    P = [softmax(r.astype(np.float64)) for r in rows]
    logits, slot_tok, offsets, k = _batch(rows, N, [4, x1, x2])
    u_acc = rng.random(3 * N).astype(np.float32)
    u_draw = rng.random(N).astype(np.float32)
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1.0, u_acc, u_draw)
    expect = {}
    for y in range(V):
        if y != x1:
            expect[(y,)] = P[0][y]
        if y != x2:
            expect[(x1, y)] = P[0][x1] * P[1][y]
        expect[(x1, x2, y)] = P[0][x1] * P[1][x2] * P[2][y]
    assert abs(sum(expect.values()) - 1.0) < 1e-12
    seqs = [tuple(t[: p]) for t, p in zip(r["out_tokens"], r["progress"])]
    counts = {}
    for sq in seqs:
        counts[sq] = counts.get(sq, 0) + 1
    assert set(counts) <= set(expect)
    for sq, p in expect.items():
        f = counts.get(sq, 0) / N
        assert abs(f - p) <= 5 * np.sqrt(p * (1 - p) / N) + 1.0 / N, (sq, f, p)
    # progress and accepted counts agree with the emitted sequence
    assert np.array_equal(r["progress"], r["accepted"] + 1)


def test_certain_and_impossible_drafts():
    rng = np.random.default_rng(3)
    n, V = 400, 6
    ninf = -np.inf
    # row 0: all mass on token 2 (the draft) -> always accepted; row 1: draft 4 has logit
    # -inf -> always rejected, never emitted; row 2 unused by the rejected requests
    rows = [[ninf, ninf, 0.0, ninf, ninf, ninf], [0.1, 0.5, -0.2, 0.3, ninf, 0.0], [0.0] * V]
    logits, slot_tok, offsets, k = _batch(rows, n, [0, 2, 4])
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1.0,
                             rng.random(3 * n).astype(np.float32), rng.random(n).astype(np.float32))
    assert np.all(r["accepted"] == 1)
    assert np.all(r["out_tokens"][:, 0] == 2)
    assert not np.any(r["bonus"] == 4)
    assert np.all(r["p_cand"][0::3] == 1.0) and np.all(r["p_cand"][1::3] == 0.0)
    # a draft outside the vocabulary has probability 0 and its removal changes nothing
    logits, slot_tok, offsets, k = _batch([[0.0] * 4, [0.0] * 4], 4, [0, 99])
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1.0, np.zeros(8, np.float32),
                             np.array([0.0, 0.3, 0.6, 0.9], np.float32))
    assert r["accepted"].tolist() == [0] * 4 and r["bonus"].tolist() == [0, 1, 2, 3]


def test_all_pass_uses_the_unmodified_last_row():
    # the last row is a point mass: the bonus is that token whatever the draw
    n = 64
    rows = [[0.0, ninf := -np.inf, ninf], [ninf, 0.0, ninf], [ninf, ninf, 0.0]]
    logits, slot_tok, offsets, k = _batch(rows, n, [1, 0, 1])
    rng = np.random.default_rng(5)
    r = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1.0,
                             rng.random(3 * n).astype(np.float32), rng.random(n).astype(np.float32))
    assert np.all(r["accepted"] == 2) and np.all(r["bonus"] == 2)
    assert np.all(r["out_tokens"][:, :3] == [0, 1, 2]) and np.all(r["out_tokens"][:, 3:] == -1)


def test_temperature_scales_logits():
    rng = np.random.default_rng(11)
    n, V, kk = 300, 50, 4
    rows = rng.standard_normal((kk, V)).astype(np.float32)
    toks = [0] + [int(np.argmax(r)) for r in rows[:-1]]
    ua = rng.random(kk * n).astype(np.float32)
    ud = rng.random(n).astype(np.float32)
    a = oracle.accept_sample(*_batch(rows, n, toks), W, 1.0, ua, ud)
    b = oracle.accept_sample(*_batch(rows * 2, n, toks), W, 2.0, ua, ud)
    for key in ("accepted", "bonus", "out_tokens"):
        assert np.array_equal(a[key], b[key])
    # p_cand is the temperature softmax at the candidate
    c = oracle.accept_sample(*_batch(rows, n, toks), W, 0.7, ua, ud)
    for j in range(kk - 1):
        assert abs(c["p_cand"][j] - softmax(rows[j].astype(np.float64) / 0.7)[toks[j + 1]]) < 1e-12


def test_low_temperature_is_greedy():
    # logit gaps >= 0.5 at T = 1e-3: P(argmax) = 1 in double, so sampling reproduces the greedy
    # verifier for any uniforms
    rng = np.random.default_rng(2)
    n_req, V = 40, 97
    k = rng.integers(0, W + 1, n_req).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
    m = int(offsets[-1])
    logits = (rng.permutation(V)[None, :] * 0.5 + rng.integers(0, 3, (m, 1))).astype(np.float32)
    logits = np.stack([rng.permutation(row) for row in logits]).astype(np.float32)
    g = np.argmax(logits, axis=1)
    slot_tok = rng.integers(0, V, m).astype(np.int32)
    # make most drafts match the target so that long prefixes are accepted
    hit = rng.random(m) < 0.8
    slot_tok[1:][hit[1:]] = g[:-1][hit[1:]]
    greedy = oracle.accept(logits, slot_tok, offsets, k, W)
    s = oracle.accept_sample(logits, slot_tok, offsets, k, W, 1e-3,
                             rng.random(m).astype(np.float32), rng.random(n_req).astype(np.float32))
    for key in ("accepted", "bonus", "progress", "out_tokens"):
        assert np.array_equal(greedy[key], s[key]), key


def test_errors():
    logits, slot_tok, offsets, k = _batch([[0.0, 1.0], [1.0, 0.0]], 2, [0, 1])
    z2, z4 = np.zeros(2, np.float32), np.zeros(4, np.float32)
    for T in (0.0, -1.0, np.inf, np.nan):
        with pytest.raises(oracle.OracleError):
            oracle.accept_sample(logits, slot_tok, offsets, k, W, T, z4, z2)
    bad = logits.copy()
    bad[1, 0] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.accept_sample(bad, slot_tok, offsets, k, W, 1.0, z4, z2)
    bad[1, 0] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.accept_sample(bad, slot_tok, offsets, k, W, 1.0, z4, z2)
    bad[1] = -np.inf
    with pytest.raises(oracle.OracleError):
        oracle.accept_sample(bad, slot_tok, offsets, k, W, 1.0, z4, z2)
    with pytest.raises(oracle.OracleError):
        oracle.accept_sample(logits, slot_tok, offsets, np.array([2, 17], np.int32), W, 1.0, z4, z2)
    # an inactive request emits nothing and its rows are never read
    bad[:] = np.nan
    r = oracle.accept_sample(bad, slot_tok, np.array([0, 0, 0], np.int32), np.zeros(2, np.int32),
                             W, 1.0, z4, z2)
    assert r["progress"].tolist() == [0, 0] and r["bonus"].tolist() == [-1, -1]
