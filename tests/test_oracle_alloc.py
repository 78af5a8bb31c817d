"""Pins of the oracle's budget allocator (DScale Sec. III-C, Acceptance predictor / Budget
allocator, Fig. 6): the printed example, the printed seed rounding, the cumulative-minimum
rule, the lowest-index tie rule, brute-force optimality on tiny batches, and the |delta| <= 7N
bound for W = 16."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_examples.json")))


def _steps(*runs):
    """Draft scores from (value, count) runs (already nonincreasing)."""
    return np.array([v for v, n in runs for _ in range(n)], np.float32)


def test_fig6_allocation():
    g = GOLDEN["fig6_allocation"]
    W = g["W"]
    scores = np.stack([
        _steps((0.9, 4), (0.8, 1), (0.1, 10)),     # seed 5, next-slot score 0.8
        _steps((0.99, 9), (0.7, 1), (0.1, 5)),     # seed 10, next-slot score 0.7
        _steps((0.9, 6), (0.6, 1), (0.125, 8)),    # seed 7, next-slot score 0.6
        _steps((0.95, 8), (0.5, 1), (0.15, 6)),    # seed 9, next-slot score 0.5
    ])
    r = oracle.allocate(scores, 4, W, g["budget"])
    assert r["k0"].tolist() == g["k0"]
    assert r["k"].tolist() == g["k"]
    p = oracle.allocate_pack(scores, 4, W, g["budget"], g["budget"], np.full(4, 100, np.int32),
                             np.arange(4, dtype=np.int64) * 200, np.zeros((4, W), np.int32))
    assert p["offsets"].tolist() == g["offsets"] + [g["end"]]


def test_seed_rounding_example():
    g = GOLDEN["seed_rounding"]
    scores = _steps((0.62, 10), (0.0, 5))[None]  # estimate 6.2
    assert abs(float(np.sum(scores.astype(np.float64))) - g["estimate"]) < 1e-5
    r = oracle.allocate(scores, 1, 16, 6)
    assert r["k0"].tolist() == [g["k0"]]


def test_cumulative_minimum():
    # acceptance needs accepted predecessors: a low score caps every later one
    scores = np.array([[0.1] + [0.9] * 14], np.float32)
    r = oracle.allocate(scores, 1, 16, 2)
    assert r["k0"].tolist() == [2]  # prefix scores 0.1 x 15 -> estimate 1.5 -> 2 (ties to even)
    nan = np.array([[0.9, np.nan] + [0.9] * 13], np.float32)
    assert oracle.allocate(nan, 1, 16, 1)["k0"].tolist() == [1]  # NaN counts as 0: estimate 0.9


def test_tie_rule_lowest_index():
    # seeds 8 each (estimate 7.5 -> 8); every next-slot and last-slot score is 0.5, so each
    # step moves the lowest-index request that can move
    s = np.full((3, 15), 0.5, np.float32)
    assert oracle.allocate(s, 3, 16, 25)["k"].tolist() == [9, 8, 8]
    assert oracle.allocate(s, 3, 16, 27)["k"].tolist() == [11, 8, 8]
    assert oracle.allocate(s, 3, 16, 23)["k"].tolist() == [7, 8, 8]
    assert oracle.allocate(s, 3, 16, 20)["k"].tolist() == [4, 8, 8]
    # a higher score elsewhere wins over the lower index
    s2 = s.copy()
    s2[2, 7] = 0.5  # unchanged
    s2[1] = 0.6     # request 1: seed round(9.0) = 9, next-slot 0.6 > 0.5
    assert oracle.allocate(s2, 3, 16, 26)["k"].tolist() == [8, 10, 8]


def _objective(q, k):
    return sum(float(np.sum(q[i, :k[i]], dtype=np.float64)) for i in range(len(k)))


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_optimal(seed):
    rng = np.random.default_rng(seed)
    W, N = 6, 3
    scores = rng.choice(np.array([0.05, 0.2, 0.5, 0.7, 0.9], np.float32), size=(N, W - 1))
    m_live = int(rng.integers(N, N * W + 1))
    r = oracle.allocate(scores, N, W, m_live)
    k0, k = r["k0"], r["k"]
    q = np.ones((N, W), np.float64)
    for i in range(N):
        for j in range(1, W):
            q[i, j] = min(q[i, j - 1], float(scores[i, j - 1]))
    assert int(k.sum()) == m_live and (k >= 1).all() and (k <= W).all()
    grow = m_live >= int(k0.sum())
    best = -1.0
    for cand in itertools.product(range(1, W + 1), repeat=N):
        cand = np.array(cand)
        if cand.sum() != m_live or ((cand < k0).any() if grow else (cand > k0).any()):
            continue
        best = max(best, _objective(q, cand))
    assert abs(_objective(q, k) - best) < 1e-9
    assert ((k >= k0).all() if grow else (k <= k0).all())


def test_adjustment_bound_and_inactive():
    rng = np.random.default_rng(7)
    for _ in range(50):
        N, n_bs = int(rng.integers(1, 40)), 48
        scores = rng.random((n_bs, 15), dtype=np.float32)
        r = oracle.allocate(scores, N, 16, 8 * N)
        assert abs(8 * N - int(r["k0"][:N].sum())) <= 7 * N
        assert int(r["k"].sum()) == 8 * N
        assert (r["k"][N:] == 0).all() and (r["k0"][N:] == 0).all()
        assert (r["k"][:N] >= 1).all() and (r["k"][:N] <= 16).all()


def test_unreachable_budget_stops():
    s = np.full((2, 3), 0.9, np.float32)
    assert oracle.allocate(s, 2, 4, 20)["k"].tolist() == [4, 4]  # everyone at W
    assert oracle.allocate(s, 2, 4, 1)["k"].tolist() == [1, 1]   # everyone at the anchor
