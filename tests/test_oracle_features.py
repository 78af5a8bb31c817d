"""Pins of the oracle's draft confidence features (DScale Sec. III-C, Acceptance predictor:
per draft position, the highest logit, its 15 gaps to ranks 2-16, the top token's
log-probability and the distribution's entropy).  Closed forms on uniform and two-level rows,
numpy's sort for the ranks (ties included), scipy's log_softmax and entropy for the two
distribution values."""
import numpy as np
import pytest
from scipy.special import log_softmax, softmax
from scipy.stats import entropy

import oracle


@pytest.mark.parametrize("V", [16, 100, 4096])
def test_uniform_row(V):
    f = oracle.draft_features(np.full((1, V), 0.75, np.float32))[0]
    assert f[0] == np.float32(0.75)
    assert np.all(f[1:16] == 0.0)
    assert abs(f[16] - (-np.log(V))) <= 1e-6 * np.log(V)
    assert abs(f[17] - np.log(V)) <= 1e-6 * np.log(V)


@pytest.mark.parametrize("V,a,b", [(16, 2.0, 0.0), (1000, 5.5, -1.25), (151936, 12.0, 0.5)])
def test_two_level_row(V, a, b):
    # one token at a, V - 1 at b: Z = 1 + (V - 1) e^(b - a)
    row = np.full(V, b, np.float32)
    row[V // 3] = a
    f = oracle.draft_features(row[None])[0]
    Z = 1.0 + (V - 1) * np.exp(b - a)
    p1, p2 = 1.0 / Z, np.exp(b - a) / Z
    H = -p1 * np.log(p1) - (V - 1) * p2 * np.log(p2)
    assert f[0] == np.float32(a)
    assert np.all(f[1:16] == np.float32(a - b))
    assert abs(f[16] - (-np.log(Z))) <= 1e-6 * max(1.0, np.log(Z))
    assert abs(f[17] - H) <= 1e-6 * max(1.0, H)


def test_ranks_against_numpy_sort():
    rng = np.random.default_rng(4)
    for V in (16, 17, 255, 5000):
        x = rng.integers(-20, 20, (30, V)).astype(np.float32) * np.float32(0.25)  # many ties
        x[:5, :3] = 7.0  # repeated maxima: the first gaps are 0
        f = oracle.draft_features(x)
        s = -np.sort(-x, axis=1)
        assert np.array_equal(f[:, 0], s[:, 0])
        gaps = (s[:, :1].astype(np.float64) - s[:, 1:16].astype(np.float64)).astype(np.float32)
        assert np.array_equal(f[:, 1:16], gaps)
        assert np.all(f[:5, 1:3] == 0.0) and np.all(np.diff(f[:, 1:16], axis=1) >= 0)


def test_distribution_values_against_scipy():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((40, 3000)) * rng.uniform(0.1, 4.0, (40, 1))).astype(np.float32)
    x[3, :2000] = -np.inf  # zero-probability tokens
    f = oracle.draft_features(x)
    x64 = x.astype(np.float64)
    lp = log_softmax(x64, axis=1)[np.arange(40), np.argmax(x64, axis=1)]
    H = entropy(softmax(x64, axis=1), axis=1)
    assert np.all(np.abs(f[:, 16] - lp) <= 1e-6 * np.maximum(1.0, np.abs(lp)))
    assert np.all(np.abs(f[:, 17] - H) <= 1e-6 * np.maximum(1.0, H))
    # fewer than 16 finite logits: the remaining gaps are infinite
    y = np.full((1, 64), -np.inf, np.float32)
    y[0, [3, 9]] = [1.0, 0.5]
    g = oracle.draft_features(y)[0]
    assert g[1] == np.float32(0.5) and np.all(np.isinf(g[2:16]))
    assert abs(g[17] - entropy(softmax(np.array([1.0, 0.5])))) < 1e-6


def test_errors():
    x = np.zeros((2, 32), np.float32)
    for bad in (np.nan, np.inf):
        y = x.copy()
        y[1, 7] = bad
        with pytest.raises(oracle.OracleError):
            oracle.draft_features(y)
    with pytest.raises(oracle.OracleError):
        oracle.draft_features(np.full((1, 32), -np.inf, np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.draft_features(np.zeros((1, 15), np.float32))
