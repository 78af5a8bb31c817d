"""Pins for the oracle's flat-buffer packer (DScale Sec. III-C, Fig. 6; Sec. II-C
Challenge 3).  These pin the oracle to the pages' printed examples and to brute-force
enumeration; they do not involve the HIP library."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_examples.json")))


def _pack(k, W=16, m_bs=None, ctx=None, base=None, tokens=None):
    k = np.asarray(k, np.int32)
    n = len(k)
    m_bs = int(k.sum()) if m_bs is None else m_bs
    ctx = np.arange(n, dtype=np.int32) * 100 + 7 if ctx is None else np.asarray(ctx, np.int32)
    base = np.arange(n, dtype=np.int64) * 10_000 if base is None else np.asarray(base, np.int64)
    tokens = (np.arange(n * W, dtype=np.int32).reshape(n, W) + 1000) if tokens is None else tokens
    return oracle.pack(k, ctx, base, tokens, W, m_bs), ctx, base, tokens


def test_layout_shift_example():
    g = GOLDEN["layout_shift"]
    for key in ("before", "after"):
        out, *_ = _pack(g[key]["k"], W=g["W"])
        assert list(out["offsets"][:-1]) == g[key]["starts"]
        assert int(out["offsets"][-1]) == g[key]["end"]
    b, _, _, _ = _pack(g["before"]["k"])
    a, _, _, _ = _pack(g["after"]["k"])
    assert b["offsets"][1] == g["r2_start_before"] and a["offsets"][1] == g["r2_start_after"]
    # equal-width padding of the same requests would need N * W rows
    assert len(g["before"]["k"]) * g["W"] == g["padded_rows"]
    # no slot of the new layout holds the same request as the old layout's slice would claim
    # for R2 unless it really is R2 (requests never mix after the shift)
    old_r2 = set(range(b["offsets"][1], b["offsets"][2]))
    assert any(a["slot_req"][s] != 1 for s in old_r2)
    for s in range(a["offsets"][1], a["offsets"][2]):
        assert a["slot_req"][s] == 1


def test_fig6_example():
    g = GOLDEN["fig6"]
    out, *_ = _pack(g["k"], m_bs=32)
    assert list(out["offsets"]) == g["offsets"] + [g["end"]]


@pytest.mark.parametrize("seed", range(20))
def test_bijection_bruteforce(seed):
    """Every (request, j < k_i) pair occupies exactly one slot below the end boundary,
    its fields carry that pair's token/position/cache reference, and every other slot is a
    tail placeholder."""
    r = np.random.default_rng(seed)
    W = int(r.integers(1, 17))
    n = int(r.integers(0, 12))
    k = r.integers(0, W + 1, size=n).astype(np.int32)
    m_bs = int(k.sum()) + int(r.integers(0, 9))
    ctx = r.integers(0, 5000, size=n).astype(np.int32)
    base = r.integers(0, 1 << 40, size=n).astype(np.int64)
    tokens = r.integers(0, 1 << 30, size=(n, W)).astype(np.int32)
    out, *_ = _pack(k, W, m_bs, ctx, base, tokens)
    seen = {}
    for s in range(m_bs):
        if out["slot_req"][s] >= 0:
            i = int(out["slot_req"][s])
            j = int(out["slot_pos"][s]) - int(ctx[i])
            assert 0 <= j < k[i]
            assert (i, j) not in seen
            seen[(i, j)] = s
            assert out["slot_tok"][s] == tokens[i, j]
            assert out["slot_cache_loc"][s] == base[i] + ctx[i] + j
        else:
            assert (out["slot_tok"][s], out["slot_pos"][s], out["slot_cache_loc"][s]) == (0, 0, -1)
    assert len(seen) == int(k.sum())
    # requests occupy consecutive slots in request order, starting at the offsets
    for (i, j), s in seen.items():
        assert s == out["offsets"][i] + j
    assert all(s < out["offsets"][-1] for s in seen.values())
    assert out["offsets"][0] == 0 and np.all(np.diff(out["offsets"]) == k)


def test_inactive_and_tail():
    out, *_ = _pack([0, 3, 0, 2, 0], m_bs=9)
    assert list(out["offsets"]) == [0, 0, 3, 3, 5, 5]
    assert list(out["slot_req"]) == [1, 1, 1, 3, 3, -1, -1, -1, -1]


def test_errors():
    with pytest.raises(oracle.OracleError):
        _pack([3, 17], W=16)
    with pytest.raises(oracle.OracleError):
        _pack([-1], W=16, m_bs=16)
    with pytest.raises(oracle.OracleError):
        _pack([8, 8, 8], m_bs=23)
    out, *_ = _pack([8, 8, 8], m_bs=24)
    assert out["offsets"][-1] == 24


def test_all_small_length_vectors_exhaustive():
    """Exhaustive over all length vectors with n=3, W=4: offsets are the running sums."""
    for k in itertools.product(range(5), repeat=3):
        out, *_ = _pack(list(k), W=4, m_bs=12)
        assert list(out["offsets"]) == [0, k[0], k[0] + k[1], k[0] + k[1] + k[2]]
