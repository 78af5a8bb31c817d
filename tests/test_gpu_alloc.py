"""GPU parity of dsv_allocate_pack (budget allocator fused with the packer) against the
oracle: adjusted lengths, seeds, offsets and every slot array bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from block_verification_attention_amd import allocate_pack, new_status, STATUS_NAN

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _case(seed, n_live, n_bs, W, levels=None, nan=False):
    rng = np.random.default_rng(seed)
    if levels is None:
        scores = rng.random((n_bs, W - 1), dtype=np.float32)
    else:  # few distinct values: many ties
        scores = rng.choice(np.array(levels, np.float32), size=(n_bs, W - 1))
    if nan and n_live > 0:
        scores[rng.integers(0, n_live), rng.integers(0, W - 1)] = np.nan
    ctx = rng.integers(0, 5000, n_bs).astype(np.int32)
    base = (np.arange(n_bs, dtype=np.int64) * 6000)
    toks = rng.integers(0, 150000, (n_bs, W)).astype(np.int32)
    return scores, ctx, base, toks


def _run(scores, ctx, base, toks, n_live, m_live, m_bs):
    st = new_status(DEV)
    out = allocate_pack(torch.from_numpy(scores).to(DEV), n_live, m_live, torch.from_numpy(ctx).to(DEV),
                        torch.from_numpy(base).to(DEV), torch.from_numpy(toks).to(DEV), m_bs, st)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, int(st.item())


def _check(seed, n_live, n_bs, W, m_live, m_bs, **kw):
    scores, ctx, base, toks = _case(seed, n_live, n_bs, W, **kw)
    g, status = _run(scores, ctx, base, toks, n_live, m_live, m_bs)
    r = oracle.allocate_pack(scores, n_live, W, m_live, m_bs, ctx, base, toks)
    tag = f"seed {seed} n_live {n_live} n_bs {n_bs} W {W} m_live {m_live}"
    for name in ("k0", "k", "offsets", "slot_req", "slot_tok", "slot_pos", "slot_cache_loc"):
        assert np.array_equal(g[name], r[name]), f"{name} differs ({tag})"
    return g, status


@pytest.mark.parametrize("n_live,n_bs", [(8, 8), (4, 8), (60, 64), (32, 48), (200, 256), (1000, 1024)])
def test_allocate_pack_parity(n_live, n_bs):
    for seed in range(3):
        _check(100 * n_live + seed, n_live, n_bs, 16, 8 * n_live, 8 * n_bs)


@pytest.mark.parametrize("levels", [[0.0, 0.5, 1.0], [0.25, 0.5], [0.5]])
def test_allocate_pack_ties(levels):
    for seed, (n_live, n_bs) in enumerate([(3, 4), (17, 32), (64, 64), (300, 512)]):
        for m_live in (n_live, 4 * n_live, 8 * n_live, 12 * n_live, 16 * n_live):
            _check(seed, n_live, n_bs, 16, m_live, 16 * n_bs, levels=levels)


def test_allocate_pack_edges():
    _check(1, 0, 8, 16, 0, 64)            # nobody live
    _check(2, 5, 5, 1, 5, 5)              # W = 1: anchors only
    _check(3, 5, 8, 4, 40, 64)            # budget above n_live * W: everyone at W
    _check(4, 5, 8, 16, 2, 64)            # budget below n_live: everyone at the anchor
    _check(5, 9, 16, 7, 30, 64)           # W below the maximum
    _, status = _check(6, 12, 16, 16, 96, 128, nan=True)
    assert status & STATUS_NAN


def test_fig6_on_gpu():
    # DScale Fig. 6: seeds [5, 10, 7, 9], budget 32 -> [6, 10, 7, 9], offsets [0, 6, 16, 23]
    def steps(*runs):
        return [v for v, n in runs for _ in range(n)]
    scores = np.array([steps((0.9, 4), (0.8, 1), (0.1, 10)), steps((0.99, 9), (0.7, 1), (0.1, 5)),
                       steps((0.9, 6), (0.6, 1), (0.125, 8)), steps((0.95, 8), (0.5, 1), (0.15, 6))], np.float32)
    ctx = np.full(4, 100, np.int32)
    base = np.arange(4, dtype=np.int64) * 200
    toks = np.arange(64, dtype=np.int32).reshape(4, 16)
    g, _ = _run(scores, ctx, base, toks, 4, 32, 32)
    assert g["k0"].tolist() == [5, 10, 7, 9]
    assert g["k"].tolist() == [6, 10, 7, 9]
    assert g["offsets"].tolist() == [0, 6, 16, 23, 32]
