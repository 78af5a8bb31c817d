"""GPU parity of dsv_pack_slots against the oracle packer: bit-exact."""
import json
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from gpu_util import DEV, device_case, gpu_pack, oracle_pack, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402

FIELDS = ("offsets", "slot_req", "slot_tok", "slot_pos", "slot_cache_loc")


def _check(got, ref, tag):
    for f in FIELDS:
        g = got[f].cpu().numpy()
        assert np.array_equal(g, ref[f]), f"{tag}: {f} differs\n{g}\n{ref[f]}"


def _pack_arrays(k, ctx, base, tokens, m_bs):
    st = dsv.new_status(DEV)
    out = dsv.pack_slots(to_dev(np.asarray(k, np.int32)), to_dev(np.asarray(ctx, np.int32)),
                         to_dev(np.asarray(base, np.int64)), to_dev(np.asarray(tokens, np.int32)),
                         m_bs, st)
    return out, int(st.item())


@pytest.mark.parametrize("cfg", ["cfg1", "cfg2a", "cfg2b", "cfg3", "cfg4", "cfg5"])
def test_pack_configs(cfg):
    if cfg == "cfg1":
        c = wl.config1()
    elif cfg.startswith("cfg2"):
        c = wl.config2()[0 if cfg == "cfg2a" else 1]
    elif cfg == "cfg3":
        c = wl.make_case(3, dtype="bf16", hq=1, hkv=1, d=64, k=[16] * 8, ctx_len=[8192] * 8, m_bs=128)
    elif cfg == "cfg4":
        g = wl.rng(4, 0)
        k = wl.lengths_geometric_rescaled(g, 32, 256)
        ctx = g.integers(4096, 8193, size=32)
        c = wl.make_case(4, dtype="bf16", hq=1, hkv=1, d=64, k=k, ctx_len=ctx, m_bs=256)
    else:
        g = wl.rng(5, 0)
        k = wl.lengths_geometric_rescaled(g, 60, 480)
        ctx = g.integers(8192, 32769, size=60)
        c = dict(k=k, ctx_len=ctx.astype(np.int32), kv_base=wl.segments(ctx, 16)[0],
                 block_tokens=wl.rng(5, 6).integers(0, 32000, size=(60, 16)).astype(np.int32),
                 W=16, m_bs=480)
    ref = oracle_pack(c)
    got, st = _pack_arrays(c["k"], c["ctx_len"], c["kv_base"], c["block_tokens"], c["m_bs"])
    assert st == 0
    _check(got, ref, cfg)


def test_layout_shift_and_fig6_examples():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_examples.json")))
    for k, starts, end in ((g["layout_shift"]["before"]["k"], g["layout_shift"]["before"]["starts"], 24),
                           (g["layout_shift"]["after"]["k"], g["layout_shift"]["after"]["starts"], 24),
                           (g["fig6"]["k"], g["fig6"]["offsets"], 32)):
        n = len(k)
        got, st = _pack_arrays(k, [10] * n, [0] * n, np.zeros((n, 16), np.int32), 32)
        off = got["offsets"].cpu().numpy()
        assert st == 0 and list(off[:-1]) == starts and off[-1] == end


@pytest.mark.parametrize("seed", range(12))
def test_pack_random(seed):
    r = np.random.default_rng(100 + seed)
    W = int(r.integers(1, 17))
    n = int(r.choice([0, 1, 7, 1000, 1025, 5000]))
    k = r.integers(0, W + 1, size=n).astype(np.int32)
    m_bs = int(k.sum()) + int(r.integers(0, 300))
    ctx = r.integers(0, 100000, size=n).astype(np.int32)
    base = r.integers(0, 1 << 40, size=n).astype(np.int64)
    tokens = r.integers(0, 1 << 31, size=(n, W), dtype=np.int64).astype(np.int32)
    import oracle
    ref = oracle.pack(k, ctx, base, tokens, W, m_bs)
    got, st = _pack_arrays(k, ctx, base, tokens.reshape(n, W), m_bs)
    assert st == 0
    _check(got, ref, f"seed {seed}")


def test_pack_bad_request_is_inactive():
    """k_i outside [0, W] or a negative context: status bit, packed as k_i = 0."""
    import oracle
    k = np.array([3, 17, 2, -1, 4], np.int32)
    ctx = np.array([5, 5, -3, 5, 5], np.int32)
    base = np.arange(5, dtype=np.int64) * 100
    tokens = np.arange(5 * 16, dtype=np.int32).reshape(5, 16)
    got, st = _pack_arrays(k, ctx, base, tokens, 16)
    assert st == dsv.STATUS_BAD_REQUEST
    sane = np.array([3, 0, 0, 0, 4], np.int32)
    _check(got, oracle.pack(sane, np.maximum(ctx, 0), base, tokens, 16, 16), "sanitized")


def test_pack_budget_overflow_drops_all():
    k = np.array([8, 8, 8], np.int32)
    got, st = _pack_arrays(k, [1, 2, 3], [0, 50, 100], np.ones((3, 16), np.int32), 23)
    assert st == dsv.STATUS_BUDGET
    assert np.all(got["offsets"].cpu().numpy() == 0)
    assert np.all(got["slot_req"].cpu().numpy() == -1)
    assert np.all(got["slot_cache_loc"].cpu().numpy() == -1)


def test_pack_empty_batch():
    got, st = _pack_arrays(np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int64),
                           np.zeros((0, 16), np.int32), 5)
    assert st == 0 and got["offsets"].cpu().tolist() == [0]
    assert got["slot_req"].cpu().tolist() == [-1] * 5
