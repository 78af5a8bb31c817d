"""GPU parity of verification attention read through a token-granular cache map
(dsv_attn_args.kv_index: position p of request i is pool row kv_index[i][p]) against the
oracle's cache-map path, and against the contiguous-segment kernel on the same values."""
import numpy as np
import pytest
import torch

import oracle
import block_verification_attention_amd as dsv
from gpu_util import DEV, compare_attn, device_case, gpu_pack, oracle_pack, small_case, to_dev, to_f64

pytestmark = pytest.mark.gpu


def scatter(c, seed, share=False):
    """Pool rows moved to random places (and a cache map pointing at them); share=True makes
    request 1's first context rows alias request 0's."""
    rng = np.random.default_rng(seed)
    rows = c["k_pool"].shape[1]
    perm = rng.permutation(rows)
    kp = np.empty_like(c["k_pool"])
    vp = np.empty_like(c["v_pool"])
    kp[:, perm] = c["k_pool"]
    vp[:, perm] = c["v_pool"]
    n_bs = len(c["k"])
    stride = int((c["ctx_len"] + c["W"]).max()) + 3
    idx = np.full((n_bs, stride), -7, np.int32)
    for i in range(n_bs):
        n = int(c["ctx_len"][i] + c["k"][i])
        idx[i, :n] = perm[int(c["kv_base"][i]) + np.arange(n)]
    if share:
        n = int(min(c["ctx_len"][0], c["ctx_len"][1]))
        idx[1, :n] = idx[0, :n]
    return kp, vp, idx


def mapped_cache_loc(c, packed, idx):
    """This step's cache references under the map: candidate j of request i goes to the row
    the map gives its position, idx[i][ctx_i + j] (a row no request reads as context)."""
    off = packed["offsets"].cpu().numpy()
    loc = np.full(c["m_bs"], -1, np.int64)
    for i in range(len(c["k"])):
        for j in range(int(c["k"][i])):
            loc[off[i] + j] = idx[i, int(c["ctx_len"][i]) + j]
    return torch.from_numpy(loc).to(DEV)


def run_mapped(c, d, packed, kp, vp, idx, *, use_new=True, kv_chunk=0, loc_idx=None):
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV)
    dsv.verify_attn(d["q"], to_dev(kp), to_dev(vp), packed["offsets"], d["k"], d["ctx_len"], d["kv_base"],
                    W=c["W"], max_ctx=int(c["ctx_len"].max()), status=d["status"], out=out, lse=lse,
                    k_new=d["k_new"] if use_new else None, v_new=d["v_new"] if use_new else None,
                    slot_cache_loc=mapped_cache_loc(c, packed, idx if loc_idx is None else loc_idx) if use_new else None, kv_chunk=kv_chunk,
                    kv_index=to_dev(idx))
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("dtype,d_head,hq,hkv", [("bf16", 128, 32, 8), ("bf16", 64, 8, 2), ("bf16", 128, 12, 4),
                                                 ("bf16", 256, 24, 2), ("bf16", 256, 2, 2), ("f32", 64, 4, 2)])
@pytest.mark.parametrize("use_new", [True, False])
def test_cache_map_parity(dtype, d_head, hq, hkv, use_new):
    c = small_case(40 + d_head + hq, dtype=dtype, hq=hq, hkv=hkv, d=d_head,
                   k=(16, 5, 0, 11, 1, 16), ctx=(700, 0, 40, 63, 1500, 129))
    d = device_case(c)
    packed = gpu_pack(c, d)
    kp, vp, idx = scatter(c, 3)
    out, lse = run_mapped(c, d, packed, kp, vp, idx, use_new=use_new, kv_chunk=128)
    assert int(d["status"].item()) == 0
    ref = oracle_pack(c)
    r_o, r_l = oracle.verify_attn(c["q"], kp, vp, ref["offsets"], c["k"], c["ctx_len"], c["kv_base"],
                                  c["k_new"] if use_new else None, c["v_new"] if use_new else None,
                                  kv_index=idx)
    compare_attn(c, ref["offsets"], out, lse, r_o, r_l, tag=f"cache map {dtype} d{d_head} g{hq // hkv}")


def test_identity_map_bit_identical_to_segments():
    c = small_case(51, k=(16, 16, 9, 1), ctx=(2000, 333, 64, 0))
    d = device_case(c)
    packed = gpu_pack(c, d)
    n_bs = len(c["k"])
    stride = int((c["ctx_len"] + c["W"]).max())
    idx = np.zeros((n_bs, stride), np.int32)
    for i in range(n_bs):
        idx[i] = int(c["kv_base"][i]) + np.arange(stride)
    idx = np.minimum(idx, c["k_pool"].shape[1] - 1).astype(np.int32)
    mo, ml = run_mapped(c, d, packed, c["k_pool"], c["v_pool"], idx, kv_chunk=256)
    seg_out = torch.full_like(d["q"], float("nan"))
    seg_lse = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV)
    dsv.verify_attn(d["q"], d["k_pool"], d["v_pool"], packed["offsets"], d["k"], d["ctx_len"], d["kv_base"],
                    W=c["W"], max_ctx=int(c["ctx_len"].max()), status=d["status"], out=seg_out, lse=seg_lse,
                    k_new=d["k_new"], v_new=d["v_new"], slot_cache_loc=packed["slot_cache_loc"], kv_chunk=256)
    torch.cuda.synchronize()
    assert torch.equal(mo, seg_out) and torch.equal(ml, seg_lse)


def test_shared_prefix_map():
    c = small_case(52, dtype="bf16", hq=32, hkv=8, k=(9, 16, 3), ctx=(1000, 1200, 70))
    d = device_case(c)
    packed = gpu_pack(c, d)
    kp, vp, idx = scatter(c, 9, share=True)
    out, lse = run_mapped(c, d, packed, kp, vp, idx)
    ref = oracle_pack(c)
    r_o, r_l = oracle.verify_attn(c["q"], kp, vp, ref["offsets"], c["k"], c["ctx_len"], c["kv_base"],
                                  c["k_new"], c["v_new"], kv_index=idx)
    compare_attn(c, ref["offsets"], out, lse, r_o, r_l, tag="shared prefix")


def test_cache_map_bad_entries_flagged():
    c = small_case(53, k=(4, 16), ctx=(100, 50))
    d = device_case(c)
    packed = gpu_pack(c, d)
    kp, vp, idx = scatter(c, 10)
    bad = idx.copy()
    bad[0, 3] = kp.shape[1] + 5  # past the pool: flagged, the nearest row is read
    run_mapped(c, d, packed, kp, vp, bad)
    assert int(d["status"].item()) & dsv.STATUS_POOL
    d["status"].zero_()
    short = np.ascontiguousarray(idx[:, :104])  # request 0 sees 100 + 4 positions, request 1 50 + 16
    out, _ = run_mapped(c, d, packed, kp, vp, short, loc_idx=idx)
    assert int(d["status"].item()) == 0
    short2 = np.ascontiguousarray(idx[:, :103])  # request 0 needs 104 entries: invalid, zeroed
    out, _ = run_mapped(c, d, packed, kp, vp, short2, loc_idx=idx)
    assert int(d["status"].item()) & dsv.STATUS_BAD_REQUEST
    assert torch.all(out[:4] == 0)


def test_cache_map_with_prefill_rejected():
    c = small_case(54, k=(4,), ctx=(10,))
    d = device_case(c)
    packed = gpu_pack(c, d)
    kp, vp, idx = scatter(c, 11)
    pf = dsv.Prefill(q_start=torch.zeros(1, dtype=torch.int32, device=DEV),
                     q_len=torch.ones(1, dtype=torch.int32, device=DEV),
                     ctx_len=torch.zeros(1, dtype=torch.int32, device=DEV),
                     kv_base=torch.zeros(1, dtype=torch.int64, device=DEV),
                     q=d["q"][:1].clone(), out=torch.empty_like(d["q"][:1]), max_len=1)
    with pytest.raises(dsv.DsvError):
        dsv.verify_attn(d["q"], to_dev(kp), to_dev(vp), packed["offsets"], d["k"], d["ctx_len"], d["kv_base"],
                        W=c["W"], max_ctx=10, status=d["status"], k_new=d["k_new"], v_new=d["v_new"],
                        slot_cache_loc=packed["slot_cache_loc"], prefill=pf, kv_index=to_dev(idx))
