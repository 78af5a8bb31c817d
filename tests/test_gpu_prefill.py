"""GPU parity of the wide-tile prefill path of dsv_verify_attn (alone and mixed with a
verification set in one call) against the oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import (DEV, TOL, compare_attn, device_case, gpu_pack, oracle_attn,  # noqa: E402
                      oracle_pack, to_dev, to_f64)
import block_verification_attention_amd as dsv  # noqa: E402


def _prefill_case(seed, q_len, ctx, hq=8, hkv=2, d=128, dtype="bf16"):
    return wl.make_mixed_case(seed, hq=hq, hkv=hkv, d=d, k=[3, 16], ctx_len=[40, 130], m_bs=20,
                              pf_q_len=q_len, pf_ctx=ctx, dtype=dtype)


def _run_mixed(c, *, with_verify, pf_new=False, rows=None, tag=""):
    pf = c["prefill"]
    d = device_case(c)
    st = d["status"]
    pf_q = to_dev(pf["q"])
    pf_out = torch.full_like(pf_q, float("nan"))
    pf_lse = torch.full((pf_q.shape[0], c["hq"]), float("nan"), device=DEV)
    k_pool_host, v_pool_host = c["k_pool"], c["v_pool"]
    pf_k_new = pf_v_new = None
    if pf_new:
        # the prefill rows' K/V come in pf_k_new/pf_v_new; the pool holds stale values there
        hkv, dd = c["hkv"], c["d"]
        rows_total = pf_q.shape[0]
        kn = np.empty((rows_total, hkv, dd), k_pool_host.dtype)
        vn = np.empty_like(kn)
        for r in range(pf["n_pf"]):
            b, cx, ql, qs = int(pf["kv_base"][r]), int(pf["ctx_len"][r]), int(pf["q_len"][r]), int(pf["q_start"][r])
            kn[qs:qs + ql] = np.transpose(k_pool_host[:, b + cx:b + cx + ql], (1, 0, 2))
            vn[qs:qs + ql] = np.transpose(v_pool_host[:, b + cx:b + cx + ql], (1, 0, 2))
        stale_k = k_pool_host.copy()
        stale_v = v_pool_host.copy()
        for r in range(pf["n_pf"]):
            b, cx, ql = int(pf["kv_base"][r]), int(pf["ctx_len"][r]), int(pf["q_len"][r])
            stale_k[:, b + cx:b + cx + ql] = wl.BF16_NAN if c["dtype"] == "bf16" else np.float32(np.nan)
            stale_v[:, b + cx:b + cx + ql] = wl.BF16_NAN if c["dtype"] == "bf16" else np.float32(np.nan)
        d["k_pool"], d["v_pool"] = to_dev(stale_k), to_dev(stale_v)
        pf_k_new, pf_v_new = to_dev(kn), to_dev(vn)
    prefill = dsv.Prefill(q_start=to_dev(pf["q_start"]), q_len=to_dev(pf["q_len"]),
                          ctx_len=to_dev(pf["ctx_len"]), kv_base=to_dev(pf["kv_base"]), q=pf_q,
                          out=pf_out, max_len=pf["max_len"], lse=pf_lse, k_new=pf_k_new, v_new=pf_v_new)
    packed = gpu_pack(c, d) if with_verify else None
    out = torch.full_like(d["q"], float("nan")) if with_verify else None
    lse = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV) if with_verify else None
    dsv.verify_attn(d["q"] if with_verify else None, d["k_pool"], d["v_pool"],
                    packed["offsets"] if with_verify else None, d["k"] if with_verify else None,
                    d["ctx_len"], d["kv_base"], W=16, max_ctx=int(c["ctx_len"].max()), status=st,
                    out=out, lse=lse, k_new=d["k_new"] if with_verify else None,
                    v_new=d["v_new"] if with_verify else None,
                    slot_cache_loc=packed["slot_cache_loc"] if with_verify else None, prefill=prefill)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, tag
    # prefill rows vs oracle
    sel_req, sel_j = [], []
    for r in range(pf["n_pf"]):
        js = range(int(pf["q_len"][r])) if rows is None else rows(r, int(pf["q_len"][r]))
        for j in js:
            sel_req.append(r)
            sel_j.append(j)
    ref_o, ref_l = oracle.prefill_attn(pf["q"], k_pool_host, v_pool_host, pf["q_start"], pf["q_len"],
                                       pf["ctx_len"], pf["kv_base"], sel_req, sel_j)
    idx = np.array([int(pf["q_start"][r]) + j for r, j in zip(sel_req, sel_j)])
    go = to_f64(pf_out)[idx]
    gl = to_f64(pf_lse)[idx]
    tol = TOL[c["dtype"]]
    assert np.all(np.isfinite(go)), tag
    assert np.abs(go - ref_o).max() <= tol["max_abs"], (tag, np.abs(go - ref_o).max())
    for h in range(c["hq"]):
        rel = np.linalg.norm(go[:, h] - ref_o[:, h]) / np.linalg.norm(ref_o[:, h])
        assert rel <= tol["rel_l2"], (tag, h, rel)
    assert np.abs(gl - ref_l).max() <= tol["lse"], (tag, np.abs(gl - ref_l).max())
    if with_verify:
        ref_pack = oracle_pack(c)
        r_o, r_l = oracle_attn(c, ref_pack["offsets"])
        compare_attn(c, ref_pack["offsets"], out, lse, r_o, r_l, tag=tag + " verify")


@pytest.mark.parametrize("d_head,hq,hkv", [(128, 8, 2), (64, 4, 4), (256, 6, 2)])
def test_prefill_ragged(d_head, hq, hkv):
    c = _prefill_case(50 + d_head, q_len=[300, 77, 128, 1], ctx=[0, 50, 0, 9], hq=hq, hkv=hkv, d=d_head)
    _run_mixed(c, with_verify=False, tag=f"prefill d{d_head}")


@pytest.mark.parametrize("d_head,hq,hkv,q_len,ctx", [
    (128, 8, 2, [1100, 300, 600, 17], [0, 20, 0, 5]),   # KV-head grouped order, 5 row blocks
    (64, 4, 4, [700, 130, 1, 260], [3, 0, 0, 40]),      # plain order (one query head per KV head), 6
])
def test_prefill_rotation_wraps(d_head, hq, hkv, q_len, ctx):
    """More row blocks than requests with fewer than 8 heads per request, so the per-row-block
    turn of requests over the XCDs wraps round: every row still comes out once and right."""
    c = _prefill_case(63 + d_head, q_len=q_len, ctx=ctx, hq=hq, hkv=hkv, d=d_head)
    _run_mixed(c, with_verify=False, tag=f"prefill rotation d{d_head}")


# Query lengths and contexts around each head_dim's tile edges, so that rows end inside a
# wave, a wave's tile or a workgroup's row block, and contexts start the diagonal mid-tile:
# head_dim 128 runs 256-row workgroups of 8 waves x 32 rows on 32-row KV tiles; head_dim 64
# 256-row workgroups of 8 waves x 32 rows on 64-row KV tiles; head_dim 256 128-row workgroups
# of 8 waves x 16 rows on 32-row KV tiles.
_EDGES = {
    128: ([1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 511, 513], [0, 5, 31, 32, 33, 64, 100, 0, 7, 130, 1, 3], 8, 2),
    64: ([1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 257], [0, 5, 63, 64, 65, 128, 100, 0, 7, 130, 1, 3], 4, 1),
    256: ([1, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 257], [0, 5, 31, 32, 33, 64, 100, 0, 7, 130, 1, 3], 6, 2),
}


@pytest.mark.parametrize("d_head", [128, 64, 256])
def test_prefill_block_edges(d_head):
    q_len, ctx, hq, hkv = _EDGES[d_head]
    c = _prefill_case(61 + d_head, q_len=q_len, ctx=ctx, hq=hq, hkv=hkv, d=d_head)
    _run_mixed(c, with_verify=False, tag=f"prefill block edges d{d_head}")


@pytest.mark.parametrize("d_head,hq,hkv", [(64, 4, 2), (128, 8, 2), (256, 6, 2)])
def test_prefill_single_row_closed_form(d_head, hq, hkv):
    """A one-row prefill request with no context sees only its own key: probability exactly 1,
    so its output is its value row (pool row kv_base + 0) bit for bit and lse = scale q.k;
    the longer requests beside it are checked against the oracle."""
    c = _prefill_case(62 + d_head, q_len=[1, 40, 1], ctx=[0, 0, 0], hq=hq, hkv=hkv, d=d_head)
    _run_mixed(c, with_verify=False, tag=f"prefill single row d{d_head}")
    pf = c["prefill"]
    d = device_case(c)
    pf_q = to_dev(pf["q"])
    pf_out = torch.full_like(pf_q, float("nan"))
    pf_lse = torch.full((pf_q.shape[0], hq), float("nan"), device=DEV)
    prefill = dsv.Prefill(q_start=to_dev(pf["q_start"]), q_len=to_dev(pf["q_len"]),
                          ctx_len=to_dev(pf["ctx_len"]), kv_base=to_dev(pf["kv_base"]), q=pf_q,
                          out=pf_out, max_len=pf["max_len"], lse=pf_lse)
    dsv.verify_attn(None, d["k_pool"], d["v_pool"], None, None, d["ctx_len"], d["kv_base"], W=16,
                    max_ctx=0, status=d["status"], prefill=prefill)
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0
    G = hq // hkv
    q = to_f64(pf_q)
    kp = to_f64(d["k_pool"])
    for r in (0, 2):
        row, base = int(pf["q_start"][r]), int(pf["kv_base"][r])
        for h in range(hq):
            g = h // G
            assert torch.equal(pf_out[row, h].view(torch.int16), d["v_pool"][g, base].view(torch.int16)), (r, h)
            z = float(q[row, h] @ kp[g, base]) / np.sqrt(d_head)
            assert abs(float(pf_lse[row, h]) - z) <= 1e-3, (r, h, float(pf_lse[row, h]), z)


def test_prefill_fp32():
    c = _prefill_case(57, q_len=[70, 5], ctx=[0, 33], hq=4, hkv=2, d=64, dtype="f32")
    _run_mixed(c, with_verify=False, tag="prefill fp32")


def test_prefill_with_new_kv():
    c = _prefill_case(58, q_len=[200, 64], ctx=[0, 20])
    _run_mixed(c, with_verify=False, pf_new=True, tag="prefill k_new")


def test_mixed_verify_and_prefill():
    c = _prefill_case(59, q_len=[257, 40], ctx=[0, 0])
    _run_mixed(c, with_verify=True, tag="mixed")
