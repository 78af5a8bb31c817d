"""dsv_verify_attn_noalloc (the split partials in the library's fixed per-GPU scratch array,
no caller workspace) against dsv_verify_attn (a caller workspace) through the C ABI: two
calls in a row on one GPU, the second with a smaller batch and other head counts, each
bit-identical to the workspace entry point and within the attention tolerances of the oracle;
a call whose partials exceed the scratch array is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import block_verification_attention_amd as dsv  # noqa: E402
from block_verification_attention_amd import _lib  # noqa: E402
from gpu_util import DEV, compare_attn, device_case, gpu_pack, oracle_attn, oracle_pack, small_case  # noqa: E402

SCRATCH_BYTES = 32 << 20  # DSV_VERIFY_SCRATCH_BYTES


def _args(c, d, packed, out, lse, kv_chunk=0):
    return dsv.attn_args(d["q"], d["k_pool"], d["v_pool"], packed["offsets"], d["k"], d["ctx_len"],
                         d["kv_base"], W=c["W"], max_ctx=int(c["ctx_len"].max()), out=out,
                         status=d["status"], lse=lse, kv_chunk=kv_chunk)


def _both(c, kv_chunk=0):
    """Runs the case through both entry points (candidates already in the pool: the calls
    only read it).  Returns (noalloc out, lse), (workspace out, lse), pack offsets."""
    d = device_case(c)
    packed = gpu_pack(c, d)
    res = []
    for noalloc in (True, False):
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV)
        a = _args(c, d, packed, out, lse, kv_chunk)
        need = dsv.verify_attn_workspace_bytes(a)
        assert 0 < need <= SCRATCH_BYTES, need  # the case uses split partials
        if noalloc:
            a.workspace, a.workspace_bytes = None, 0
            dsv.verify_attn_noalloc_call(a)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
            dsv.verify_attn_call(a)
        torch.cuda.synchronize()
        assert int(d["status"].item()) == 0
        res.append((out, lse))
    return res[0], res[1], oracle_pack(c)["offsets"]


def test_noalloc_matches_workspace_entry_point_twice():
    big = small_case(901, hq=32, hkv=8, d=128, k=(16,) * 8, ctx=(4096,) * 8, extra_tail=0)
    small = small_case(902, hq=12, hkv=2, d=128, k=(9, 0, 16, 3), ctx=(1500, 10, 777, 2100))
    sizes = []
    for c in (big, small):
        (o1, l1), (o2, l2), off = _both(c)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
        ref_o, ref_l = oracle_attn(c, off, use_new=False)
        compare_attn(c, off, o1, l1, ref_o, ref_l, tag=f"noalloc {c['hq']}/{c['hkv']}")
        sizes.append(int(off[-1]))
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_partials_beyond_the_scratch_array():
    c = small_case(903, hq=32, hkv=8, d=128, k=(16,) * 8, ctx=(8192,) * 8, extra_tail=0)
    d = device_case(c)
    packed = gpu_pack(c, d)
    out = torch.zeros_like(d["q"])
    a = _args(c, d, packed, out, None, kv_chunk=64)  # 129 splits x 2 MB of partials
    assert dsv.verify_attn_workspace_bytes(a) > SCRATCH_BYTES
    rc = _lib.load().dsv_verify_attn_noalloc(ctypes.byref(a), None)
    assert rc == 3  # DSV_ERR_WORKSPACE, nothing enqueued
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0 and torch.count_nonzero(out.view(torch.int16)) == 0
