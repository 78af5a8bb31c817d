"""GPU parity of dsv_pack_verify_attn (the packer fused into the verification launch): its
packer outputs equal dsv_pack_slots' bit for bit, and its attention outputs equal, bit for
bit, those of dsv_pack_slots followed by dsv_verify_attn (same kernels and arithmetic once the
offsets are formed), and the oracle's within the attention tolerances.  Malformed requests
and a budget overflow take no slots and get no rows; graph replays repeat the eager call."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from gpu_util import (DEV, compare_attn, device_case, gpu_attn, gpu_pack, oracle_attn,  # noqa: E402
                      oracle_pack, small_case, to_dev)
import block_verification_attention_amd as dsv  # noqa: E402

PACK_KEYS = ("offsets", "slot_req", "slot_tok", "slot_pos", "slot_cache_loc")


def _fused(c, d, *, kv_chunk=0, k=None, ctx_len=None, kv_base=None, status=None):
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV)
    st = d["status"] if status is None else status
    args = dsv.attn_args(d["q"], d["k_pool"], d["v_pool"], None, d["k"] if k is None else k,
                         d["ctx_len"] if ctx_len is None else ctx_len,
                         d["kv_base"] if kv_base is None else kv_base, W=c["W"],
                         max_ctx=int(c["ctx_len"].max()), out=out, status=st, lse=lse,
                         k_new=d["k_new"], v_new=d["v_new"], kv_chunk=kv_chunk)
    ws = torch.empty(max(dsv.verify_attn_workspace_bytes(args), 256), dtype=torch.uint8, device=DEV)
    args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    packed = dsv.pack_verify_attn(args, d["block_tokens"])
    return packed, out, lse, (args, ws)


def _same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _check_against_composed_and_oracle(c, kv_chunk=0, tag=""):
    d = device_case(c)
    ref_pack_gpu = gpu_pack(c, d)
    ref_out, ref_lse = gpu_attn(c, d, ref_pack_gpu, kv_chunk=kv_chunk)
    # a fresh pool: the composed call already wrote this step's candidate KV into the first one
    d2 = device_case(c)
    packed, out, lse, _ = _fused(c, d2, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0 and int(d2["status"].item()) == 0, tag
    for key in PACK_KEYS:
        assert torch.equal(packed[key], ref_pack_gpu[key]), (tag, key)
    assert _same_bits(out, ref_out) and _same_bits(lse, ref_lse), tag
    assert torch.equal(d2["k_pool"].view(torch.int16), d["k_pool"].view(torch.int16)), tag
    assert torch.equal(d2["v_pool"].view(torch.int16), d["v_pool"].view(torch.int16)), tag
    ref = oracle_pack(c)
    r_o, r_l = oracle_attn(c, ref["offsets"])
    compare_attn(c, ref["offsets"], out, lse, r_o, r_l, tag=tag)


def test_config3_full():
    _check_against_composed_and_oracle(wl.config3(with_logits=False), tag="cfg3")


@pytest.mark.parametrize("d_head,hq,hkv", [(128, 32, 8), (64, 16, 2), (256, 24, 2), (128, 13, 1), (256, 4, 4)])
@pytest.mark.parametrize("kv_chunk", [0, 64])
def test_ragged(d_head, hq, hkv, kv_chunk):
    c = small_case(300 + d_head + hq, hq=hq, hkv=hkv, d=d_head,
                   k=(16, 5, 0, 11, 1, 16, 3), ctx=(700, 0, 40, 63, 64, 1000, 129))
    _check_against_composed_and_oracle(c, kv_chunk=kv_chunk, tag=f"d{d_head} hq{hq} chunk{kv_chunk}")


def test_many_requests():
    g = np.random.default_rng(5)
    k = wl.lengths_geometric_rescaled(g, 200, 1600)
    c = small_case(333, hq=32, hkv=8, d=128, k=tuple(int(x) for x in k),
                   ctx=tuple(int(x) for x in g.integers(0, 300, 200)))
    _check_against_composed_and_oracle(c, tag="200 requests")


def test_1500_requests():
    # more requests than one 1024-thread block covers: every workgroup's prologue sums 1500
    # effective lengths; short contexts keep the oracle quick
    g = np.random.default_rng(6)
    k = wl.lengths_geometric_rescaled(g, 1500, 12000)
    c = small_case(334, hq=8, hkv=2, d=64, k=tuple(int(x) for x in k),
                   ctx=tuple(int(x) for x in g.integers(0, 120, 1500)))
    _check_against_composed_and_oracle(c, tag="1500 requests")


def test_malformed_requests_take_no_slots():
    c = small_case(340, hq=8, hkv=2, d=128, k=(4, 6, 3, 5, 2), ctx=(10, 20, 30, 40, 50))
    d = device_case(c)
    k_bad = d["k"].clone()
    k_bad[1] = 17                     # longer than W
    ctx_bad = d["ctx_len"].clone()
    ctx_bad[3] = -1                   # negative context
    st = dsv.new_status(DEV)
    packed, out, lse, _ = _fused(c, d, k=k_bad, ctx_len=ctx_bad, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == dsv.STATUS_BAD_REQUEST
    off = packed["offsets"].cpu().numpy()
    assert list(off) == [0, 4, 4, 7, 7, 9]
    assert np.all(packed["slot_req"].cpu().numpy()[:9] == [0, 0, 0, 0, 2, 2, 2, 4, 4])
    assert torch.all(out[9:] == 0) and torch.all(torch.isneginf(lse[9:]))
    # the well-formed requests match the oracle run on them alone
    keep = [0, 2, 4]
    sub = dict(c, n_bs=3, k=c["k"][keep], ctx_len=c["ctx_len"][keep], kv_base=c["kv_base"][keep],
               block_tokens=c["block_tokens"][keep])
    ref_off = np.array([0, 4, 7, 9], np.int32)
    r_o, r_l = oracle_attn(sub, ref_off)
    compare_attn(dict(sub, m_bs=9), ref_off, out[:9], lse[:9], r_o[:9], r_l[:9], tag="malformed")


def test_budget_overflow_drops_every_request():
    c = small_case(341, hq=8, hkv=2, d=128, k=(16, 16, 16), ctx=(100, 200, 300), extra_tail=0)
    d = device_case(c)
    k_big = d["k"].clone()
    k_big[0] = 15  # valid, but the lengths below sum above m_bs
    c2 = dict(c, m_bs=40)
    d2 = dict(d, q=d["q"][:40].contiguous(), k_new=d["k_new"][:40].contiguous(),
              v_new=d["v_new"][:40].contiguous())
    st = dsv.new_status(DEV)
    packed, out, lse, _ = _fused(c2, d2, k=k_big, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == dsv.STATUS_BUDGET
    assert np.all(packed["offsets"].cpu().numpy() == 0)
    assert torch.all(packed["slot_req"] == -1) and torch.all(packed["slot_cache_loc"] == -1)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_graph_replays_match_eager():
    c = small_case(342, hq=32, hkv=8, d=128, k=(16, 9, 1, 12, 0, 7), ctx=(900, 1500, 5, 260, 3, 2000))
    d = device_case(c)
    packed, out, lse, (args, ws) = _fused(c, d, kv_chunk=256)
    torch.cuda.synchronize()
    eager = [t.clone() for t in [packed[k] for k in PACK_KEYS] + [out, lse]]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dsv.pack_verify_attn(args, d["block_tokens"], out=packed)
    for r in range(3):
        for t in [packed[k] for k in PACK_KEYS] + [out, lse]:
            t.fill_(-7) if t.dtype in (torch.int32, torch.int64) else t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (t, e) in enumerate(zip([packed[k] for k in PACK_KEYS] + [out, lse], eager)):
            assert _same_bits(t, e), f"replay {r}, output {j}"
    assert int(d["status"].item()) == 0
