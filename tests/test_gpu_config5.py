"""Parity at the full size of the mixed launch whose parts the bench times (its long-context
verification set and its prefill wide tile): 60 verification requests with ragged prefixes in
a 480-slot budget and contexts U[8192, 32768], and 4 fresh prefill requests of 4096 causal
rows, in ONE dsv_verify_attn call; 32 query / 8 KV heads, head_dim 128, bf16.

The K/V pool (2 x 8 x 1.27M x 128, ~5 GB) is drawn on the device from seeded generators,
N(0,1) * 0.5 rounded to bf16 (the workload's distribution; a numpy draw of that size would
take minutes).  The oracle receives host copies of the pool and checks every verification
slot and head of all 60 requests, and 512 rows of every prefill request (the first 64, the
last 64 and 384 seeded ones between them); every prefill output row is checked to be finite.
The candidate K/V written into the pool are checked bit for bit at the packed cache
references of all 60 requests.  The launch runs both as dsv_pack_slots + dsv_verify_attn and
as dsv_pack_verify_attn (the packer fused into it)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import DEV, TOL, bits_of, compare_attn, to_dev, to_f64  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402


def _dev_normal(seed, shape, scale=0.5):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("fused_pack", [False, True])
def test_config5_mixed_launch(fused_pack):
    c = wl.config5(draw=False)
    hq, hkv, d, W = c["hq"], c["hkv"], c["d"], c["W"]
    n, m_bs, pool_rows = c["n_bs"], c["m_bs"], c["pool_rows"]
    pf = c["prefill"]
    pf_rows = int(pf["q_len"].sum())
    k_pool = _dev_normal(5101, (hkv, pool_rows, d))
    v_pool = _dev_normal(5102, (hkv, pool_rows, d))
    q = _dev_normal(5103, (m_bs, hq, d))
    k_new = _dev_normal(5104, (m_bs, hkv, d))
    v_new = _dev_normal(5105, (m_bs, hkv, d))
    pf_q = _dev_normal(5109, (pf_rows, hq, d))

    ref_pack = oracle.pack(c["k"], c["ctx_len"], c["kv_base"], c["block_tokens"], W, m_bs)
    offs = ref_pack["offsets"]
    pf_lo = int(pf["kv_base"][0])
    assert np.array_equal(pf["kv_base"] - pf_lo, np.asarray(pf["q_start"], np.int64))

    st = dsv.new_status(DEV)
    kd, cd, bd = to_dev(c["k"]), to_dev(c["ctx_len"]), to_dev(c["kv_base"])
    tok = to_dev(c["block_tokens"])
    packed = dsv.pack_slots(kd, cd, bd, tok, m_bs, st)
    if fused_pack:  # the fused call must produce these outputs itself
        for t in packed.values():
            t.fill_(-3)
    pf_out = torch.full_like(pf_q, float("nan"))
    pf_lse = torch.full((pf_rows, hq), float("nan"), device=DEV)
    prefill = dsv.Prefill(q_start=to_dev(pf["q_start"]), q_len=to_dev(pf["q_len"]),
                          ctx_len=to_dev(pf["ctx_len"]), kv_base=to_dev(pf["kv_base"]), q=pf_q,
                          out=pf_out, max_len=pf["max_len"], lse=pf_lse)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((m_bs, hq), float("nan"), device=DEV)
    if fused_pack:
        args = dsv.attn_args(q, k_pool, v_pool, None, kd, cd, bd, W=W, max_ctx=int(c["ctx_len"].max()),
                             out=out, status=st, lse=lse, k_new=k_new, v_new=v_new, prefill=prefill)
        ws = torch.empty(max(dsv.verify_attn_workspace_bytes(args), 256), dtype=torch.uint8, device=DEV)
        args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
        dsv.pack_verify_attn(args, tok, out=packed)
    else:
        dsv.verify_attn(q, k_pool, v_pool, packed["offsets"], kd, cd, bd, W=W,
                        max_ctx=int(c["ctx_len"].max()), status=st, out=out, lse=lse, k_new=k_new,
                        v_new=v_new, slot_cache_loc=packed["slot_cache_loc"], prefill=prefill)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(packed["offsets"].cpu().numpy(), offs)
    for key in ("slot_req", "slot_tok", "slot_pos", "slot_cache_loc"):
        assert np.array_equal(packed[key].cpu().numpy(), ref_pack[key]), key

    # candidate K/V at the packed cache references, all requests, bit for bit
    loc = torch.as_tensor(ref_pack["slot_cache_loc"][:int(offs[-1])], device=DEV)
    assert torch.equal(k_pool[:, loc].transpose(0, 1).view(torch.int16), k_new[:int(offs[-1])].view(torch.int16))
    assert torch.equal(v_pool[:, loc].transpose(0, 1).view(torch.int16), v_new[:int(offs[-1])].view(torch.int16))

    # every verification slot and head (the call wrote only candidate rows of the pool, which
    # the oracle takes from k_new/v_new; the context rows it reads are unchanged)
    kp_h, vp_h = bits_of(k_pool), bits_of(v_pool)
    ref_o, ref_l = oracle.verify_attn(bits_of(q), kp_h, vp_h, offs, c["k"], c["ctx_len"], c["kv_base"],
                                      k_new=bits_of(k_new), v_new=bits_of(v_new))
    mc = dict(n_bs=n, k=c["k"], hq=hq, dtype="bf16", m_bs=m_bs)
    compare_attn(mc, offs, out, lse, ref_o, ref_l, tag="config 5 verification")

    # prefill rows: the first 64, the last 64 and 384 seeded ones between them, per request
    assert torch.isfinite(pf_out.float()).all() and torch.isfinite(pf_lse).all()
    g = np.random.default_rng(5110)
    sel_req, sel_j = [], []
    for r in range(pf["n_pf"]):
        ql = int(pf["q_len"][r])
        mid = g.choice(np.arange(64, ql - 64), 384, replace=False).tolist()
        js = sorted(set(list(range(64)) + list(range(ql - 64, ql)) + mid))
        assert len(js) == 512
        sel_req += [r] * len(js)
        sel_j += js
    kp_pf, vp_pf = kp_h[:, pf_lo:pf_lo + pf_rows], vp_h[:, pf_lo:pf_lo + pf_rows]
    ref_po, ref_pl = oracle.prefill_attn(bits_of(pf_q), kp_pf, vp_pf, pf["q_start"], pf["q_len"],
                                         pf["ctx_len"], np.asarray(pf["q_start"], np.int64),
                                         sel_req, sel_j)
    idx = torch.as_tensor([int(pf["q_start"][r]) + j for r, j in zip(sel_req, sel_j)], device=DEV)
    go, gl = to_f64(pf_out[idx]), to_f64(pf_lse[idx])
    tol = TOL["bf16"]
    assert np.all(np.isfinite(go))
    assert np.abs(go - ref_po).max() <= tol["max_abs"], np.abs(go - ref_po).max()
    for h in range(hq):
        rel = np.linalg.norm(go[:, h] - ref_po[:, h]) / np.linalg.norm(ref_po[:, h])
        assert rel <= tol["rel_l2"], (h, rel)
    assert np.abs(gl - ref_pl).max() <= tol["lse"], np.abs(gl - ref_pl).max()
