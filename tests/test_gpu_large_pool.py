"""Verification attention on KV pools past 2^31 elements per tensor (32-bit element offsets
would wrap): 2 KV heads x (2^24 + 40,000) rows x head_dim 128 per pool, 8.6 GB each, with the
requests' segments near the end of the pool, so both the row offset within a head and the
second head's offset exceed 2^31 elements.  Only the rows the call reads are filled (seeded);
the oracle receives compact copies of them.  The candidates' K/V written at their cache
references are checked bit for bit, for the separate and the fused packer and through a cache
map (int32 entries naming rows past 2^24); a prefill set
at the pool's end is checked row by row."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from gpu_util import DEV, TOL, bits_of, compare_attn, to_dev, to_f64  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402

POOL_ROWS = (1 << 24) + 40_000
HQ, HKV, D, W = 8, 2, 128, 16


def _dev_normal(g, shape):
    return (torch.randn(shape, generator=g, device=DEV) * 0.5).to(torch.bfloat16)


@pytest.mark.parametrize("mode", ["separate", "fused", "cache_map"])
def test_pool_offsets_past_2_31_elements(mode):
    assert (POOL_ROWS - 40_000) * D >= 1 << 31 and POOL_ROWS * D * HKV > 1 << 32
    k = np.array([16, 7, 1], np.int32)
    ctx = np.array([3000, 500, 1200], np.int32)
    base = np.array([POOL_ROWS - 39_000, POOL_ROWS - 30_000, POOL_ROWS - 1_300], np.int64)
    m_bs = int(k.sum()) + 5
    g = torch.Generator(device=DEV)
    g.manual_seed(7100 + ["separate", "fused", "cache_map"].index(mode))
    k_pool = torch.empty((HKV, POOL_ROWS, D), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.empty((HKV, POOL_ROWS, D), dtype=torch.bfloat16, device=DEV)
    for lo, cx in zip(base, ctx):
        k_pool[:, lo:lo + cx + W] = _dev_normal(g, (HKV, int(cx) + W, D))
        v_pool[:, lo:lo + cx + W] = _dev_normal(g, (HKV, int(cx) + W, D))
    q = _dev_normal(g, (m_bs, HQ, D))
    k_new = _dev_normal(g, (m_bs, HKV, D))
    v_new = _dev_normal(g, (m_bs, HKV, D))
    tokens = np.arange(3 * W, dtype=np.int32).reshape(3, W)

    # compact copies for the oracle, taken before the call writes the candidates
    kp_m = bits_of(torch.cat([k_pool[:, lo:lo + cx + W] for lo, cx in zip(base, ctx)], dim=1))
    vp_m = bits_of(torch.cat([v_pool[:, lo:lo + cx + W] for lo, cx in zip(base, ctx)], dim=1))
    kb_m = np.concatenate([[0], np.cumsum(ctx.astype(np.int64) + W)[:-1]]).astype(np.int64)

    st = dsv.new_status(DEV)
    kd, cd, bd, td = to_dev(k), to_dev(ctx), to_dev(base), to_dev(tokens)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((m_bs, HQ), float("nan"), device=DEV)
    if mode == "fused":
        args = dsv.attn_args(q, k_pool, v_pool, None, kd, cd, bd, W=W, max_ctx=int(ctx.max()),
                             out=out, status=st, lse=lse, k_new=k_new, v_new=v_new)
        ws = torch.empty(max(dsv.verify_attn_workspace_bytes(args), 256), dtype=torch.uint8, device=DEV)
        args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
        packed = dsv.pack_verify_attn(args, td)
    elif mode == "cache_map":
        # identity map: position p of request i -> pool row base[i] + p (int32 entries)
        stride = int((ctx + W).max())
        idx = np.minimum(base[:, None] + np.arange(stride)[None, :], POOL_ROWS - 1).astype(np.int32)
        packed = dsv.pack_slots(kd, cd, bd, td, m_bs, st)
        a = dsv.attn_args(q, k_pool, v_pool, packed["offsets"], kd, cd, bd, W=W, max_ctx=int(ctx.max()),
                          out=out, status=st, lse=lse, k_new=k_new, v_new=v_new,
                          slot_cache_loc=packed["slot_cache_loc"], kv_index=to_dev(idx))
        ws = torch.empty(max(dsv.verify_attn_workspace_bytes(a), 256), dtype=torch.uint8, device=DEV)
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        dsv.verify_attn_call(a)
    else:
        packed = dsv.pack_slots(kd, cd, bd, td, m_bs, st)
        dsv.verify_attn(q, k_pool, v_pool, packed["offsets"], kd, cd, bd, W=W, max_ctx=int(ctx.max()),
                        status=st, out=out, lse=lse, k_new=k_new, v_new=v_new,
                        slot_cache_loc=packed["slot_cache_loc"])
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref_pack = oracle.pack(k, ctx, base, tokens, W, m_bs)
    offs = ref_pack["offsets"]
    assert np.array_equal(packed["offsets"].cpu().numpy(), offs)
    assert np.array_equal(packed["slot_cache_loc"].cpu().numpy(), ref_pack["slot_cache_loc"])

    n = int(offs[-1])
    loc = torch.as_tensor(ref_pack["slot_cache_loc"][:n], device=DEV)
    assert torch.equal(k_pool[:, loc].transpose(0, 1).view(torch.int16), k_new[:n].view(torch.int16))
    assert torch.equal(v_pool[:, loc].transpose(0, 1).view(torch.int16), v_new[:n].view(torch.int16))

    ref_o, ref_l = oracle.verify_attn(bits_of(q[:n]), kp_m, vp_m, offs, k, ctx, kb_m,
                                      k_new=bits_of(k_new[:n]), v_new=bits_of(v_new[:n]))
    c = dict(n_bs=3, k=k, hq=HQ, dtype="bf16", m_bs=n)
    compare_attn(c, offs, out[:n], lse[:n], ref_o, ref_l, tag=f"large pool, {mode}")
    assert torch.all(out[n:] == 0) and torch.all(torch.isneginf(lse[n:]))
    del k_pool, v_pool
    torch.cuda.empty_cache()


def test_prefill_pool_offsets_past_2_31_elements():
    # two prefill requests whose KV segments lie past element 2^31 of both heads; every row
    # of both against the oracle on compact copies
    q_len = np.array([300, 77], np.int32)
    ctx = np.array([0, 150], np.int32)
    base = np.array([POOL_ROWS - 20_000, POOL_ROWS - 400], np.int64)
    q_start = np.array([0, 300], np.int32)
    rows = int(q_len.sum())
    g = torch.Generator(device=DEV)
    g.manual_seed(7110)
    k_pool = torch.empty((HKV, POOL_ROWS, D), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.empty((HKV, POOL_ROWS, D), dtype=torch.bfloat16, device=DEV)
    for lo, n in zip(base, ctx + q_len):
        k_pool[:, lo:lo + n] = _dev_normal(g, (HKV, int(n), D))
        v_pool[:, lo:lo + n] = _dev_normal(g, (HKV, int(n), D))
    q = _dev_normal(g, (rows, HQ, D))
    kp_m = bits_of(torch.cat([k_pool[:, lo:lo + n] for lo, n in zip(base, ctx + q_len)], dim=1))
    vp_m = bits_of(torch.cat([v_pool[:, lo:lo + n] for lo, n in zip(base, ctx + q_len)], dim=1))
    kb_m = np.array([0, int(ctx[0] + q_len[0])], np.int64)

    st = dsv.new_status(DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((rows, HQ), float("nan"), device=DEV)
    pf = dsv.Prefill(q_start=to_dev(q_start), q_len=to_dev(q_len), ctx_len=to_dev(ctx),
                     kv_base=to_dev(base), q=q, out=out, max_len=int(q_len.max()), lse=lse)
    args = dsv.attn_args(None, k_pool, v_pool, None, None, None, None, W=W, max_ctx=0, out=None,
                         status=st, prefill=pf)
    dsv.verify_attn_call(args)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    sel_req = [r for r in range(2) for _ in range(int(q_len[r]))]
    sel_j = [j for r in range(2) for j in range(int(q_len[r]))]
    ref_o, ref_l = oracle.prefill_attn(bits_of(q), kp_m, vp_m, q_start, q_len, ctx, kb_m, sel_req, sel_j)
    go, gl = to_f64(out), to_f64(lse)
    tol = TOL["bf16"]
    assert np.all(np.isfinite(go))
    assert np.abs(go - ref_o).max() <= tol["max_abs"], np.abs(go - ref_o).max()
    for h in range(HQ):
        rel = np.linalg.norm(go[:, h] - ref_o[:, h]) / np.linalg.norm(ref_o[:, h])
        assert rel <= tol["rel_l2"], (h, rel)
    assert np.abs(gl - ref_l).max() <= tol["lse"], np.abs(gl - ref_l).max()
    del k_pool, v_pool
    torch.cuda.empty_cache()
