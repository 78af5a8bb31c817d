"""GPU parity of dsv_verify_attn (verification path) against the oracle."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from gpu_util import (DEV, bits_of, compare_attn, device_case, gpu_attn, gpu_pack,  # noqa: E402
                      oracle_attn, oracle_pack, small_case, to_dev, to_f64)
import block_verification_attention_amd as dsv  # noqa: E402


def _run(c, *, use_new=True, kv_chunk=0, tag=""):
    d = device_case(c)
    packed = gpu_pack(c, d)
    ref_pack = oracle_pack(c)
    assert np.array_equal(packed["offsets"].cpu().numpy(), ref_pack["offsets"])
    out, lse = gpu_attn(c, d, packed, use_new=use_new, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0
    ref_out, ref_lse = oracle_attn(c, ref_pack["offsets"], use_new=use_new)
    w = compare_attn(c, ref_pack["offsets"], out, lse, ref_out, ref_lse, tag=tag or c["name"])
    return d, packed, out, lse, w


def test_config1_fp32():
    _run(wl.config1(), tag="cfg1")


@pytest.mark.parametrize("d_head,hq,hkv", [(64, 4, 1), (128, 8, 2), (128, 32, 8), (256, 24, 2),
                                            (128, 12, 4), (256, 4, 4), (128, 16, 1), (128, 24, 2),
                                            (256, 8, 1), (256, 6, 2), (64, 16, 2), (128, 13, 1),
                                            # groups split unevenly over workgroups (the last
                                            # one holds fewer heads) or padded to a wider one
                                            (128, 9, 1), (128, 11, 1), (256, 5, 1), (256, 7, 1),
                                            (256, 10, 1), (256, 13, 1), (128, 2, 1), (128, 6, 1),
                                            # head_dim 256 with one or two query heads per KV
                                            # head (waves without heads in the 4-wave kernel)
                                            (256, 2, 1), (256, 8, 4),
                                            # head_dim 128 groups of 5 and 7, head_dim 64 of
                                            # 7 and 6 (padded to 8 waves)
                                            (128, 5, 1), (128, 14, 2), (64, 7, 1), (64, 12, 2),
                                            # head_dim 256 with 8 KV heads and one workgroup
                                            # per KV head (the ten-per-CU split plan)
                                            (256, 8, 8), (256, 32, 8)])
@pytest.mark.parametrize("kv_chunk", [0, 64, 256])
def test_bf16_ragged(d_head, hq, hkv, kv_chunk):
    c = small_case(10 + d_head + hq, hq=hq, hkv=hkv, d=d_head,
                   k=(16, 5, 0, 11, 1, 16, 3), ctx=(700, 0, 40, 63, 64, 1000, 129))
    _run(c, kv_chunk=kv_chunk, tag=f"d{d_head} hq{hq} hkv{hkv} chunk{kv_chunk}")


@pytest.mark.parametrize("kv_chunk", [0, 128])
def test_wide_heads_score_jump_sharp_sentinel(kv_chunk):
    """head_dim 256 with 12 query heads per KV head (head groups of up to 4, one wave per head): keys
    deep in a split whose scores jump far above the split's first tile (a query row's own
    direction x 30, so the softmax reference must move); the sharp (queries x 8) and
    leak-detector variants of the same batch run too."""
    base = small_case(61, hq=12, hkv=1, d=256, k=(16, 7, 3, 1, 12), ctx=(1500, 600, 90, 2000, 33))
    off = oracle_pack(base)["offsets"]
    kp = wl.bf16_bits_to_f32(base["k_pool"]).copy()
    q = wl.bf16_bits_to_f32(base["q"])
    for i, pos, j, h in ((0, 1330, 5, 2), (3, 1960, 0, 7), (1, 300, 6, 11)):
        kp[0, int(base["kv_base"][i]) + pos] = q[int(off[i]) + j, h] * np.float32(30.0)
    jump = dict(base, k_pool=wl.to_bf16_bits(kp), name=base["name"] + "-jump")
    _run(jump, kv_chunk=kv_chunk, tag=f"score jump chunk{kv_chunk}")
    _run(wl.sharp_variant(base), kv_chunk=kv_chunk, tag=f"wide sharp chunk{kv_chunk}")
    _run(wl.sentinel_variant(base), kv_chunk=kv_chunk, tag=f"wide sentinel chunk{kv_chunk}")


@pytest.mark.parametrize("d_head", [64, 128, 256])
def test_fp32_small(d_head):
    c = small_case(31 + d_head, dtype="f32", hq=4, hkv=2, d=d_head, k=(4, 0, 16, 1), ctx=(50, 3, 0, 300))
    _run(c)


def test_pool_candidates_without_k_new():
    c = small_case(41, k=(7, 16, 2), ctx=(100, 0, 500))
    _run(c, use_new=False, kv_chunk=128)


def test_sharp_and_sentinel():
    base = small_case(42, hq=16, hkv=4, d=128, k=(16, 9, 4, 1), ctx=(1000, 20, 333, 0))
    _run(wl.sharp_variant(base), tag="sharp")
    _run(wl.sentinel_variant(base), kv_chunk=256, tag="sentinel")
    _run(wl.sentinel_variant(wl.sharp_variant(base)), tag="sentinel+sharp")


def test_candidate_kv_written_at_cache_refs():
    c = small_case(43, k=(5, 0, 16), ctx=(10, 7, 200))
    d, packed, *_ = _run(c)
    ref_k, ref_v = oracle.scatter_candidates(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                             oracle_pack(c)["slot_cache_loc"])
    assert np.array_equal(bits_of(d["k_pool"]), ref_k)
    assert np.array_equal(bits_of(d["v_pool"]), ref_v)


def test_pools_interleaved_by_head():
    """K and V pools as two views of one allocation [hkv][2][rows][d]: interleaved by head,
    their byte ranges overlap, which the aliasing check allows for the pools (they are
    compared only with the other buffers).  Parity, and the candidate rows written into
    their own view."""
    c = small_case(44, hq=8, hkv=2, d=128, k=(16, 5, 0, 11), ctx=(300, 0, 40, 129))
    d = device_case(c)
    hkv, rows, dd = d["k_pool"].shape
    buf = torch.empty((hkv, 2, rows, dd), dtype=d["k_pool"].dtype, device=DEV)
    buf[:, 0] = d["k_pool"]
    buf[:, 1] = d["v_pool"]
    d["k_pool"], d["v_pool"] = buf[:, 0], buf[:, 1]
    packed = gpu_pack(c, d)
    ref_pack = oracle_pack(c)
    out, lse = gpu_attn(c, d, packed)
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0
    ref_out, ref_lse = oracle_attn(c, ref_pack["offsets"])
    compare_attn(c, ref_pack["offsets"], out, lse, ref_out, ref_lse, tag="pools interleaved by head")
    ref_k, ref_v = oracle.scatter_candidates(c["k_pool"], c["v_pool"], c["k_new"], c["v_new"],
                                             ref_pack["slot_cache_loc"])
    assert np.array_equal(bits_of(buf[:, 0]), ref_k)
    assert np.array_equal(bits_of(buf[:, 1]), ref_v)


def test_packed_equals_padded_and_deterministic():
    """Same requests launched packed and padded (each request owns W rows, gaps between
    them): valid rows are bit-identical with the split size pinned; two runs agree bitwise."""
    c = small_case(44, hq=8, hkv=2, d=128, k=(3, 16, 7, 1), ctx=(300, 64, 0, 1025), extra_tail=0)
    d = device_case(c)
    packed = gpu_pack(c, d)
    o1, l1 = gpu_attn(c, d, packed, use_new=False, kv_chunk=128)
    o2, l2 = gpu_attn(c, d, packed, use_new=False, kv_chunk=128)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    n, W = c["n_bs"], c["W"]
    off = packed["offsets"].cpu().numpy()
    q_pad = torch.zeros((n * W, c["hq"], c["d"]), dtype=torch.bfloat16, device=DEV)
    for i in range(n):
        q_pad[i * W:i * W + c["k"][i]] = d["q"][off[i]:off[i] + c["k"][i]]
    pad_off = torch.arange(0, n * W + 1, W, dtype=torch.int32, device=DEV)
    cp = dict(c, m_bs=n * W)
    dp = dict(d, q=q_pad)
    out_pad = torch.full_like(q_pad, float("nan"))
    op, lp = gpu_attn(cp, dp, packed, use_new=False, kv_chunk=128, out=out_pad, offsets=pad_off)
    torch.cuda.synchronize()
    for i in range(n):
        kk = int(c["k"][i])
        assert torch.equal(op[i * W:i * W + kk].view(torch.int16), o1[off[i]:off[i] + kk].view(torch.int16))
        assert torch.equal(lp[i * W:i * W + kk], l1[off[i]:off[i] + kk])
        # gap rows of the padded layout are not touched
        assert torch.isnan(op[i * W + kk:(i + 1) * W].float()).all()


def test_config2_two_steps_layout_shift():
    """Step 1 [4,12,8] then step 2 [10,8,6] in the same pool: step 1's candidates are written
    at their cache references, the committed prefix (anchor + accepted drafts) becomes step 2's
    context, and step 2's new boundaries never mix requests."""
    s1, s2 = wl.config2()
    d1 = device_case(s1)
    p1 = gpu_pack(s1, d1)
    o1, l1 = gpu_attn(s1, d1, p1)
    torch.cuda.synchronize()
    ref1 = oracle_pack(s1)
    r1o, r1l = oracle_attn(s1, ref1["offsets"])
    compare_attn(s1, ref1["offsets"], o1, l1, r1o, r1l, tag="cfg2 step1")
    # oracle's view of the pool after step 1
    kp, vp = oracle.scatter_candidates(s1["k_pool"], s1["v_pool"], s1["k_new"], s1["v_new"],
                                       ref1["slot_cache_loc"])
    # step 2 runs on the device pool step 1 wrote
    d2 = device_case(s2)
    d2["k_pool"], d2["v_pool"] = d1["k_pool"], d1["v_pool"]
    p2 = gpu_pack(s2, d2)
    o2, l2 = gpu_attn(s2, d2, p2)
    torch.cuda.synchronize()
    assert int(d1["status"].item()) == 0 and int(d2["status"].item()) == 0
    ref2 = oracle_pack(s2)
    assert list(ref1["offsets"]) == [0, 4, 16, 24] and list(ref2["offsets"]) == [0, 10, 18, 24]
    r2o, r2l = oracle_attn(s2, ref2["offsets"], k_pool=kp, v_pool=vp)
    compare_attn(s2, ref2["offsets"], o2, l2, r2o, r2l, tag="cfg2 step2")


def test_config3_full():
    c = wl.config3(with_logits=False)
    _run(c, tag="cfg3")


def test_config4_full():
    c = wl.config4(with_draft_logits=False)
    _run(c, tag="cfg4")


def test_invalid_requests_flagged_and_zeroed():
    c = small_case(45, k=(4, 6, 3), ctx=(10, 20, 30))
    d = device_case(c)
    packed = gpu_pack(c, d)
    # request 1's segment pushed past the pool; request 2 claims k > W
    kb = d["kv_base"].clone()
    kb[1] = c["pool_rows"] - 5
    d2 = dict(d, kv_base=kb)
    k_bad = d["k"].clone()
    k_bad[2] = 17
    out, lse = gpu_attn(c, d2, packed, k=k_bad)
    torch.cuda.synchronize()
    st = int(d["status"].item())
    assert st & dsv.STATUS_POOL and st & dsv.STATUS_BAD_REQUEST
    off = packed["offsets"].cpu().numpy()
    assert torch.all(out[off[1]:off[1] + 6] == 0)
    assert torch.isfinite(out[off[0]:off[0] + 4].float()).all()
    # request 2 (k > W) has out-of-range k: its rows are left untouched
    assert torch.isnan(out[off[2]:off[2] + 3].float()).all()


@pytest.mark.parametrize("d_head,hq,hkv", [(64, 4, 2), (128, 8, 2), (256, 6, 2), (256, 2, 2)])
def test_zero_context_requests(d_head, hq, hkv):
    """Requests with no committed context.  A single anchor (k_i = 1, ctx_i = 0) sees only
    itself: its probability is exactly 1, so its output is its own value row bit for bit and
    lse = scale q.k; longer zero-context requests attend over their candidates only (oracle)."""
    c = small_case(48 + d_head, hq=hq, hkv=hkv, d=d_head, k=(1, 16, 1, 0, 2, 1), ctx=(0, 0, 0, 0, 0, 0))
    d, packed, out, lse, _ = _run(c, tag=f"zero context d{d_head}")
    off = packed["offsets"].cpu().numpy()
    G = hq // hkv
    q = to_f64(d["q"])
    kn = to_f64(d["k_new"])
    for i in np.nonzero(c["k"] == 1)[0]:
        s = int(off[i])
        for h in range(hq):
            assert torch.equal(out[s, h].view(torch.int16), d["v_new"][s, h // G].view(torch.int16)), (i, h)
            z = float(q[s, h] @ kn[s, h // G]) / np.sqrt(d_head)
            assert abs(float(lse[s, h]) - z) <= 1e-3, (i, h, float(lse[s, h]), z)


def test_all_requests_inactive():
    """Every k_i = 0: nothing is attended, every row is a tail row (zero output, lse -inf)
    and the pool is left as it was."""
    c = small_case(49, k=(0, 0, 0, 0), ctx=(40, 0, 700, 3), extra_tail=8)
    d = device_case(c)
    packed = gpu_pack(c, d)
    assert int(packed["offsets"][-1].item()) == 0
    k_pool0, v_pool0 = d["k_pool"].clone(), d["v_pool"].clone()
    out, lse = gpu_attn(c, d, packed, kv_chunk=64)
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0
    assert torch.all(out.float() == 0)
    assert torch.all(torch.isneginf(lse))
    assert torch.equal(d["k_pool"].view(torch.int16), k_pool0.view(torch.int16))
    assert torch.equal(d["v_pool"].view(torch.int16), v_pool0.view(torch.int16))


def test_context_beyond_plan_is_exact():
    """max_ctx only shapes the split plan: a request whose context exceeds it is still computed
    exactly (its last split is longer)."""
    c = small_case(46, k=(4, 16, 2), ctx=(900, 100, 2500))
    d = device_case(c)
    packed = gpu_pack(c, d)
    out, lse = gpu_attn(c, d, packed, kv_chunk=64, max_ctx=500)
    torch.cuda.synchronize()
    assert int(d["status"].item()) == 0
    ref = oracle_pack(c)
    r_o, r_l = oracle_attn(c, ref["offsets"])
    compare_attn(c, ref["offsets"], out, lse, r_o, r_l, tag="beyond plan")


def test_workspace_reused_across_calls():
    """One workspace serves consecutive calls at a fixed address, across different requests."""
    cases = [small_case(47 + s, hq=8, hkv=2, d=128, k=(16, 7, 3), ctx=(900, 1500, 64)) for s in range(3)]
    dev_ws = None
    for c in cases:
        d = device_case(c)
        packed = gpu_pack(c, d)
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV)
        args = dsv.attn_args(d["q"], d["k_pool"], d["v_pool"], packed["offsets"], d["k"], d["ctx_len"],
                             d["kv_base"], W=16, max_ctx=1500, out=out, status=d["status"], lse=lse,
                             k_new=d["k_new"], v_new=d["v_new"], slot_cache_loc=packed["slot_cache_loc"],
                             kv_chunk=128)
        need = dsv.verify_attn_workspace_bytes(args)
        if dev_ws is None:
            dev_ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)  # no clearing needed
        args.workspace, args.workspace_bytes = dev_ws.data_ptr(), dev_ws.numel()
        dsv.verify_attn_call(args)
        torch.cuda.synchronize()
        assert int(d["status"].item()) == 0
        ref = oracle_pack(c)
        r_o, r_l = oracle_attn(c, ref["offsets"])
        compare_attn(c, ref["offsets"], out, lse, r_o, r_l, tag=f"reuse {c['name']}")


def test_step_graph_capture_replays_match_eager():
    """The three calls of a step (pack, verify attention with candidate KV writes and split
    merge, accept) are capturable: a captured step replayed several times, with eager work and
    synchronisation between replays, reproduces the eager outputs bit for bit each time."""
    c = small_case(48, hq=8, hkv=2, d=128, k=(16, 9, 1, 12), ctx=(700, 1300, 5, 260), vocab=3000)
    d = device_case(c)
    logits = to_dev(c["logits"])
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    acc_ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    packed = dsv.pack_slots(d["k"], d["ctx_len"], d["kv_base"], d["block_tokens"], c["m_bs"], d["status"])
    out = torch.zeros_like(d["q"])
    lse = torch.zeros((c["m_bs"], c["hq"]), device=DEV)
    acc = {}

    def step():
        dsv.pack_slots(d["k"], d["ctx_len"], d["kv_base"], d["block_tokens"], c["m_bs"], d["status"], out=packed)
        a = dsv.attn_args(d["q"], d["k_pool"], d["v_pool"], packed["offsets"], d["k"], d["ctx_len"],
                          d["kv_base"], W=16, max_ctx=1300, out=out, status=d["status"], lse=lse,
                          k_new=d["k_new"], v_new=d["v_new"], slot_cache_loc=packed["slot_cache_loc"],
                          kv_chunk=256, workspace=ws)
        dsv.verify_attn_call(a)
        dsv.accept(n_bs=c["n_bs"], W=16, status=d["status"], target_logits=logits,
                   slot_tok=packed["slot_tok"], offsets=packed["offsets"], k=d["k"], out=acc, workspace=acc_ws)

    step()
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone(), {key: v.clone() for key, v in acc.items()})
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.zero_()
        lse.zero_()
        for v in acc.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[0].view(torch.int16)), f"replay {r}"
        assert torch.equal(lse, eager[1]), f"replay {r}"
        for key, v in acc.items():
            assert torch.equal(v, eager[2][key]), f"replay {r} {key}"
    assert int(d["status"].item()) == 0
    ref = oracle_pack(c)
    r_o, r_l = oracle_attn(c, ref["offsets"])
    compare_attn(c, ref["offsets"], out, lse, r_o, r_l, tag="graph")
