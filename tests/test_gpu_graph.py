"""HIP-graph capture of the calls beyond the greedy step: budget allocator + pack, verification
attention through a cache map, a head_dim-256 launch with head groups (one wave per head),
the sampling-mode verifier on uniforms drawn in the graph by the counter-based generator, and
the draft confidence features.  One captured graph holds all
of them; three replays, with eager work and synchronisation between them, reproduce the eager
outputs bit for bit."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as wl  # noqa: E402
from gpu_util import DEV, device_case, gpu_pack, small_case, to_dev  # noqa: E402
import block_verification_attention_amd as dsv  # noqa: E402


def test_next_rows_graph_capture_replays_match_eager():
    g = np.random.default_rng(90)
    st = dsv.new_status(DEV)
    # budget allocator fused with the packer
    n_bs = 12
    scores = to_dev(g.random((n_bs, 15), dtype=np.float32))
    actx = to_dev(g.integers(0, 500, n_bs).astype(np.int32))
    abase = to_dev((np.arange(n_bs) * 600).astype(np.int64))
    atok = to_dev(g.integers(0, 1000, (n_bs, 16)).astype(np.int32))
    alloc = dsv.allocate_pack(scores, 10, 80, actx, abase, atok, 96, st)
    # cache-map verification (identity map over contiguous segments)
    c = small_case(91, hq=8, hkv=2, d=128, k=(16, 9, 1, 12), ctx=(700, 1300, 5, 260))
    d = device_case(c)
    packed = gpu_pack(c, d)
    stride = int((c["ctx_len"] + c["k"]).max())
    idx = np.minimum(c["kv_base"][:, None] + np.arange(stride)[None, :], c["k_pool"].shape[1] - 1)
    kv_index = to_dev(idx.astype(np.int32))
    out = torch.zeros_like(d["q"])
    lse = torch.zeros((c["m_bs"], c["hq"]), device=DEV)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    # head_dim 256, 6 query heads per KV head (head groups of 3, one wave per head)
    c2 = small_case(92, hq=12, hkv=2, d=256, k=(16, 3, 9), ctx=(900, 40, 2100))
    d2 = device_case(c2)
    packed2 = gpu_pack(c2, d2)
    out2 = torch.zeros_like(d2["q"])
    lse2 = torch.zeros((c2["m_bs"], c2["hq"]), device=DEV)
    ws2 = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    # sampling-mode verifier
    sk = np.array([16, 5, 0, 11], np.int32)
    slog, sbt = wl.sampling_logits(g, sk, 3000, int(sk.sum()) + 2, g.integers(0, 3000, (4, 16)).astype(np.int32),
                                   boost=(0.0, 8.0))
    sp = dsv.pack_slots(to_dev(sk), to_dev(np.zeros(4, np.int32)), to_dev(np.zeros(4, np.int64)),
                        to_dev(sbt), int(sk.sum()) + 2, st)
    slogits = to_dev(slog)
    u_acc = torch.empty(slog.shape[0], dtype=torch.float32, device=DEV)
    u_draw = torch.empty(4, dtype=torch.float32, device=DEV)
    skd = to_dev(sk)
    sws = torch.zeros(dsv.accept_sample_workspace_bytes(4, slog.shape[0], 3000), dtype=torch.uint8, device=DEV)
    sout = {}
    # draft features
    dl = to_dev(g.standard_normal((3, 15, 4096), dtype=np.float32))
    fout = torch.zeros((3, 15, 18), dtype=torch.float32, device=DEV)
    fws = torch.zeros(dsv.draft_features_workspace_bytes(45, 4096), dtype=torch.uint8, device=DEV)

    def calls():
        dsv.allocate_pack(scores, 10, 80, actx, abase, atok, 96, st, out=alloc)
        a = dsv.attn_args(d["q"], d["k_pool"], d["v_pool"], packed["offsets"], d["k"], d["ctx_len"],
                          d["kv_base"], W=16, max_ctx=1300, out=out, status=st, lse=lse,
                          k_new=d["k_new"], v_new=d["v_new"], slot_cache_loc=packed["slot_cache_loc"],
                          workspace=ws, kv_index=kv_index)
        dsv.verify_attn_call(a)
        a2 = dsv.attn_args(d2["q"], d2["k_pool"], d2["v_pool"], packed2["offsets"], d2["k"], d2["ctx_len"],
                           d2["kv_base"], W=16, max_ctx=2100, out=out2, status=st, lse=lse2,
                           k_new=d2["k_new"], v_new=d2["v_new"], slot_cache_loc=packed2["slot_cache_loc"],
                           kv_chunk=256, workspace=ws2)
        dsv.verify_attn_call(a2)
        dsv.philox_uniforms(0xABC, 0, slog.shape[0], out=u_acc)
        dsv.philox_uniforms(0xABC, (slog.shape[0] + 3) // 4, 4, out=u_draw)
        dsv.accept_sample(n_bs=4, W=16, status=st, target_logits=slogits, temperature=0.8,
                          slot_tok=sp["slot_tok"], offsets=sp["offsets"], k=skd, u_accept=u_acc,
                          u_draw=u_draw, out=sout, workspace=sws)
        dsv.draft_features(dl, st, out=fout, workspace=fws)

    calls()
    torch.cuda.synchronize()
    results = lambda: [alloc[k] for k in sorted(alloc)] + [out, lse, out2, lse2] + \
        [u_acc, u_draw] + [sout[k] for k in sorted(sout)] + [fout]  # noqa: E731
    eager = [t.clone() for t in results()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for r in range(3):
        for t in results():
            if t.dtype in (torch.float32, torch.bfloat16):
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (t, e) in enumerate(zip(results(), eager)):
            if t.dtype == torch.bfloat16:
                ok = torch.equal(t.view(torch.int16), e.view(torch.int16))
            elif t.dtype == torch.float32:
                ok = torch.equal(t.view(torch.int32), e.view(torch.int32))
            else:
                ok = torch.equal(t, e)
            assert ok, f"replay {r}, output {j}"
    assert int(st.item()) == 0


def test_mixed_and_noalloc_graph_capture_replays_match_eager():
    """The mixed call (a prefill set beside the verification set in one dsv_verify_attn) and
    the no-allocation entry point (split partials in the library's scratch array, the call
    meant for code under capture), captured in one graph: three replays, with eager work and
    synchronisation between them, reproduce the eager outputs bit for bit."""
    st = dsv.new_status(DEV)
    c = wl.make_mixed_case(95, hq=8, hkv=2, d=128, k=[3, 16], ctx_len=[40, 1300], m_bs=20,
                           pf_q_len=[300, 77], pf_ctx=[0, 33])
    d = device_case(c)
    packed = gpu_pack(c, d)
    pf = c["prefill"]
    pf_q = to_dev(pf["q"])
    prefill = dsv.Prefill(q_start=to_dev(pf["q_start"]), q_len=to_dev(pf["q_len"]),
                          ctx_len=to_dev(pf["ctx_len"]), kv_base=to_dev(pf["kv_base"]), q=pf_q,
                          out=torch.zeros_like(pf_q), max_len=pf["max_len"],
                          lse=torch.zeros((pf_q.shape[0], c["hq"]), device=DEV))
    out = torch.zeros_like(d["q"])
    lse = torch.zeros((c["m_bs"], c["hq"]), device=DEV)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    c2 = small_case(96, hq=12, hkv=4, d=128, k=(16, 9, 1, 12), ctx=(2000, 700, 5, 1300))
    d2 = device_case(c2)
    packed2 = gpu_pack(c2, d2)
    out2 = torch.zeros_like(d2["q"])
    lse2 = torch.zeros((c2["m_bs"], c2["hq"]), device=DEV)

    def calls():
        a = dsv.attn_args(d["q"], d["k_pool"], d["v_pool"], packed["offsets"], d["k"], d["ctx_len"],
                          d["kv_base"], W=16, max_ctx=1300, out=out, status=st, lse=lse,
                          k_new=d["k_new"], v_new=d["v_new"], slot_cache_loc=packed["slot_cache_loc"],
                          kv_chunk=256, workspace=ws, prefill=prefill)
        dsv.verify_attn_call(a)
        a2 = dsv.attn_args(d2["q"], d2["k_pool"], d2["v_pool"], packed2["offsets"], d2["k"],
                           d2["ctx_len"], d2["kv_base"], W=16, max_ctx=2000, out=out2, status=st,
                           lse=lse2, k_new=d2["k_new"], v_new=d2["v_new"],
                           slot_cache_loc=packed2["slot_cache_loc"], kv_chunk=256)
        dsv.verify_attn_noalloc_call(a2)

    calls()
    torch.cuda.synchronize()
    results = lambda: [out, lse, prefill.out, prefill.lse, out2, lse2]  # noqa: E731
    eager = [t.clone() for t in results()]
    # outputs finite (tail rows zero-filled); lse of the tail rows is -inf by definition
    assert all(bool(torch.isfinite(eager[j].float()).all()) for j in (0, 2, 3, 4))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for r in range(3):
        for t in results():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j, (t, e) in enumerate(zip(results(), eager)):
            bits = torch.int16 if t.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(t.view(bits), e.view(bits)), f"replay {r}, output {j}"
    assert int(st.item()) == 0
