"""Benchmark of the packed verification hot path on one MI355X.

A step is one pass of the hot path over the full-width verification workload (8 requests x
16 slots = 128 packed slots, 32 query / 8 KV heads, head_dim 128, context 8192, bf16;
target logits [128, 151936] fp32): dsv_pack_verify_attn (the packer fused into the
verification launch: offsets and slot fields, this step's candidate KV written at the packed
cache references, split-KV attention; then the merge) -> dsv_accept (per-slot argmax, longest
exact prefix, bonus token).  The same step with the packer as its own launch (dsv_pack_slots
-> dsv_verify_attn -> dsv_accept) is replayed beside it and reported as
`separate_pack_ms_per_step`.

Inputs are resident in HBM before timing.  To keep the 256 MiB Infinity Cache from serving
the KV stream, the step rotates over enough copies of the KV pool and logits to exceed 1 GB
(each copy holds the same seeded values).

Two timed passes over the same steps: (1) direct calls, with HIP events recorded by the
library around every verification-attention kernel on its launch stream; (2) the same steps
captured once each as HIP graphs and replayed (the library's calls allocate nothing, never
synchronise the host and record no memset, so a serving loop can replay them).

Prints one JSON line.  `value` is verified slots per second of the whole step (graph replay;
`--no-graph` reports the direct-call pass); `roofline` reports the verification-attention
kernel (the dominant one): algorithmic KV bytes per launch (every visible K and V row read
once) over its average duration from pass (1), against 8 TB/s and against the box's measured
streaming-read ceiling.  `cpu_baseline` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILED_KERNEL = "attn_bf16_kernel<128, 8, false, 64, 2, false>"
# HBM bytes per launch of that kernel on this workload, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs (profiles/attn_verify_cfg3_hbm_traffic.md, calibrated there against the
# streaming-read probe and a pool copy), valid for the kernel source with this SHA-256 only.
COUNTED_SOURCE = ("block_verification_attention_amd/csrc/dsv_attn.hip",
                  "e33a614536fe03d2c045884511b6ee94b89c5054c76af562c1448b7104bf82f8")
COUNTED_READ_BYTES = 270_444_171
COUNTED_WRITE_BYTES = 5_523_292


def counted_traffic():
    """HBM bytes per launch from the committed counter runs, or None once the kernel source
    has changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, COUNTED_SOURCE[0])
    try:
        with open(path, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    return COUNTED_READ_BYTES + COUNTED_WRITE_BYTES if digest == COUNTED_SOURCE[1] else None


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (timing on any stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def kv_bytes(ctx_len, k, hkv, d, elem=2):
    return int(sum((int(c) + int(kk)) * hkv * d * 2 * elem for c, kk in zip(ctx_len, k)))


def time_allocator(dev, iters: int = 50):
    """Latency of the budget allocator fused with the packer (dsv_allocate_pack) next to the
    plain packer, at the request counts of the 8-request and 60-request verification sets
    (W = 16, live budget 8 N in a bucket of 8 n_bs slots), with seeded synthetic scores.  Both
    are single-workgroup launches; reported as device microseconds per call, from HIP-graph
    replays of back-to-back calls timed with HIP events."""
    import numpy as np
    import torch
    import block_verification_attention_amd as dsv
    out = {}
    for n_live, n_bs in ((8, 8), (60, 64)):
        rng = np.random.default_rng(5000 + n_live)
        scores = torch.from_numpy(rng.random((n_bs, 15), dtype=np.float32)).to(dev)
        ctx = torch.from_numpy(rng.integers(0, 8192, n_bs).astype(np.int32)).to(dev)
        base = torch.from_numpy(np.arange(n_bs, dtype=np.int64) * 40000).to(dev)
        toks = torch.from_numpy(rng.integers(0, 150000, (n_bs, 16)).astype(np.int32)).to(dev)
        k = torch.from_numpy(np.minimum(rng.integers(1, 17, n_bs), 16).astype(np.int32)).to(dev)
        st = dsv.new_status(dev)
        alloc = dsv.allocate_pack(scores, n_live, 8 * n_live, ctx, base, toks, 8 * n_bs, st)
        packed = dsv.pack_slots(k, ctx, base, toks, 16 * n_bs, st)
        res = {}
        for name, fn in (("allocate_pack_us", lambda: dsv.allocate_pack(scores, n_live, 8 * n_live, ctx, base, toks,
                                                                        8 * n_bs, st, out=alloc)),
                         ("pack_only_us", lambda: dsv.pack_slots(k, ctx, base, toks, 16 * n_bs, st, out=packed))):
            # `iters` back-to-back calls captured in one HIP graph, so that the host's launch
            # latency does not separate them; device time per call
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(3):
                    fn()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for _ in range(iters):
                        fn()
            torch.cuda.current_stream().wait_stream(s)
            g.replay()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(5):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            res[name] = a.elapsed_time(b) * 1e3 / (5 * iters)
        res["budget_met"] = int(alloc["k"].sum().item()) == 8 * n_live
        out[f"n_live_{n_live}"] = res
    return out


def time_sampling(dev, copies: int, iters: int = 20):
    """Sampling-mode verifier (dsv_accept_sample) next to the greedy verifier (dsv_accept) on
    the full-width batch: 8 requests x 16 slots, target logits [128, 151936] fp32 at T = 1,
    drafts that are the target's likely picks (seeded synthetic logits, boosted so that about
    five drafts per request pass), seeded uniforms.  The logits are rotated over `copies`
    device copies so that the Infinity Cache cannot serve them between calls; device
    microseconds per call from HIP-graph replays of back-to-back calls, and the logits sweep
    rate that implies (one read of the 77.8 MB of logits per call)."""
    import numpy as np
    import torch
    import block_verification_attention_amd as dsv
    import workloads as wl
    g = np.random.default_rng(6000)
    n_bs, W, vocab = 8, 16, 151936
    k = np.full(n_bs, W, np.int32)
    bt = g.integers(0, vocab, (n_bs, W)).astype(np.int32)
    logits, bt = wl.sampling_logits(g, k, vocab, n_bs * W, bt, boost=(8.0, 12.0), p_random=0.05)
    slot_tok = torch.from_numpy(bt.reshape(-1)).to(dev)  # W slots per request: packed layout
    offsets = torch.from_numpy(np.arange(n_bs + 1, dtype=np.int32) * W).to(dev)
    kd = torch.from_numpy(k).to(dev)
    lg0 = torch.from_numpy(logits).to(dev)
    lgs = [lg0] + [lg0.clone() for _ in range(copies - 1)]
    u_acc = torch.from_numpy(wl.uniforms(g, n_bs * W)).to(dev)
    u_draw = torch.from_numpy(wl.uniforms(g, n_bs)).to(dev)
    st = dsv.new_status(dev)
    so = dsv.accept_sample(n_bs=n_bs, W=W, status=st, target_logits=lg0, temperature=1.0,
                           slot_tok=slot_tok, offsets=offsets, k=kd, u_accept=u_acc, u_draw=u_draw)
    sws = torch.empty(max(dsv.accept_sample_workspace_bytes(n_bs, n_bs * W, vocab), 256),
                      dtype=torch.uint8, device=dev)
    go = dsv.accept(n_bs=n_bs, W=W, status=st, target_logits=lg0, slot_tok=slot_tok,
                    offsets=offsets, k=kd)
    gws = torch.empty(max(dsv.accept_workspace_bytes(n_bs * W, vocab, 0, 0, 0), 256),
                      dtype=torch.uint8, device=dev)
    calls = {
        "sample_us": lambda j: dsv.accept_sample(
            n_bs=n_bs, W=W, status=st, target_logits=lgs[j % copies], temperature=1.0,
            slot_tok=slot_tok, offsets=offsets, k=kd, u_accept=u_acc, u_draw=u_draw, out=so,
            workspace=sws),
        "greedy_us": lambda j: dsv.accept(
            n_bs=n_bs, W=W, status=st, target_logits=lgs[j % copies], slot_tok=slot_tok,
            offsets=offsets, k=kd, out=go, workspace=gws),
    }
    res = {}
    for name, fn in calls.items():
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for j in range(3):
                fn(j)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s):
                for j in range(iters):
                    fn(j)
        torch.cuda.current_stream().wait_stream(s)
        gr.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / (5 * iters)
    res["sample_sweep_GBs"] = logits.nbytes / (res["sample_us"] * 1e-6) / 1e9
    res["mean_progress"] = float(so["progress"].float().mean().item())
    res["status"] = int(st.item())
    return res


def time_features(dev, copies: int = 2, iters: int = 10):
    """Draft confidence features (dsv_draft_features: top logit, gaps to ranks 2-16, top
    log-probability, entropy per draft position) on the drafter workload's logits: 32
    requests x 15 positions over a 248,320-token vocabulary, fp32 (476.8 MB), rotated over
    `copies` device copies; next to the top-1/top-2 margin sweep of dsv_accept on the same
    logits.  Device microseconds per call from HIP-graph replays of back-to-back calls, and
    the read rate that implies."""
    import numpy as np
    import torch
    import block_verification_attention_amd as dsv
    import workloads as wl
    x0 = torch.from_numpy(wl.draft_logits(4, 32, 248320)).to(dev)
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    st = dsv.new_status(dev)
    feat = dsv.draft_features(x0, st)
    fws = torch.empty(max(dsv.draft_features_workspace_bytes(32 * 15, 248320), 256),
                      dtype=torch.uint8, device=dev)
    mo = dsv.accept(n_bs=32, W=16, status=st, draft_logits=x0)
    mws = torch.empty(max(dsv.accept_workspace_bytes(0, 0, 32, 15, 248320), 256),
                      dtype=torch.uint8, device=dev)
    calls = {
        "features_us": lambda j: dsv.draft_features(xs[j % copies], st, out=feat, workspace=fws),
        "top2_margin_us": lambda j: dsv.accept(n_bs=32, W=16, status=st, draft_logits=xs[j % copies],
                                               out=mo, workspace=mws),
    }
    res = {}
    for name, fn in calls.items():
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for j in range(2):
                fn(j)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=s):
                for j in range(iters):
                    fn(j)
        torch.cuda.current_stream().wait_stream(s)
        gr.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / (5 * iters)
    nbytes = x0.numel() * 4
    res["features_GBs"] = nbytes / (res["features_us"] * 1e-6) / 1e9
    res["top2_margin_GBs"] = nbytes / (res["top2_margin_us"] * 1e-6) / 1e9
    res["status"] = int(st.item())
    return res


def time_prefill(dev, iters: int = 20, lens=(4096,) * 4, hq: int = 32, hkv: int = 8, seed: int = 5005,
                 d: int = 128):
    """Prefill attention with the 128-row wide tile (bf16 MFMA-bound).  Default: the
    mixed workload's prefill set, 4 fresh requests of 4096 causal rows (context 0), 32 query /
    8 KV heads, head_dim 128, seeded N(0,1) * 0.5 inputs made on the device.  Work per call:
    sum over rows of the visible keys x query heads x 128 x 4 flop (Q.K and P.V): 5.50e11 flop
    for the default set.  Device time per call from HIP events around each dsv_verify_attn call
    (prefill only, the pool already holding the rows' K/V), median of `iters`, against the
    dense bf16 MFMA peak of 2.5 PFLOP/s.  `lens`, `hq`, `hkv` and `d` give other sets (ragged
    lengths, fewer KV heads, head_dim 256)."""
    import numpy as np
    import torch
    import block_verification_attention_amd as dsv
    lens = [int(x) for x in lens]
    n_req = len(lens)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    rows = sum(lens)
    starts = np.cumsum([0] + lens[:-1]).tolist()
    kp = (torch.randn((hkv, rows, d), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    vp = (torch.randn((hkv, rows, d), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    q = (torch.randn((rows, hq, d), generator=g, device=dev) * 0.5).to(torch.bfloat16)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)  # noqa: E731
    pf = dsv.Prefill(q_start=i32(starts), q_len=i32(lens), ctx_len=i32([0] * n_req),
                     kv_base=torch.tensor(starts, dtype=torch.int64, device=dev),
                     q=q, out=torch.empty_like(q), max_len=max(lens),
                     lse=torch.empty((rows, hq), dtype=torch.float32, device=dev))
    st = dsv.new_status(dev)
    args = dsv.attn_args(None, kp, vp, None, None, None, None, W=16, max_ctx=0, out=None, status=st,
                         prefill=pf)
    for _ in range(3):
        dsv.verify_attn_call(args)
    evs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dsv.verify_attn_call(args)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
    flop = sum(4.0 * hq * d * n * (n + 1) / 2 for n in lens)
    tflops = flop / (us * 1e-6) / 1e12
    shape = (f"{n_req} x {lens[0]}" if len(set(lens)) == 1
             else "lengths " + ", ".join(str(n) for n in lens))
    return {"workload": f"prefill, {shape} causal rows, {hq}/{hkv} heads, head_dim {d}, bf16",
            "kernel": f"attn_bf16_kernel<{d}, 8, true, {64 if d == 64 else 32}, 1, false>", "us": us,
            "flop": flop,
            "TFLOPs": tflops, "peak_TFLOPs": 2500.0, "frac": tflops / 2500.0,
            "status": int(st.item())}


def time_mixed(dev, iters: int = 10):
    """The mixed launch (60 verification requests with ragged prefixes in 480 slots at
    contexts U[8192, 32768], plus 4 fresh prefill requests of 4096 causal rows; 32 / 8 heads,
    head_dim 128, bf16) as ONE dsv_verify_attn call, next to its two halves called alone on
    the same inputs: median of `iters` calls each, HIP events around each call.  K/V pool
    drawn on the device, N(0,1) * 0.5 (about 5 GB, far above the Infinity Cache)."""
    import numpy as np
    import torch
    import block_verification_attention_amd as dsv
    import workloads as wl
    c = wl.config5(draw=False)
    hq, hkv, d, W = c["hq"], c["hkv"], c["d"], c["W"]
    pf = c["prefill"]
    pf_rows = int(pf["q_len"].sum())
    g = torch.Generator(device=dev)
    g.manual_seed(5201)
    rnd = lambda shape: (torch.randn(shape, generator=g, device=dev) * 0.5).to(torch.bfloat16)  # noqa: E731
    kp, vp = rnd((hkv, c["pool_rows"], d)), rnd((hkv, c["pool_rows"], d))
    q, kn, vn, pq = rnd((c["m_bs"], hq, d)), rnd((c["m_bs"], hkv, d)), rnd((c["m_bs"], hkv, d)), rnd((pf_rows, hq, d))
    td = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    kd, cd, bd, tok = td(c["k"]), td(c["ctx_len"]), td(c["kv_base"]), td(c["block_tokens"])
    st = dsv.new_status(dev)
    packed = dsv.pack_slots(kd, cd, bd, tok, c["m_bs"], st)
    prefill = dsv.Prefill(q_start=td(pf["q_start"]), q_len=td(pf["q_len"]), ctx_len=td(pf["ctx_len"]),
                          kv_base=td(pf["kv_base"]), q=pq, out=torch.empty_like(pq), max_len=pf["max_len"],
                          lse=torch.empty((pf_rows, hq), dtype=torch.float32, device=dev))
    out = torch.empty_like(q)
    lse = torch.empty((c["m_bs"], hq), dtype=torch.float32, device=dev)
    max_ctx = int(c["ctx_len"].max())

    def make(verify, pre):
        if verify:
            a = dsv.attn_args(q, kp, vp, packed["offsets"], kd, cd, bd, W=W, max_ctx=max_ctx, out=out, status=st,
                              lse=lse, k_new=kn, v_new=vn, slot_cache_loc=packed["slot_cache_loc"],
                              prefill=prefill if pre else None)
        else:
            a = dsv.attn_args(None, kp, vp, None, None, None, None, W=W, max_ctx=0, out=None, status=st,
                              prefill=prefill)
        return a

    res = {}
    for name, a in (("mixed_us", make(True, True)), ("verify_only_us", make(True, False)),
                    ("prefill_only_us", make(False, True))):
        ws = torch.empty(max(dsv.verify_attn_workspace_bytes(a), 256), dtype=torch.uint8, device=dev)
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        for _ in range(2):
            dsv.verify_attn_call(a)
        evs = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dsv.verify_attn_call(a)
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        res[name] = float(np.median([x.elapsed_time(y) for x, y in evs])) * 1e3
        del ws
    res["mixed_over_sum_of_halves"] = res["mixed_us"] / (res["verify_only_us"] + res["prefill_only_us"])
    res["slots"] = int(c["k"].sum())
    res["prefill_rows"] = pf_rows
    res["status"] = int(st.item())
    del kp, vp
    torch.cuda.empty_cache()
    return res


def time_other_verify(dev, ev, iters: int = 20):
    """Verification attention on the two other verification shapes of the configuration set,
    with their seeded prefix lengths and contexts and seeded N(0,1) * 0.5 device-made K/V:
    32 requests sharing 256 slots at contexts U[4096, 8192], 24 query / 2 KV heads, head_dim
    256 (12 query heads per KV head); and 60 requests sharing 480 slots at contexts
    U[8192, 32768], 32 / 8 heads, head_dim 128.  Also the first shape's requests with 8 query
    heads on 8 KV heads (one per KV head, head_dim 256) and with 64 query heads on 8 KV heads
    (eight per KV head, head_dim 128).  Kernel time from the start/stop events
    attached to the verification kernel's launch (median of `iters`), algorithmic KV bytes
    (every visible K and V row once) over it, against 8 TB/s."""
    import numpy as np
    import torch
    import block_verification_attention_amd as dsv
    import workloads as wl
    out = {}
    shapes = {
        "32x256_slots_ctx4k-8k_24q2kv_d256": (4, 32, 256, 4096, 8193, 24, 2, 256, 2),
        "60x480_slots_ctx8k-32k_32q8kv_d128": (5, 60, 480, 8192, 32769, 32, 8, 128, 1),
        "32x256_slots_ctx4k-8k_8q8kv_d256": (4, 32, 256, 4096, 8193, 8, 8, 256, 1),
        "32x256_slots_ctx4k-8k_64q8kv_d128": (4, 32, 256, 4096, 8193, 64, 8, 128, 1),
    }
    for name, (cfg, n, m_bs, lo, hi, hq, hkv, d, copies) in shapes.items():
        g = wl.rng(cfg, 0)
        k = wl.lengths_geometric_rescaled(g, n, m_bs)
        ctx = g.integers(lo, hi, size=n).astype(np.int32)
        seg = (ctx + 16).astype(np.int64)
        base = np.concatenate([[0], np.cumsum(seg)[:-1]]).astype(np.int64)
        rows = int(seg.sum())
        tg = torch.Generator(device=dev)
        tg.manual_seed(7000 + cfg)
        pools = [((torch.randn((hkv, rows, d), generator=tg, device=dev) * 0.5).to(torch.bfloat16),
                  (torch.randn((hkv, rows, d), generator=tg, device=dev) * 0.5).to(torch.bfloat16))
                 for _ in range(copies)]
        q = (torch.randn((m_bs, hq, d), generator=tg, device=dev) * 0.5).to(torch.bfloat16)
        kn = (torch.randn((m_bs, hkv, d), generator=tg, device=dev) * 0.5).to(torch.bfloat16)
        vn = (torch.randn((m_bs, hkv, d), generator=tg, device=dev) * 0.5).to(torch.bfloat16)
        kd, cd, bd = (torch.from_numpy(a).to(dev) for a in (k, ctx, base))
        tok = torch.zeros((n, 16), dtype=torch.int32, device=dev)
        st = dsv.new_status(dev)
        packed = dsv.pack_slots(kd, cd, bd, tok, m_bs, st)
        o = torch.empty_like(q)
        lse = torch.empty((m_bs, hq), dtype=torch.float32, device=dev)
        evs = ev.create(2 * iters)
        args = [dsv.attn_args(q, *pools[j % copies], packed["offsets"], kd, cd, bd, W=16,
                              max_ctx=int(ctx.max()), out=o, status=st, lse=lse, k_new=kn, v_new=vn,
                              slot_cache_loc=packed["slot_cache_loc"],
                              events=(evs[2 * j].value, evs[2 * j + 1].value)) for j in range(iters)]
        ws = torch.empty(max(dsv.verify_attn_workspace_bytes(args[0]), 256), dtype=torch.uint8, device=dev)
        for a in args:
            a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        for j in range(3):
            dsv.verify_attn_call(args[j])
        torch.cuda.synchronize()
        for a in args:
            dsv.verify_attn_call(a)
        torch.cuda.synchronize()
        us = float(np.median([ev.elapsed_ms(evs[2 * j], evs[2 * j + 1]) for j in range(iters)])) * 1e3
        ev.destroy(evs)
        kvb = int(((ctx.astype(np.int64) + k) * hkv * d * 2 * 2).sum())
        out[name] = {"kernel_us": us, "algorithmic_bytes": kvb, "GBs": kvb / (us * 1e-6) / 1e9,
                     "frac": kvb / (us * 1e-6) / 8e12, "slots": int(k.sum()), "status": int(st.item())}
        del pools, args
        torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    """The host CPU's model name (first processor of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, n_req_sample: int, min_seconds: float = 10.0, max_reps: int = 40,
                 threads: int = 0):
    """The oracle (pack + fp64 attention + greedy accept) on the first n_req_sample requests,
    repeated until at least min_seconds of CPU work have run (at most max_reps passes); the
    rate is slots over the mean time of a pass.  threads > 0 runs the oracle on that many
    threads (else its default: every core OpenMP offers)."""
    import numpy as np

    import oracle

    default_threads = oracle.threads()
    if threads > 0:
        oracle.set_threads(threads)
    try:
        return _cpu_baseline(case, n_req_sample, min_seconds, max_reps)
    finally:
        oracle.set_threads(default_threads)


def _cpu_baseline(case, n_req_sample, min_seconds, max_reps):
    import oracle

    c = case
    sel = slice(0, n_req_sample)
    k = c["k"][sel]
    ctx = c["ctx_len"][sel]
    base = c["kv_base"][sel]
    tok = c["block_tokens"][sel]
    m = int(k.sum())
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        p = oracle.pack(k, ctx, base, tok, c["W"], m)
        oracle.verify_attn(c["q"][:m], c["k_pool"], c["v_pool"], p["offsets"], k, ctx, base,
                           c["k_new"][:m], c["v_new"][:m])
        oracle.accept(c["logits"][:m], p["slot_tok"], p["offsets"], k, c["W"])
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    threads = min(oracle.threads(), n_req_sample * c["hkv"])
    return {
        "value": m / dt,
        "unit": "slots/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_req_sample} of {c['n_bs']} requests ({m} slots), full context, fp64 "
                  f"attention over (request, KV head) units on {threads} threads; {reps} passes, "
                  f"{total:.1f} s in all, {dt:.2f} s per pass",
        "cpu_model": cpu_model(),
        "host_threads": os.cpu_count(),
    }


def cpu_configs(dev):
    """The oracle on every configuration of the workload set, on one host thread and on every
    host thread: pack + fp64 verification attention (+ greedy accept over the target logits,
    or the draft top-1/top-2 margin), computed in full for configs 1-4; for config 5 all 480
    verification slots plus 512 prefill rows of each of its 4 requests (the first 64, the last
    64 and 384 seeded ones between them).  Wall time is the best of 3 passes, or one pass when
    it exceeds 10 s.  Config 5's pool (~5 GB) is drawn on the device and copied to the host."""
    import numpy as np
    import torch

    import oracle
    import workloads as wl

    def best_of(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
            if ts[-1] > 10.0:
                break
        return min(ts), len(ts)

    def verify_pass(c):
        p = oracle.pack(c["k"], c["ctx_len"], c["kv_base"], c["block_tokens"], c["W"], c["m_bs"])
        oracle.verify_attn(c["q"], c["k_pool"], c["v_pool"], p["offsets"], c["k"], c["ctx_len"], c["kv_base"],
                           c["k_new"], c["v_new"])
        return p

    cases = {}
    def verify_accept(*steps):
        for c in steps:
            p = verify_pass(c)
            oracle.accept(c["logits"], p["slot_tok"], p["offsets"], c["k"], c["W"])

    c1 = wl.config1()
    cases["1"] = (int(c1["k"].sum()), lambda: verify_accept(c1))
    s1, s2 = wl.config2()
    cases["2"] = (int(s1["k"].sum() + s2["k"].sum()), lambda: verify_accept(s1, s2))
    c3 = wl.config3()
    cases["3"] = (int(c3["k"].sum()), lambda: verify_accept(c3))
    c4 = wl.config4()

    def cfg4():
        verify_pass(c4)
        oracle.top2_margin(c4["draft_logits"])
    cases["4"] = (int(c4["k"].sum()), cfg4)
    # config 5: pool, queries and candidates drawn on the device, then copied to the host
    c5 = wl.config5(draw=False)
    g = torch.Generator(device=dev)
    g.manual_seed(5301)
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    rnd = lambda shape: bits((torch.randn(shape, generator=g, device=dev) * 0.5).to(torch.bfloat16))  # noqa: E731
    hkv, hq, d = c5["hkv"], c5["hq"], c5["d"]
    pf = c5["prefill"]
    pf_rows = int(pf["q_len"].sum())
    c5 = dict(c5, k_pool=rnd((hkv, c5["pool_rows"], d)), v_pool=rnd((hkv, c5["pool_rows"], d)),
              q=rnd((c5["m_bs"], hq, d)), k_new=rnd((c5["m_bs"], hkv, d)), v_new=rnd((c5["m_bs"], hkv, d)))
    pq = rnd((pf_rows, hq, d))
    sel = np.random.default_rng(5110)
    sel_req, sel_j = [], []
    for r in range(pf["n_pf"]):
        ql = int(pf["q_len"][r])
        js = sorted(set(range(64)) | set(range(ql - 64, ql)) |
                    set(sel.choice(np.arange(64, ql - 64), 384, replace=False).tolist()))
        sel_req += [r] * len(js)
        sel_j += js

    def cfg5():
        verify_pass(c5)
        oracle.prefill_attn(pq, c5["k_pool"], c5["v_pool"], pf["q_start"], pf["q_len"], pf["ctx_len"],
                            pf["kv_base"], sel_req, sel_j)
    cases["5"] = (int(c5["k"].sum()), cfg5)

    nproc = os.cpu_count() or 1
    default_threads = oracle.threads()
    out = {}
    try:
        for name, (slots, fn) in cases.items():
            row = {"slots": slots}
            for th in (1, default_threads):
                oracle.set_threads(th)
                sec, passes = best_of(fn)
                row[f"threads_{th}"] = {"seconds": sec, "slots_per_s": slots / sec, "passes": passes}
                print(f"cpu config {name} threads {th}: {sec:.3f} s", file=sys.stderr, flush=True)
            out[name] = row
    finally:
        oracle.set_threads(default_threads)
    out["5"]["sample"] = "all 480 verification slots + 512 prefill rows per request (first 64, last 64, 384 seeded)"
    return {"cpu_configs": out, "cpu_model": cpu_model(), "nproc": nproc, "oracle_threads": default_threads}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=4, help="KV/logits copies rotated per step")
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=8, help="requests in the oracle sample (0 = skip)")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="only time the CPU oracle on every configuration (1 and all host threads)")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="launch each step's calls directly instead of replaying a captured HIP graph")
    ap.add_argument("--only", choices=["prefill", "other_verify"], default=None,
                    help="only run that section, `--steps` times, and print its JSON (for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "dsv runs on one GPU: splitting a step over several GPUs "
                                   "is not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import block_verification_attention_amd as dsv
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.cpu_configs:
        print(json.dumps(cpu_configs(dev)))
        return
    dsv.load_library()
    if args.only == "prefill":
        print(json.dumps(time_prefill(dev, iters=args.steps)))
        return
    if args.only == "other_verify":
        print(json.dumps(time_other_verify(dev, HipEvents(), iters=args.steps)))
        return
    c = wl.config3()

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    k = to_dev(c["k"])
    ctx = to_dev(c["ctx_len"])
    base = to_dev(c["kv_base"])
    tok = to_dev(c["block_tokens"])
    q = to_dev(c["q"])
    k_new = to_dev(c["k_new"])
    v_new = to_dev(c["v_new"])
    kp0, vp0, lg0 = to_dev(c["k_pool"]), to_dev(c["v_pool"]), to_dev(c["logits"])
    pools = [(kp0, vp0, lg0)] + [(kp0.clone(), vp0.clone(), lg0.clone()) for _ in range(args.copies - 1)]
    status = dsv.new_status(dev)
    m_bs, W = c["m_bs"], c["W"]
    packed = dsv.pack_slots(k, ctx, base, tok, m_bs, status)  # allocates fixed-address outputs
    out = torch.empty_like(q)
    lse = torch.empty((m_bs, c["hq"]), dtype=torch.float32, device=dev)
    acc_out = {}
    ev = HipEvents()
    n_total = args.warmup + args.steps
    main_ev = ev.create(2 * n_total)
    max_ctx = int(c["ctx_len"].max())

    def make_args(s, events):
        kp, vp, _ = pools[s % len(pools)]
        return dsv.attn_args(q, kp, vp, packed["offsets"], k, ctx, base, W=W, max_ctx=max_ctx,
                             out=out, status=status, lse=lse, k_new=k_new, v_new=v_new,
                             slot_cache_loc=packed["slot_cache_loc"], kv_chunk=args.kv_chunk,
                             events=events)

    timed_args = [make_args(s, (main_ev[2 * s].value, main_ev[2 * s + 1].value)) for s in range(n_total)]
    plain_args = [make_args(s, None) for s in range(n_total)]
    ws_bytes = dsv.verify_attn_workspace_bytes(timed_args[0])
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    for a in timed_args + plain_args:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
    acc_ws = torch.empty(max(dsv.accept_workspace_bytes(m_bs, c["logits"].shape[1], 0, 0, 0), 256),
                         dtype=torch.uint8, device=dev)

    def step(s, arg_list):
        dsv.pack_verify_attn(arg_list[s], tok, out=packed)
        dsv.accept(n_bs=c["n_bs"], W=W, status=status, target_logits=pools[s % len(pools)][2],
                   slot_tok=packed["slot_tok"], offsets=packed["offsets"], k=k, out=acc_out,
                   workspace=acc_ws)

    def step_separate_pack(s, arg_list):
        dsv.pack_slots(k, ctx, base, tok, m_bs, status, out=packed)
        dsv.verify_attn_call(arg_list[s])
        dsv.accept(n_bs=c["n_bs"], W=W, status=status, target_logits=pools[s % len(pools)][2],
                   slot_tok=packed["slot_tok"], offsets=packed["offsets"], k=k, out=acc_out,
                   workspace=acc_ws)

    def timed(fn):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    for s in range(args.warmup):
        step(s, plain_args)
    # timed region 1: direct calls, HIP events around every verification-attention kernel
    direct_ms = timed(lambda: [step(s, timed_args) for s in range(args.warmup, n_total)])
    total_ms = direct_ms
    if args.graph:
        # one captured step per timed step (each with its own KV copy); the library makes no
        # allocation, host synchronisation or memset inside its calls
        graphs = []
        for s in range(args.warmup, n_total):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(s, plain_args)
            graphs.append(g)
        graphs[0].replay()
        # timed region 2: the same steps replayed as HIP graphs
        total_ms = timed(lambda: [g.replay() for g in graphs])
        # the step with the packer as its own launch, for comparison (not the reported value)
        sep_graphs = []
        for s in range(args.warmup, n_total):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_separate_pack(s, plain_args)
            sep_graphs.append(g)
        sep_graphs[0].replay()
        sep_ms = timed(lambda: [g.replay() for g in sep_graphs])
        del sep_graphs
    st = int(status.item())
    if st != 0:
        print(json.dumps({"error": f"device status {st}"}))
        sys.exit(1)
    # sanity: the planted acceptance came out
    if not np.array_equal(acc_out["accepted"].cpu().numpy(), c["planted_accepted"]):
        print(json.dumps({"error": "accepted lengths differ from the planted ones"}))
        sys.exit(1)
    # the whole calls, by events recorded on the stream around each of back-to-back direct
    # calls: dsv_verify_attn (attention kernel + split merge) and dsv_pack_verify_attn (the
    # packer fused into it), with no kernel events attached
    def time_calls(fn):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(n_total)]
        torch.cuda.synchronize()
        for s in range(n_total):
            pairs[s][0].record()
            fn(s)
            pairs[s][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in pairs[args.warmup:]]))
    call_ms = time_calls(lambda s: dsv.verify_attn_call(plain_args[s]))
    fused_call_ms = time_calls(lambda s: dsv.pack_verify_attn(plain_args[s], tok, out=packed))
    attn_ms = [ev.elapsed_ms(main_ev[2 * s], main_ev[2 * s + 1]) for s in range(args.warmup, n_total)]
    ev.destroy(main_ev)
    attn_avg_ms = float(np.mean(attn_ms))
    slots = int(c["k"].sum())
    ms_per_step = total_ms / args.steps
    kvb = kv_bytes(c["ctx_len"], c["k"], c["hkv"], c["d"])
    achieved = kvb / (attn_avg_ms * 1e-3) / 1e9
    res = {
        "metric": "verified candidate slots/sec at fixed context; % of MI355X HBM peak (KV read)",
        "value": slots / (ms_per_step * 1e-3),
        "unit": "slots/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; KV/logits rotated over %d copies, %.2f GB)" % (
            len(pools), len(pools) * (2 * kp0.numel() * 2 + lg0.numel() * 4) / 1e9),
        "config": {
            "workload": "full-width verify: 8 requests x 16 slots (128 packed), 32 query / 8 KV "
                        "heads, head_dim 128, context 8192, bf16; fp32 logits [128, 151936]",
            "n_requests": 8, "slots": slots, "context": 8192, "hq": 32, "hkv": 8, "head_dim": 128,
            "vocab": 151936, "step": "pack fused into verify attention (incl. candidate KV write, "
                                      "split-KV merge) + accept",
            "launch": "HIP graph per step" if args.graph else "direct calls",
        },
        "roofline": {
            "kernel": PROFILED_KERNEL,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": counted_traffic(),
            "algorithmic_bytes": kvb,
            "avg_launch_us": attn_avg_ms * 1e3,
            # the dsv_verify_attn call (attention + split merge) and the fused packer call
            "call_us": call_ms * 1e3,
            "call_frac": kvb / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "fused_call_us": fused_call_ms * 1e3,
            "fused_call_frac": kvb / (fused_call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "attn_kernel_slots_per_s": slots / (attn_avg_ms * 1e-3),
        "direct_call_ms_per_step": direct_ms / args.steps,
    }
    if args.graph:
        res["separate_pack_ms_per_step"] = sep_ms / args.steps
    # practical read ceiling of this machine: a plain streaming read of the same KV bytes
    lib = dsv._lib.load()
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    probe_ms = []  # per step: the K pool and the V pool read, each timed on its own
    for s in range(3 + args.steps):
        kp, vp, _ = pools[s % len(pools)]
        pair = []
        for t in (kp, vp):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dsv._lib.check(lib.dsv_probe_stream_read(ctypes.c_void_p(t.data_ptr()), t.numel() * 2,
                                                     ctypes.c_void_p(sink.data_ptr()), stream),
                           "dsv_probe_stream_read")
            e1.record()
            pair.append((e0, e1))
        probe_ms.append(pair)
    torch.cuda.synchronize()
    probe_avg = float(np.mean([sum(a.elapsed_time(b) for a, b in pair) for pair in probe_ms[3:]]))
    pool_bytes = 2 * kp0.numel() * 2
    res["roofline"]["stream_read_ceiling_GBs"] = pool_bytes / (probe_avg * 1e-3) / 1e9
    res["roofline"]["frac_of_ceiling"] = achieved / res["roofline"]["stream_read_ceiling_GBs"]
    # token-granular cache map (kv_index): the same launch with every K/V row read through a
    # per-position row table -- the identity map, and rows scattered over the whole pool (a
    # random permutation, so every pool row is still read once)
    def time_mapped(idx_t):
        evs = ev.create(2 * n_total)
        margs = [make_args(s, (evs[2 * s].value, evs[2 * s + 1].value)) for s in range(n_total)]
        for a in margs:
            a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
            a.kv_index, a.kv_index_stride = idx_t.data_ptr(), idx_t.shape[1]
        for s in range(n_total):
            dsv.verify_attn_call(margs[s])
        torch.cuda.synchronize()
        t = float(np.mean([ev.elapsed_ms(evs[2 * s], evs[2 * s + 1]) for s in range(args.warmup, n_total)]))
        ev.destroy(evs)
        return t * 1e3
    stride_map = int((c["ctx_len"] + c["k"]).max())
    pos = np.arange(stride_map, dtype=np.int64)[None, :]
    ident = (c["kv_base"][:, None] + pos).astype(np.int64)
    rows = c["k_pool"].shape[1]
    perm = np.random.default_rng(77).permutation(rows)
    maps = {"identity": np.minimum(ident, rows - 1), "scattered": perm[np.minimum(ident, rows - 1)]}
    res["cache_map"] = {"contiguous_us": attn_avg_ms * 1e3}
    for name, m in maps.items():
        res["cache_map"][f"{name}_us"] = time_mapped(torch.from_numpy(m.astype(np.int32)).to(dev))
    res["cache_map"]["scattered_GBs"] = kvb / (res["cache_map"]["scattered_us"] * 1e-6) / 1e9
    res["allocator"] = time_allocator(dev)
    res["sampling"] = time_sampling(dev, args.copies)
    res["features"] = time_features(dev)
    res["prefill"] = time_prefill(dev)
    # ragged lengths with 2 KV heads (8 query heads each): the row blocks of a request are
    # spread over the XCDs by the launch's block order
    res["prefill_ragged"] = time_prefill(dev, lens=(4096, 1024, 1024, 1024), hq=16, hkv=2, seed=5006)
    # head_dim 256 (16 query / 8 KV heads)
    res["prefill_d256"] = time_prefill(dev, hq=16, hkv=8, seed=5007, d=256)
    # head_dim 64 (32 query / 8 KV heads)
    res["prefill_d64"] = time_prefill(dev, hq=32, hkv=8, seed=5008, d=64)
    res["other_verify"] = time_other_verify(dev, ev)
    res["mixed_launch"] = time_mixed(dev)
    if args.cpu_sample > 0:
        res["cpu_baseline"] = cpu_baseline(c, args.cpu_sample)
        # the same oracle on one thread, over one request (16 slots)
        one = cpu_baseline(c, 1, min_seconds=5.0, threads=1)
        res["cpu_baseline"]["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
