"""Helpers shared by the GPU parity tests: move seeded inputs to the device, run the HIP
path through the binding, and compare with the oracle under the parity rules.

Attention tolerances (bf16 inputs / fp32 inputs):
  * max |out - oracle| <= 1e-2 / 1e-4 (the stated parity bound) for outputs of magnitude
    <= 1; for larger outputs (the leak-detector variant scales V by 100) the bound scales with
    max |oracle|, since the output is rounded to the storage type;
  * per (request, head) relative L2 error <= 2e-2 / 1e-5, because near-uniform attention
    over thousands of keys gives outputs of size ~0.005 where 1e-2 alone says nothing;
  * |lse - oracle| <= 1e-3 / 1e-5.
The bf16 bound follows from the arithmetic: the output is rounded to bf16 (relative
2^-9 ~ 2e-3) and the probabilities are rounded to bf16 before the P V product (relative
2^-9 per term, averaging out over the keys); the fp32 bound from fp32 accumulation over at
most a few thousand terms (~1e-7 relative per term)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wl
import block_verification_attention_amd as dsv

DEV = "cuda"

TOL = {
    "bf16": dict(max_abs=1e-2, rel_l2=2e-2, lse=1e-3),
    "f32": dict(max_abs=1e-4, rel_l2=1e-5, lse=1e-5),
}


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_of(t):
    """bf16 tensor -> uint16 bit patterns (numpy)."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def oracle_pack(c):
    return oracle.pack(c["k"], c["ctx_len"], c["kv_base"], c["block_tokens"], c["W"], c["m_bs"])


def device_case(c):
    d = dict(
        k=to_dev(c["k"]), ctx_len=to_dev(c["ctx_len"]), kv_base=to_dev(c["kv_base"]),
        block_tokens=to_dev(c["block_tokens"]), k_pool=to_dev(c["k_pool"]),
        v_pool=to_dev(c["v_pool"]), q=to_dev(c["q"]), k_new=to_dev(c["k_new"]),
        v_new=to_dev(c["v_new"]), status=dsv.new_status(DEV),
    )
    return d


def gpu_pack(c, d):
    return dsv.pack_slots(d["k"], d["ctx_len"], d["kv_base"], d["block_tokens"], c["m_bs"], d["status"])


def gpu_attn(c, d, packed, *, use_new=True, kv_chunk=0, lse=True, out=None, k=None, offsets=None,
             max_ctx=None):
    lse_t = torch.full((c["m_bs"], c["hq"]), float("nan"), device=DEV) if lse else None
    if out is None:
        out = torch.full_like(d["q"], float("nan"))
    dsv.verify_attn(
        d["q"], d["k_pool"], d["v_pool"], packed["offsets"] if offsets is None else offsets,
        d["k"] if k is None else k, d["ctx_len"], d["kv_base"], W=c["W"],
        max_ctx=int(c["ctx_len"].max()) if max_ctx is None else max_ctx, status=d["status"],
        out=out, lse=lse_t, k_new=d["k_new"] if use_new else None,
        v_new=d["v_new"] if use_new else None,
        slot_cache_loc=packed["slot_cache_loc"] if use_new else None, kv_chunk=kv_chunk)
    return out, lse_t


def compare_attn(c, offsets, got_out, got_lse, ref_out, ref_lse, *, rows=None, tag=""):
    """Checks valid rows against the oracle (and tail rows against zero)."""
    tol = TOL[c["dtype"]]
    go = to_f64(got_out)
    gl = to_f64(got_lse) if got_lse is not None else None
    offsets = np.asarray(offsets)
    end = int(offsets[-1])
    worst = dict(max_abs=0.0, rel_l2=0.0, lse=0.0)
    for i in range(c["n_bs"]):
        kk = int(c["k"][i])
        if kk == 0:
            continue
        sl = slice(int(offsets[i]), int(offsets[i]) + kk)
        for h in range(c["hq"]):
            r = ref_out[sl, h]
            g = go[sl, h]
            if rows is not None:
                keep = rows[sl]
                if not keep.any():
                    continue
                r, g = r[keep], g[keep]
            err = np.abs(g - r)
            assert np.all(np.isfinite(g)), f"{tag} non-finite output request {i} head {h}"
            worst["max_abs"] = max(worst["max_abs"], float(err.max()))
            rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30))
            worst["rel_l2"] = max(worst["rel_l2"], rel)
            if gl is not None:
                lr = ref_lse[sl, h]
                lg_ = gl[sl, h]
                if rows is not None:
                    lr, lg_ = lr[keep], lg_[keep]
                worst["lse"] = max(worst["lse"], float(np.abs(lg_ - lr).max()))
    # outputs are rounded to the storage type, so the absolute bound scales with their size
    scale = max(1.0, float(np.abs(ref_out[:end][np.isfinite(ref_out[:end])]).max(initial=0.0)))
    bound = dict(tol, max_abs=tol["max_abs"] * scale)
    for key in worst:
        assert worst[key] <= bound[key], f"{tag}: {key} {worst[key]:.3e} > {bound[key]:.1e} ({worst})"
    if rows is None and end < c["m_bs"]:
        assert np.all(go[end:] == 0.0), f"{tag}: tail rows not zero"
        if gl is not None:
            assert np.all(np.isneginf(gl[end:])), f"{tag}: tail lse not -inf"
    return worst


def oracle_attn(c, offsets, use_new=True, slot_mask=None, k_pool=None, v_pool=None):
    return oracle.verify_attn(
        c["q"], c["k_pool"] if k_pool is None else k_pool, c["v_pool"] if v_pool is None else v_pool,
        offsets, c["k"], c["ctx_len"], c["kv_base"],
        k_new=c["k_new"] if use_new else None, v_new=c["v_new"] if use_new else None,
        slot_mask=slot_mask)


def small_case(seed, *, dtype="bf16", hq=8, hkv=2, d=128, k=(16, 5, 0, 11, 1, 16), ctx=None,
               extra_tail=4, qkv_scale=0.5, vocab=None):
    k = np.asarray(k, np.int32)
    if ctx is None:
        ctx = np.random.default_rng(seed).integers(0, 700, size=len(k)).astype(np.int32)
    return wl.make_case(seed, dtype=dtype, hq=hq, hkv=hkv, d=d, k=k, ctx_len=ctx,
                        m_bs=int(k.sum()) + extra_tail, qkv_scale=qkv_scale, vocab=vocab)
