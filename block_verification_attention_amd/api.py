"""Thin PyTorch-facing binding of libdsv: argument marshalling only.

Every step runs in the HIP kernels of libdsv.so; PyTorch provides device memory and the
stream.  Names follow the C ABI (include/dsv.h): pack_slots, allocate_pack, verify_attn,
accept, accept_sample, draft_features, philox_uniforms.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import AttnArgs, check


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, device):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def new_status(device) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device)


# ---------------------------------------------------------------------------
# dsv_pack_slots
# ---------------------------------------------------------------------------
def pack_slots(k, ctx_len, kv_base, block_tokens, m_bs: int, status, out=None, stream=None) -> dict:
    """Packs per-request prefixes into m_bs slots.  Returns offsets, slot_req, slot_tok,
    slot_pos, slot_cache_loc (device tensors; `out` may supply them for fixed addresses)."""
    lib = _lib.load()
    dev = k.device
    n_bs, W = block_tokens.shape
    for t, dt, nm in ((k, torch.int32, "k"), (ctx_len, torch.int32, "ctx_len"),
                      (kv_base, torch.int64, "kv_base"), (block_tokens, torch.int32, "block_tokens")):
        _need(t, dt, nm, dev)
    if out is None:
        out = dict(
            offsets=torch.empty(n_bs + 1, dtype=torch.int32, device=dev),
            slot_req=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_tok=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_pos=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_cache_loc=torch.empty(m_bs, dtype=torch.int64, device=dev),
        )
    check(lib.dsv_pack_slots(n_bs, W, m_bs, _ptr(k), _ptr(ctx_len), _ptr(kv_base), _ptr(block_tokens),
                             _ptr(out["offsets"]), _ptr(out["slot_req"]), _ptr(out["slot_tok"]),
                             _ptr(out["slot_pos"]), _ptr(out["slot_cache_loc"]), _ptr(status),
                             _stream(stream)), "dsv_pack_slots")
    return out


def allocate_pack(scores, n_live: int, m_live: int, ctx_len, kv_base, block_tokens, m_bs: int, status,
                  out=None, stream=None) -> dict:
    """Budget allocator fused with the packer: draft scores [n_bs, W-1] fp32 -> adjusted
    lengths k, seeds k0, offsets and slot arrays (device tensors; `out` may supply them)."""
    lib = _lib.load()
    dev = ctx_len.device
    n_bs, W = block_tokens.shape
    _need(scores, torch.float32, "scores", dev)
    if tuple(scores.shape) != (n_bs, W - 1):
        raise ValueError(f"scores must be [{n_bs}, {W - 1}], got {tuple(scores.shape)}")
    for t, dt, nm in ((ctx_len, torch.int32, "ctx_len"), (kv_base, torch.int64, "kv_base"),
                      (block_tokens, torch.int32, "block_tokens")):
        _need(t, dt, nm, dev)
    if out is None:
        out = dict(
            k=torch.empty(n_bs, dtype=torch.int32, device=dev),
            k0=torch.empty(n_bs, dtype=torch.int32, device=dev),
            offsets=torch.empty(n_bs + 1, dtype=torch.int32, device=dev),
            slot_req=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_tok=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_pos=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_cache_loc=torch.empty(m_bs, dtype=torch.int64, device=dev),
        )
    check(lib.dsv_allocate_pack(n_live, n_bs, W, m_live, m_bs, _ptr(scores), _ptr(ctx_len), _ptr(kv_base),
                                _ptr(block_tokens), _ptr(out["k"]), _ptr(out.get("k0")), _ptr(out["offsets"]),
                                _ptr(out["slot_req"]), _ptr(out["slot_tok"]), _ptr(out["slot_pos"]),
                                _ptr(out["slot_cache_loc"]), _ptr(status), _stream(stream)),
          "dsv_allocate_pack")
    return out


# ---------------------------------------------------------------------------
# dsv_verify_attn
# ---------------------------------------------------------------------------
@dataclass
class Prefill:
    """Prefill set of a dsv_verify_attn call (device tensors except max_len)."""
    q_start: torch.Tensor
    q_len: torch.Tensor
    ctx_len: torch.Tensor
    kv_base: torch.Tensor
    q: torch.Tensor
    out: torch.Tensor
    max_len: int
    lse: torch.Tensor | None = None
    k_new: torch.Tensor | None = None
    v_new: torch.Tensor | None = None


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _lib.DSV_BF16
    if t.dtype == torch.float32:
        return _lib.DSV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def attn_args(q, k_pool, v_pool, offsets, k, ctx_len, kv_base, *, W: int, max_ctx: int, out,
              status, lse=None, k_new=None, v_new=None, slot_cache_loc=None, scale: float = 0.0,
              kv_chunk: int = 0, prefill: Prefill | None = None, workspace=None,
              events=None, kv_index=None) -> AttnArgs:
    """Builds the dsv_attn_args struct.  q [m_bs, hq, d]; pools [hkv, rows, d] (row stride may
    exceed d); out like q; kv_index (optional) [n_bs, stride] int32 token-granular cache map."""
    a = AttnArgs()
    ref = q if q is not None else prefill.q
    a.dtype = _dtype_code(ref)
    hkv, rows, d = k_pool.shape
    a.hq = ref.shape[1]
    a.hkv = hkv
    a.d = d
    a.softmax_scale = scale
    a.kv_chunk = kv_chunk
    a.max_ctx = max_ctx
    a.k_pool, a.v_pool = k_pool.data_ptr(), v_pool.data_ptr()
    a.pool_rows = rows
    a.stride_head = k_pool.stride(0)
    a.stride_row = k_pool.stride(1)
    if k_pool.stride(2) != 1 or v_pool.stride() != k_pool.stride():
        raise ValueError("pools must share strides with unit stride along head_dim")
    if q is not None and k is not None and k.numel() > 0:
        a.n_bs = k.shape[0]
        a.m_bs = q.shape[0]
        a.W = W
        a.offsets = offsets.data_ptr() if offsets is not None else None  # None: pack_verify_attn
        a.k, a.ctx_len, a.kv_base = (t.data_ptr() for t in (k, ctx_len, kv_base))
        a.slot_cache_loc = slot_cache_loc.data_ptr() if slot_cache_loc is not None else None
        a.q = q.data_ptr()
        a.k_new = k_new.data_ptr() if k_new is not None else None
        a.v_new = v_new.data_ptr() if v_new is not None else None
        a.out = out.data_ptr()
        a.lse = lse.data_ptr() if lse is not None else None
    else:
        a.W = W
    if prefill is not None:
        a.n_pf = prefill.q_len.shape[0]
        a.pf_max_len = prefill.max_len
        a.pf_q_rows = prefill.q.shape[0]
        a.pf_q_start, a.pf_q_len = prefill.q_start.data_ptr(), prefill.q_len.data_ptr()
        a.pf_ctx_len, a.pf_kv_base = prefill.ctx_len.data_ptr(), prefill.kv_base.data_ptr()
        a.pf_q = prefill.q.data_ptr()
        a.pf_k_new = prefill.k_new.data_ptr() if prefill.k_new is not None else None
        a.pf_v_new = prefill.v_new.data_ptr() if prefill.v_new is not None else None
        a.pf_out = prefill.out.data_ptr()
        a.pf_lse = prefill.lse.data_ptr() if prefill.lse is not None else None
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.status = status.data_ptr()
    if events is not None:
        a.main_begin, a.main_end = events
    if kv_index is not None:
        if kv_index.dtype != torch.int32 or kv_index.dim() != 2 or not kv_index.is_contiguous():
            raise ValueError("kv_index must be a contiguous [n_bs, stride] int32 tensor")
        a.kv_index = kv_index.data_ptr()
        a.kv_index_stride = kv_index.shape[1]
    return a


def verify_attn_workspace_bytes(args: AttnArgs) -> int:
    return int(_lib.load().dsv_verify_attn_workspace_bytes(ctypes.byref(args)))


def verify_attn_call(args: AttnArgs, stream=None):
    check(_lib.load().dsv_verify_attn(ctypes.byref(args), _stream(stream)), "dsv_verify_attn")


def verify_attn_noalloc_call(args: AttnArgs, stream=None):
    """dsv_verify_attn_noalloc: as verify_attn_call, with the split partials in the library's
    fixed per-GPU scratch array (args.workspace is ignored; no device memory is allocated)."""
    check(_lib.load().dsv_verify_attn_noalloc(ctypes.byref(args), _stream(stream)),
          "dsv_verify_attn_noalloc")


def pack_verify_attn(args: AttnArgs, block_tokens, out=None, stream=None) -> dict:
    """dsv_pack_verify_attn: the packer fused into the verification launch.  `args` as for
    verify_attn_call (its offsets and slot_cache_loc are ignored); block_tokens [n_bs, W]
    int32.  Returns the packer's outputs (as pack_slots; `out` may supply them)."""
    lib = _lib.load()
    dev = block_tokens.device
    _need(block_tokens, torch.int32, "block_tokens", dev)
    n_bs, m_bs = int(args.n_bs), int(args.m_bs)
    if tuple(block_tokens.shape) != (n_bs, int(args.W)):
        raise ValueError("block_tokens: expected [n_bs, W]")
    if out is None:
        out = dict(
            offsets=torch.empty(n_bs + 1, dtype=torch.int32, device=dev),
            slot_req=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_tok=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_pos=torch.empty(m_bs, dtype=torch.int32, device=dev),
            slot_cache_loc=torch.empty(m_bs, dtype=torch.int64, device=dev),
        )
    for key, dt, n in (("offsets", torch.int32, n_bs + 1), ("slot_req", torch.int32, m_bs),
                       ("slot_tok", torch.int32, m_bs), ("slot_pos", torch.int32, m_bs),
                       ("slot_cache_loc", torch.int64, m_bs)):
        _need(out[key], dt, key, dev)
        if out[key].numel() < n:
            raise ValueError(f"{key}: expected at least {n} elements")
    check(lib.dsv_pack_verify_attn(ctypes.byref(args), _ptr(block_tokens), _ptr(out["offsets"]),
                                   _ptr(out["slot_req"]), _ptr(out["slot_tok"]), _ptr(out["slot_pos"]),
                                   _ptr(out["slot_cache_loc"]), _stream(stream)), "dsv_pack_verify_attn")
    return out


def verify_attn(q, k_pool, v_pool, offsets, k, ctx_len, kv_base, *, W: int, max_ctx: int,
                status, out=None, lse=None, k_new=None, v_new=None, slot_cache_loc=None,
                scale: float = 0.0, kv_chunk: int = 0, prefill: Prefill | None = None,
                workspace=None, stream=None, kv_index=None):
    """Attention over packed verification slots (and an optional prefill set).  Allocates
    `out` and the workspace when they are not given.  Returns (out, lse)."""
    if out is None and q is not None:
        out = torch.empty_like(q)
    args = attn_args(q, k_pool, v_pool, offsets, k, ctx_len, kv_base, W=W, max_ctx=max_ctx,
                     out=out, status=status, lse=lse, k_new=k_new, v_new=v_new,
                     slot_cache_loc=slot_cache_loc, scale=scale, kv_chunk=kv_chunk,
                     prefill=prefill, kv_index=kv_index)
    need = verify_attn_workspace_bytes(args)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=k_pool.device)
    if workspace is not None:
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    verify_attn_call(args, stream)
    return out, lse


# ---------------------------------------------------------------------------
# dsv_accept
# ---------------------------------------------------------------------------
def accept_workspace_bytes(m_bs, vocab, n_bs, n_pos, draft_vocab) -> int:
    return int(_lib.load().dsv_accept_workspace_bytes(m_bs, vocab, n_bs, n_pos, draft_vocab))


def accept(*, n_bs: int, W: int, status, target_logits=None, slot_tok=None, offsets=None, k=None,
           draft_logits=None, out=None, workspace=None, stream=None) -> dict:
    """Greedy prefix verification over target_logits [m_bs, vocab] and/or the draft top-1/top-2
    margin over draft_logits [n_bs, n_pos, draft_vocab].  Returns the output tensors."""
    lib = _lib.load()
    dev = status.device
    m_bs = vocab = n_pos = dvocab = 0
    if target_logits is not None:
        _need(target_logits, torch.float32, "target_logits", dev)
        m_bs, vocab = target_logits.shape
    if draft_logits is not None:
        _need(draft_logits, torch.float32, "draft_logits", dev)
        _, n_pos, dvocab = draft_logits.shape
    o = out if out is not None else {}
    if target_logits is not None:
        o.setdefault("slot_argmax", torch.empty(m_bs, dtype=torch.int32, device=dev))
        for nm in ("accepted", "bonus", "progress"):
            o.setdefault(nm, torch.empty(n_bs, dtype=torch.int32, device=dev))
        o.setdefault("out_tokens", torch.empty((n_bs, W), dtype=torch.int32, device=dev))
    if draft_logits is not None:
        o.setdefault("margin", torch.empty((n_bs, n_pos), dtype=torch.float32, device=dev))
        o.setdefault("draft_top1", torch.empty((n_bs, n_pos), dtype=torch.int32, device=dev))
    need = accept_workspace_bytes(m_bs, vocab, n_bs if draft_logits is not None else 0, n_pos, dvocab)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    check(lib.dsv_accept(
        n_bs, m_bs, W, vocab, _ptr(target_logits), _ptr(slot_tok), _ptr(offsets), _ptr(k),
        _ptr(o.get("slot_argmax")), _ptr(o.get("accepted")), _ptr(o.get("bonus")),
        _ptr(o.get("progress")), _ptr(o.get("out_tokens")), _ptr(draft_logits), n_pos, dvocab,
        _ptr(o.get("margin")), _ptr(o.get("draft_top1")), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _ptr(status), _stream(stream)),
        "dsv_accept")
    return o


# ---------------------------------------------------------------------------
# dsv_accept_sample
# ---------------------------------------------------------------------------
def accept_sample_workspace_bytes(n_bs, m_bs, vocab) -> int:
    return int(_lib.load().dsv_accept_sample_workspace_bytes(n_bs, m_bs, vocab))


def accept_sample(*, n_bs: int, W: int, status, target_logits, temperature: float, slot_tok,
                  offsets, k, u_accept, u_draw, out=None, workspace=None, stream=None) -> dict:
    """Sampling-mode prefix verification over target_logits [m_bs, vocab] at `temperature`,
    with the caller's uniforms u_accept [m_bs] and u_draw [n_bs].  Returns accepted, bonus,
    progress, out_tokens and p_cand."""
    lib = _lib.load()
    dev = status.device
    _need(target_logits, torch.float32, "target_logits", dev)
    m_bs, vocab = target_logits.shape
    for t, dt, nm in ((slot_tok, torch.int32, "slot_tok"), (offsets, torch.int32, "offsets"),
                      (k, torch.int32, "k"), (u_accept, torch.float32, "u_accept"),
                      (u_draw, torch.float32, "u_draw")):
        _need(t, dt, nm, dev)
    if slot_tok.numel() < m_bs or u_accept.numel() < m_bs or u_draw.numel() < n_bs:
        raise ValueError("slot_tok and u_accept need m_bs entries, u_draw n_bs")
    if offsets.numel() < n_bs + 1 or k.numel() < n_bs:
        raise ValueError("offsets needs n_bs + 1 entries, k n_bs")
    o = out if out is not None else {}
    for nm in ("accepted", "bonus", "progress"):
        o.setdefault(nm, torch.empty(n_bs, dtype=torch.int32, device=dev))
    o.setdefault("out_tokens", torch.empty((n_bs, W), dtype=torch.int32, device=dev))
    o.setdefault("p_cand", torch.full((m_bs,), float("nan"), dtype=torch.float32, device=dev))
    need = accept_sample_workspace_bytes(n_bs, m_bs, vocab)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    check(lib.dsv_accept_sample(
        n_bs, m_bs, W, vocab, _ptr(target_logits), float(temperature), _ptr(slot_tok),
        _ptr(offsets), _ptr(k), _ptr(u_accept), _ptr(u_draw), _ptr(o["accepted"]),
        _ptr(o["bonus"]), _ptr(o["progress"]), _ptr(o.get("out_tokens")), _ptr(o.get("p_cand")),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _ptr(status),
        _stream(stream)), "dsv_accept_sample")
    return o


# ---------------------------------------------------------------------------
# dsv_draft_features
# ---------------------------------------------------------------------------
def draft_features_workspace_bytes(rows, vocab) -> int:
    return int(_lib.load().dsv_draft_features_workspace_bytes(rows, vocab))


def draft_features(draft_logits, status, out=None, workspace=None, stream=None):
    """Confidence features of draft_logits [..., vocab] (vocab >= 16): float32 [..., 18] =
    top logit, gaps to ranks 2..16, top log-probability, entropy."""
    lib = _lib.load()
    dev = status.device
    _need(draft_logits, torch.float32, "draft_logits", dev)
    lead = tuple(draft_logits.shape[:-1])
    vocab = draft_logits.shape[-1]
    rows = 1
    for n in lead:
        rows *= n
    if out is None:
        out = torch.empty(lead + (18,), dtype=torch.float32, device=dev)
    _need(out, torch.float32, "out", dev)
    need = draft_features_workspace_bytes(rows, vocab)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    check(lib.dsv_draft_features(rows, vocab, _ptr(draft_logits), _ptr(out), _ptr(workspace),
                                 workspace.numel() if workspace is not None else 0, _ptr(status),
                                 _stream(stream)), "dsv_draft_features")
    return out


# ---------------------------------------------------------------------------
# dsv_philox_uniforms
# ---------------------------------------------------------------------------
def philox_uniforms(key: int, counter: int, n: int, device=None, out=None, stream=None):
    """n float32 uniforms in [0, 1) from Philox4x64-10 under the 128-bit key, starting at the
    128-bit counter (ceil(n / 4) counter values are consumed)."""
    lib = _lib.load()
    key, counter = int(key), int(counter)
    if not (0 <= key < 1 << 128 and 0 <= counter < 1 << 128):
        raise DsvError(1, "dsv_philox_uniforms")
    if out is None:
        if device is None:
            raise ValueError("philox_uniforms: give the device or an output tensor")
        out = torch.empty(int(n), dtype=torch.float32, device=device)
    if out.device.type != "cuda" or out.numel() < int(n):
        raise ValueError("philox_uniforms: out must be a GPU tensor of at least n floats")
    _need(out, torch.float32, "out", out.device)
    m = (1 << 64) - 1
    check(lib.dsv_philox_uniforms(key & m, key >> 64, counter & m, counter >> 64, int(n), _ptr(out),
                                  _stream(stream)), "dsv_philox_uniforms")
    return out
