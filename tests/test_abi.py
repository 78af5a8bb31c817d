"""CPU checks of the C ABI: the library loads (no GPU needed to dlopen it) and exports every
function include/*.h declares, and the binding's struct matches the library's."""
import ctypes
import glob
import os
import re

import block_verification_attention_amd as dsv
from block_verification_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(dsv_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    dsv.load_library()
    lib = ctypes.CDLL(_lib.LIB_PATH)
    declared = _declared_functions()
    assert {"dsv_pack_slots", "dsv_verify_attn", "dsv_accept"} <= declared
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_struct_layout_and_version():
    lib = _lib.load()
    assert lib.dsv_attn_args_size() == ctypes.sizeof(_lib.AttnArgs)
    assert lib.dsv_abi_version() == 1
    assert _lib.status_string(0) == "ok"
    assert "workspace" in _lib.status_string(3)


def test_host_validation_without_gpu():
    """Host-detectable errors return before anything is enqueued (no GPU is touched)."""
    lib = _lib.load()
    st = ctypes.c_int32(0)
    # W out of range
    assert lib.dsv_pack_slots(1, 17, 4, None, None, None, None, ctypes.byref(st), None, None, None,
                              None, ctypes.byref(st), None) == 1
    a = _lib.AttnArgs()
    a.dtype = 0
    a.d = 96  # unsupported head_dim
    a.hq = a.hkv = 1
    a.status = ctypes.addressof(st)
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 2
    a.d = 128
    a.hq, a.hkv = 34, 2  # G = 17 > 16
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 2
    a.hq, a.hkv = 3, 2
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1
    # bf16 verification at head_dim 256 takes every grouping of one to sixteen query heads per
    # KV head (also through the fused packer): these pass the grouping checks and fail a later
    # one (no pools)
    a.d, a.n_bs, a.m_bs, a.W = 256, 2, 8, 16
    for hq, hkv in ((4, 4), (2, 1), (8, 4), (6, 2), (16, 1)):
        a.hq, a.hkv = hq, hkv
        assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1, (hq, hkv)
        dmy = ctypes.c_void_p(16)
        assert lib.dsv_pack_verify_attn(ctypes.byref(a), dmy, dmy, dmy, dmy, dmy, dmy, None) == 1
    a.hq, a.hkv, a.dtype = 4, 4, 1
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1
    a.dtype, a.n_bs = 0, 0
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1
    a.d, a.hq, a.hkv, a.m_bs, a.W = 128, 1, 1, 0, 0
    # accept: missing workspace for a real sweep
    assert lib.dsv_accept(1, 4, 16, 100, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                          ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16),
                          ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, 0, 0, None, None,
                          None, 0, ctypes.byref(st), None) == 3
    # fused packer + verification: fp32, a cache map, no requests or a missing packer output
    # are refused before anything is enqueued
    b = _lib.AttnArgs()
    b.dtype, b.d, b.hq, b.hkv, b.n_bs, b.m_bs, b.W = 1, 128, 8, 2, 2, 8, 16
    b.status = ctypes.addressof(st)
    dummy = ctypes.c_void_p(16)
    outs = [dummy] * 6
    assert lib.dsv_pack_verify_attn(ctypes.byref(b), *outs, None) == 2    # fp32
    b.dtype = 0
    b.kv_index = 16
    assert lib.dsv_pack_verify_attn(ctypes.byref(b), *outs, None) == 2    # cache map
    b.kv_index = None
    b.n_bs = 0
    assert lib.dsv_pack_verify_attn(ctypes.byref(b), *outs, None) == 2    # no verification set
    b.n_bs = 2
    assert lib.dsv_pack_verify_attn(ctypes.byref(b), dummy, None, dummy, dummy, dummy, dummy, None) == 1
    # the no-allocation verification call validates like dsv_verify_attn before it touches
    # the device (its scratch array is looked up only for a call that needs it)
    assert lib.dsv_verify_attn_noalloc(None, None) == 1
    a.d = 96
    assert lib.dsv_verify_attn_noalloc(ctypes.byref(a), None) == 2
    a.d = 128
    assert lib.dsv_verify_attn_noalloc(ctypes.byref(a), None) == 1  # no pools
    # counter-based uniforms: negative length, missing output; an empty stream enqueues nothing
    assert lib.dsv_philox_uniforms(0, 0, 0, 0, -1, ctypes.c_void_p(16), None) == 1
    assert lib.dsv_philox_uniforms(0, 0, 0, 0, 8, None, None) == 1
    assert lib.dsv_philox_uniforms(0, 0, 0, 0, 0, None, None) == 0
    assert st.value == 0


def test_host_validation_next_rows_without_gpu():
    """The allocator, the sampling verifier, the draft features and the read probe refuse
    bad sizes and missing pointers before any HIP call; empty batches enqueue nothing."""
    lib = _lib.load()
    st = ctypes.c_int32(0)
    sp = ctypes.addressof(st)
    d = ctypes.c_void_p(16)
    # allocator + pack: more than 1024 requests, W out of range, missing k, m_bs < m_live
    alloc = lambda n_live, n_bs, W, m_live, m_bs, k=d: lib.dsv_allocate_pack(  # noqa: E731
        n_live, n_bs, W, m_live, m_bs, d, d, d, d, k, d, d, d, d, d, d, sp, None)
    assert alloc(4, 1025, 16, 8, 64) == 1
    assert alloc(4, 8, 17, 8, 64) == 1
    assert alloc(4, 8, 16, 8, 64, k=None) == 1
    assert alloc(4, 8, 16, 65, 64) == 1
    assert alloc(9, 8, 16, 8, 64) == 1
    # sampling verifier: temperature not positive and finite, W out of range, missing output
    samp = lambda n_bs, W, T, acc=d: lib.dsv_accept_sample(  # noqa: E731
        n_bs, 64, W, 1000, d, T, d, d, d, d, d, acc, d, d, d, d, d, 1 << 20, sp, None)
    for T in (0.0, -1.0, float("nan"), float("inf")):
        assert samp(4, 16, T) == 1, T
    assert samp(4, 0, 0.8) == 1
    assert samp(4, 16, 0.8, acc=None) == 1
    assert samp(0, 16, 0.8) == 0
    # draft features: fewer than 16 logits, missing input, too small a workspace, no rows
    assert lib.dsv_draft_features(4, 15, d, d, d, 1 << 20, sp, None) == 1
    assert lib.dsv_draft_features(4, 4096, None, d, d, 1 << 20, sp, None) == 1
    need = lib.dsv_draft_features_workspace_bytes(4, 4096)
    assert lib.dsv_draft_features(4, 4096, d, d, d, need - 1, sp, None) == 3
    assert lib.dsv_draft_features(0, 4096, None, None, None, 0, sp, None) == 0
    # read probe: null, unaligned or shorter than 16 bytes
    assert lib.dsv_probe_stream_read(None, 1 << 20, d, None) == 1
    assert lib.dsv_probe_stream_read(ctypes.c_void_p(24), 1 << 20, d, None) == 1
    assert lib.dsv_probe_stream_read(d, 15, d, None) == 1
    assert st.value == 0


def test_aliasing_refused_without_gpu():
    """An output that shares a byte with another output or with an input is refused with
    DSV_ERR_INVALID_ARG before anything is enqueued (fake, 256-byte aligned, far-apart device
    addresses; each call has exactly one overlap)."""
    lib = _lib.load()
    st = ctypes.c_int32(0)
    sp = ctypes.addressof(st)
    base = 1 << 40
    slot = iter(range(1, 1000))
    fresh = lambda: base + next(slot) * (1 << 32)  # noqa: E731
    P = ctypes.c_void_p
    # pack: offsets[1] is k[0]; slot_pos is slot_tok shifted by 4 bytes
    k, ctx, kvb, tok = fresh(), fresh(), fresh(), fresh()
    outs = [fresh() for _ in range(5)]
    assert lib.dsv_pack_slots(4, 16, 64, P(k), P(ctx), P(kvb), P(tok), P(k - 4), P(outs[1]), P(outs[2]),
                              P(outs[3]), P(outs[4]), sp, None) == 1
    assert lib.dsv_pack_slots(4, 16, 64, P(k), P(ctx), P(kvb), P(tok), P(outs[0]), P(outs[1]),
                              P(outs[2]), P(outs[2] + 4), P(outs[4]), sp, None) == 1
    # the status word inside an output
    assert lib.dsv_pack_slots(4, 16, 64, P(k), P(ctx), P(kvb), P(tok), P(outs[0]), P(outs[1]),
                              P(outs[2]), P(outs[3]), P(outs[4]), P(outs[1] + 8), None) == 1
    # allocator: the adjusted lengths over the last score row
    sc = fresh()
    assert lib.dsv_allocate_pack(4, 8, 16, 32, 64, P(sc), P(ctx), P(kvb), P(tok), P(sc + 3 * 15 * 4),
                                 None, P(outs[0]), P(outs[1]), P(outs[2]), P(outs[3]), P(outs[4]),
                                 sp, None) == 1

    def attn(**over):
        a = _lib.AttnArgs()
        a.dtype, a.hq, a.hkv, a.d, a.W, a.max_ctx = 0, 8, 2, 128, 16, 64
        a.n_bs, a.m_bs = 2, 32
        a.pool_rows, a.stride_row = 256, 128
        a.stride_head = 256 * 128
        for name in ("k_pool", "v_pool", "offsets", "k", "ctx_len", "kv_base", "slot_cache_loc",
                     "q", "k_new", "v_new", "out", "lse"):
            setattr(a, name, fresh())
        a.status = sp
        for name, v in over.items():
            setattr(a, name, v(a) if callable(v) else v)
        return a

    # verification: out over q, lse inside out, out over a pool, q over a pool (pools are read
    # and written), a pool over the status word
    for over in ({"out": lambda a: a.q}, {"lse": lambda a: a.out + 1024},
                 {"out": lambda a: a.k_pool + 2 * 256 * 128}, {"q": lambda a: a.v_pool},
                 {"status": lambda a: a.k_pool + 64}):
        a = attn(**over)
        assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1, over
        assert lib.dsv_verify_attn_noalloc(ctypes.byref(a), None) == 1, over
    # fused packer: a packer output over the request lengths
    a = attn(offsets=None)
    bt = fresh()
    assert lib.dsv_pack_verify_attn(ctypes.byref(a), P(bt), P(fresh()), P(a.k), P(fresh()),
                                    P(fresh()), P(fresh()), None) == 1
    # accept: the argmax output over the logits; the workspace over the draft tokens
    need = lib.dsv_accept_workspace_bytes(64, 1000, 4, 15, 1000)
    lg, stok, ws = fresh(), fresh(), fresh()
    args = lambda sa, wsp: (4, 64, 16, 1000, P(lg), P(stok), P(fresh()), P(fresh()), P(sa),  # noqa: E731
                            P(fresh()), P(fresh()), P(fresh()), P(fresh()), P(fresh()), 15, 1000,
                            P(fresh()), P(fresh()), P(wsp), need, sp, None)
    assert lib.dsv_accept(*args(lg + 4 * 1000 * 63, ws)) == 1
    assert lib.dsv_accept(*args(fresh(), stok - 256)) == 1
    # sampling verifier: p_cand over the acceptance uniforms
    need = lib.dsv_accept_sample_workspace_bytes(4, 64, 1000)
    ua = fresh()
    assert lib.dsv_accept_sample(4, 64, 16, 1000, P(lg), 1.0, P(stok), P(fresh()), P(fresh()), P(ua),
                                 P(fresh()), P(fresh()), P(fresh()), P(fresh()), P(fresh()), P(ua),
                                 P(fresh()), need, sp, None) == 1
    # draft features: the features over the logits
    need = lib.dsv_draft_features_workspace_bytes(4, 4096)
    dl = fresh()
    assert lib.dsv_draft_features(4, 4096, P(dl), P(dl + 4096 * 4 * 3), P(fresh()), need, sp, None) == 1
    assert st.value == 0


def test_launch_limits_refused_without_gpu():
    """A call whose launches would exceed a dispatch's 2^32 - 1 work-items is refused with
    DSV_ERR_INVALID_ARG before anything is enqueued (fake, far-apart device addresses)."""
    lib = _lib.load()
    st = ctypes.c_int32(0)
    sp = ctypes.addressof(st)
    base = 1 << 40
    slot = iter(range(1, 1000))
    fresh = lambda: ctypes.c_void_p(base + next(slot) * (1 << 36))  # noqa: E731
    # fp32 prefill: one 256-thread workgroup per (row, query head): 2^25 rows x 8 heads
    a = _lib.AttnArgs()
    a.dtype, a.hq, a.hkv, a.d, a.W = 1, 8, 8, 64, 16
    a.pool_rows, a.stride_row, a.stride_head = 64, 64, 64 * 64
    a.k_pool, a.v_pool = fresh().value, fresh().value
    a.n_pf, a.pf_max_len, a.pf_q_rows = 1, 1 << 25, 16
    for name in ("pf_q_start", "pf_q_len", "pf_ctx_len", "pf_kv_base", "pf_q", "pf_out"):
        setattr(a, name, fresh().value)
    a.status = sp
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1
    # bf16 verification with 64-row splits over a context of 2^30 rows: 2^24 splits x 8
    # KV heads x up to 1024 threads
    b = _lib.AttnArgs()
    b.dtype, b.hq, b.hkv, b.d, b.W, b.max_ctx, b.kv_chunk = 0, 32, 8, 128, 16, 1 << 30, 64
    b.n_bs, b.m_bs = 1, 16
    b.pool_rows, b.stride_row, b.stride_head = 1 << 20, 128, 128 << 20
    for name in ("k_pool", "v_pool", "offsets", "k", "ctx_len", "kv_base", "slot_cache_loc", "q",
                 "out"):
        setattr(b, name, fresh().value)
    b.status = sp
    assert lib.dsv_verify_attn(ctypes.byref(b), None) == 1
    # greedy accept and the sampling verifier over 2^24 + 1 rows of 16 logits
    m = (1 << 24) + 1
    need = lib.dsv_accept_workspace_bytes(m, 16, 0, 0, 0)
    assert lib.dsv_accept(1, m, 16, 16, fresh(), fresh(), fresh(), fresh(), fresh(), fresh(), fresh(),
                          fresh(), None, None, 0, 0, None, None, fresh(), need, sp, None) == 1
    need = lib.dsv_accept_sample_workspace_bytes(1, m, 16)
    assert lib.dsv_accept_sample(1, m, 16, 16, fresh(), 1.0, fresh(), fresh(), fresh(), fresh(),
                                 fresh(), fresh(), fresh(), fresh(), None, None, fresh(), need, sp,
                                 None) == 1
    # draft features over 2^24 rows; uniforms: 2^40 values
    need = lib.dsv_draft_features_workspace_bytes(1 << 24, 16)
    assert lib.dsv_draft_features(1 << 24, 16, fresh(), fresh(), fresh(), need, sp, None) == 1
    assert lib.dsv_philox_uniforms(1, 2, 0, 0, 1 << 40, fresh(), None) == 1
    # absurd counts whose block products pass 64 bits are refused too (no wrap-around)
    assert lib.dsv_draft_features(1 << 62, 16, fresh(), fresh(), fresh(), 1 << 20, sp, None) == 1
    a.n_pf, a.pf_max_len, a.hq, a.hkv = (1 << 31) - 1, (1 << 31) - 1, 1 << 20, 1 << 20
    assert lib.dsv_verify_attn(ctypes.byref(a), None) == 1
    assert st.value == 0


def test_workspace_queries():
    lib = _lib.load()
    assert lib.dsv_accept_workspace_bytes(128, 151936, 0, 0, 0) > 0
    assert lib.dsv_accept_workspace_bytes(0, 0, 32, 15, 248320) > 0
    a = _lib.AttnArgs()
    a.dtype, a.hq, a.hkv, a.d = 0, 32, 8, 128
    a.n_bs, a.m_bs, a.W, a.max_ctx = 8, 128, 16, 8192
    n = lib.dsv_verify_attn_workspace_bytes(ctypes.byref(a))
    assert n > 0 and n % 256 == 0
    a.max_ctx = 16  # one split: no workspace
    assert lib.dsv_verify_attn_workspace_bytes(ctypes.byref(a)) == 0
