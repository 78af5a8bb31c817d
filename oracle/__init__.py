"""CPU oracle for packed block verification -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It shares no code with the HIP library: the
arithmetic lives in ``dsv_oracle.c`` (plain C, fp64 attention, integer
acceptance), compiled with gcc into ``libdsv_oracle.so`` next to this file;
this module only marshals numpy arrays.

Each wrapper cites the passage of the pages it follows (see the C file for the
full definitions):

* ``pack``: DScale Sec. III-C "Flat-buffer packer" and Fig. 6 (exclusive-scan
  offsets, identical row mapping for tokens, positions and cache references).
* ``verify_attn`` / ``attn_per_request`` / ``attn_padded``: DScale Sec. III-B
  (tile routing) and Sec. III-D (request-local causal row mask), the packed,
  per-request and padded-and-masked formulations of the same attention.
* ``prefill_attn``: the wide-tile prefill path of Sec. III-B.
* ``accept``: DScale Sec. III-D "Prefix verifier" (greedy), DFlash-Mini-Lab
  exact-prefix acceptance with a non-drafted anchor.
* ``accept_sample``: the same passage's sampling rule (accept with P(x), on the
  first rejection draw from P without x, renormalised).
* ``top2_margin``: the Top1-Top2 draft logit gap of DScale Fig. 4 and the
  DFlash7-ACT margin of DFlash-Mini-Lab.
* ``draft_features``: the 18 per-position confidence values of DScale Sec. III-C
  (Acceptance predictor).
* ``philox_raw`` / ``philox_uniforms``: the counter-based generator for the sampling
  verifier's uniforms, Philox4x64-10 as published by Salmon et al. (SC 2011).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdsv_oracle.so")

BF16 = 0
F32 = 1

_ERRORS = {
    1: "malformed arguments",
    2: "a prefix length outside [0, W] or a bad context/offset",
    3: "sum of prefix lengths exceeds the slot capacity",
    4: "NaN logit",
    5: "visible KV row outside the pool",
}


class OracleError(ValueError):
    """The inputs violate a precondition of the method."""

    def __init__(self, code: int):
        super().__init__(_ERRORS.get(code, f"oracle error {code}"))
        self.code = code


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        # DSV_ORACLE_LIBRARY: another build of the same C source (the sanitizer runs use one)
        lib = ctypes.CDLL(os.environ.get("DSV_ORACLE_LIBRARY") or build())
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_pack.argtypes = [i32, i32, i32] + [P] * 9
        lib.oracle_verify_attn.argtypes = [i32, i32, i32, i32, dbl, P, P, i64, i64, i64, i32, i32] + [P] * 5 + [i64] + [P] * 6
        lib.oracle_attn_one_request.argtypes = [i32, i32, i32, i32, dbl, i32, i32, i64] + [P] * 5
        lib.oracle_attn_padded_masked.argtypes = [i32, i32, i32, i32, i32, i32, dbl, i64] + [P] * 6
        lib.oracle_softmax_probs.argtypes = [i32, i32, dbl, P, P, i64, P]
        lib.oracle_prefill_attn.argtypes = [i32, i32, i32, i32, dbl, P, P, i64, i64, i64, i32] + [P] * 5 + [i32] + [P] * 4
        lib.oracle_argmax_rows.argtypes = [i64, i64, P, P]
        lib.oracle_accept.argtypes = [i32, i32, i32] + [P] * 8
        lib.oracle_top2_margin.argtypes = [i64, i64, P, P, P]
        lib.oracle_draft_features.argtypes = [i64, i64, P, P]
        lib.oracle_accept_sample.argtypes = [i32, i32, i32, i64, P, dbl] + [P] * 12
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_allocate.argtypes = [i32, i32, i32, i32, P, P, P]
        u64 = ctypes.c_uint64
        lib.oracle_philox_raw.argtypes = [u64, u64, u64, u64, i64, P]
        lib.oracle_philox_uniforms.argtypes = [u64, u64, u64, u64, i64, P]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(code: int):
    if code != 0:
        raise OracleError(code)


def _elem_array(a):
    """Returns (contiguous array, oracle dtype code): uint16 = bf16 bits, float32 = fp32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float32:
        return a, F32
    raise TypeError(f"oracle inputs are bf16 bits (uint16) or float32, got {a.dtype}")


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> int:
    """Runs the following oracle calls on n threads (results do not depend on the count);
    returns the count in effect."""
    return int(_load().oracle_set_threads(int(n)))


# --------------------------------------------------------------------------
# Flat-buffer packer
# --------------------------------------------------------------------------
def pack(k, ctx_len, kv_base, block_tokens, W: int, m_bs: int) -> dict:
    lib = _load()
    k = _c(k, np.int32)
    n_bs = k.shape[0]
    ctx_len = _c(ctx_len, np.int32)
    kv_base = _c(kv_base, np.int64)
    block_tokens = _c(block_tokens, np.int32).reshape(n_bs, W)
    out = dict(
        offsets=np.zeros(n_bs + 1, np.int32),
        slot_req=np.zeros(m_bs, np.int32),
        slot_tok=np.zeros(m_bs, np.int32),
        slot_pos=np.zeros(m_bs, np.int32),
        slot_cache_loc=np.zeros(m_bs, np.int64),
    )
    _check(
        lib.oracle_pack(
            n_bs, W, m_bs, _p(k), _p(ctx_len), _p(kv_base), _p(block_tokens),
            _p(out["offsets"]), _p(out["slot_req"]), _p(out["slot_tok"]), _p(out["slot_pos"]),
            _p(out["slot_cache_loc"]),
        )
    )
    return out


# --------------------------------------------------------------------------
# Budget allocator
# --------------------------------------------------------------------------
def allocate(scores, n_live: int, W: int, m_live: int) -> dict:
    """Seeded lengths k0 and adjusted lengths k ([n_bs] int32) from draft scores [n_bs, W-1]
    (rows >= n_live are inactive).  DScale Sec. III-C, Budget allocator."""
    lib = _load()
    scores = _c(scores, np.float32)
    n_bs = scores.shape[0]
    scores = scores.reshape(n_bs, W - 1) if n_bs else scores.reshape(0, max(W - 1, 0))
    out = dict(k0=np.zeros(n_bs, np.int32), k=np.zeros(n_bs, np.int32))
    _check(lib.oracle_allocate(n_live, n_bs, W, m_live, _p(scores), _p(out["k0"]), _p(out["k"])))
    return out


def allocate_pack(scores, n_live: int, W: int, m_live: int, m_bs: int, ctx_len, kv_base, block_tokens) -> dict:
    """Budget allocator followed by the flat-buffer packer on the adjusted lengths."""
    a = allocate(scores, n_live, W, m_live)
    out = pack(a["k"], ctx_len, kv_base, block_tokens, W, m_bs)
    out.update(a)
    return out


# --------------------------------------------------------------------------
# Verification attention: packed, per-request, padded-and-masked
# --------------------------------------------------------------------------
def _scale(d, scale):
    return 1.0 / np.sqrt(d) if not scale else float(scale)


def verify_attn(q, k_pool, v_pool, offsets, k, ctx_len, kv_base, k_new=None, v_new=None,
                scale=0.0, slot_mask=None, kv_index=None):
    """Packed attention.  q [m_bs, hq, d]; pools [hkv, rows, d]; returns (out, lse) in float64.
    kv_index [n_bs, stride] int32, if given, maps position p of request i to pool row
    kv_index[i, p] (token-granular cache map) instead of kv_base[i] + p.

    Rows that no request owns and that precede offsets[-1] come back as NaN (not written)."""
    lib = _load()
    q, dt = _elem_array(q)
    k_pool, dt2 = _elem_array(k_pool)
    v_pool, _ = _elem_array(v_pool)
    assert dt == dt2
    m_bs, hq, d = q.shape
    hkv, rows, d2 = k_pool.shape
    assert d2 == d and v_pool.shape == k_pool.shape
    k = _c(k, np.int32)
    n_bs = k.shape[0]
    offsets = _c(offsets, np.int32)
    ctx_len = _c(ctx_len, np.int32)
    kv_base = _c(kv_base, np.int64)
    if k_new is not None:
        k_new, _ = _elem_array(k_new)
        v_new, _ = _elem_array(v_new)
        assert k_new.shape == (m_bs, hkv, d) and v_new.shape == (m_bs, hkv, d)
    if slot_mask is not None:
        slot_mask = _c(slot_mask, np.uint8)
    stride = 0
    if kv_index is not None:
        kv_index = _c(kv_index, np.int32)
        assert kv_index.ndim == 2 and kv_index.shape[0] == n_bs
        stride = kv_index.shape[1]
    out = np.full((m_bs, hq, d), np.nan)
    lse = np.full((m_bs, hq), np.nan)
    _check(
        lib.oracle_verify_attn(
            dt, hq, hkv, d, _scale(d, scale), _p(k_pool), _p(v_pool), rows, rows * d, d,
            n_bs, m_bs, _p(offsets), _p(k), _p(ctx_len), _p(kv_base), _p(kv_index), stride, _p(q),
            _p(k_new), _p(v_new), _p(slot_mask), _p(out), _p(lse),
        )
    )
    return out, lse


def _request_sequence(k_pool, v_pool, i, offsets, k, ctx_len, kv_base, k_new, v_new):
    """Key/value sequence of request i in position order: [hkv, ctx_i + k_i, d]."""
    c, b, kk, off = int(ctx_len[i]), int(kv_base[i]), int(k[i]), int(offsets[i])
    Ks = k_pool[:, b:b + c + kk, :].copy()
    Vs = v_pool[:, b:b + c + kk, :].copy()
    if k_new is not None:
        Ks[:, c:c + kk, :] = np.transpose(k_new[off:off + kk], (1, 0, 2))
        Vs[:, c:c + kk, :] = np.transpose(v_new[off:off + kk], (1, 0, 2))
    return Ks, Vs


def attn_per_request(q, k_pool, v_pool, offsets, k, ctx_len, kv_base, k_new=None, v_new=None,
                     scale=0.0):
    """Each request on its own (unpacked); results scattered back to packed rows."""
    lib = _load()
    q, dt = _elem_array(q)
    m_bs, hq, d = q.shape
    hkv = k_pool.shape[0]
    out = np.full((m_bs, hq, d), np.nan)
    lse = np.full((m_bs, hq), np.nan)
    for i in range(len(k)):
        kk = int(k[i])
        if kk == 0:
            continue
        Ks, Vs = _request_sequence(k_pool, v_pool, i, offsets, k, ctx_len, kv_base, k_new, v_new)
        Ks, _ = _elem_array(Ks)
        Vs, _ = _elem_array(Vs)
        qr = np.ascontiguousarray(q[offsets[i]:offsets[i] + kk])
        o = np.zeros((kk, hq, d))
        l = np.zeros((kk, hq))
        _check(lib.oracle_attn_one_request(dt, hq, hkv, d, _scale(d, scale), int(ctx_len[i]), kk,
                                           Ks.shape[1], _p(qr), _p(Ks), _p(Vs), _p(o), _p(l)))
        out[offsets[i]:offsets[i] + kk] = o
        lse[offsets[i]:offsets[i] + kk] = l
    end = int(offsets[len(k)])
    out[end:] = 0.0
    lse[end:] = -np.inf
    return out, lse


def attn_padded(q, k_pool, v_pool, offsets, k, ctx_len, kv_base, W, k_new=None, v_new=None,
                scale=0.0):
    """Padded-and-masked: every request gets W query rows and a key sequence padded to the
    longest one, with a materialised visibility mask; rows j >= k_i are computed and then
    discarded.  Results are scattered back to packed rows."""
    lib = _load()
    q, dt = _elem_array(q)
    m_bs, hq, d = q.shape
    hkv = k_pool.shape[0]
    n = len(k)
    L = max(1, max(int(ctx_len[i]) + int(k[i]) for i in range(n)) if n else 1)
    zero = np.zeros((), q.dtype)
    q_pad = np.full((n, W, hq, d), zero, q.dtype)
    K_pad = np.full((n, hkv, L, d), zero, q.dtype)
    V_pad = np.full((n, hkv, L, d), zero, q.dtype)
    mask = np.zeros((n, W, L), np.uint8)
    for i in range(n):
        kk, c = int(k[i]), int(ctx_len[i])
        if kk:
            q_pad[i, :kk] = q[offsets[i]:offsets[i] + kk]
            Ks, Vs = _request_sequence(k_pool, v_pool, i, offsets, k, ctx_len, kv_base, k_new, v_new)
            K_pad[i, :, :c + kk] = Ks
            V_pad[i, :, :c + kk] = Vs
        for j in range(W):
            mask[i, j, : c + j + 1] = 1
    o = np.zeros((n, W, hq, d))
    l = np.zeros((n, W, hq))
    _check(lib.oracle_attn_padded_masked(dt, n, W, hq, hkv, d, _scale(d, scale), L, _p(q_pad),
                                         _p(K_pad), _p(V_pad), _p(mask), _p(o), _p(l)))
    out = np.full((m_bs, hq, d), np.nan)
    lse = np.full((m_bs, hq), np.nan)
    for i in range(n):
        kk = int(k[i])
        out[offsets[i]:offsets[i] + kk] = o[i, :kk]
        lse[offsets[i]:offsets[i] + kk] = l[i, :kk]
    end = int(offsets[n])
    out[end:] = 0.0
    lse[end:] = -np.inf
    return out, lse


def softmax_probs(q_row, K_rows, scale=0.0):
    """Materialised attention weights of one query row over K_rows [n, d]."""
    lib = _load()
    q_row, dt = _elem_array(q_row)
    K_rows, _ = _elem_array(K_rows)
    n, d = K_rows.shape
    p = np.zeros(n)
    _check(lib.oracle_softmax_probs(dt, d, _scale(d, scale), _p(q_row), _p(K_rows), n, _p(p)))
    return p


def prefill_attn(pf_q, k_pool, v_pool, q_start, q_len, ctx_len, kv_base, sel_req, sel_j, scale=0.0):
    """Prefill rows (request sel_req[t], row sel_j[t]); returns (out [n_sel, hq, d], lse [n_sel, hq])."""
    lib = _load()
    pf_q, dt = _elem_array(pf_q)
    k_pool, _ = _elem_array(k_pool)
    v_pool, _ = _elem_array(v_pool)
    _, hq, d = pf_q.shape
    hkv, rows, _ = k_pool.shape
    q_start, q_len, ctx_len = (_c(x, np.int32) for x in (q_start, q_len, ctx_len))
    kv_base = _c(kv_base, np.int64)
    sel_req, sel_j = _c(sel_req, np.int32), _c(sel_j, np.int32)
    n_sel = sel_req.shape[0]
    out = np.zeros((n_sel, hq, d))
    lse = np.zeros((n_sel, hq))
    _check(lib.oracle_prefill_attn(dt, hq, hkv, d, _scale(d, scale), _p(k_pool), _p(v_pool), rows,
                                   rows * d, d, len(q_len), _p(q_start), _p(q_len), _p(ctx_len),
                                   _p(kv_base), _p(pf_q), n_sel, _p(sel_req), _p(sel_j), _p(out), _p(lse)))
    return out, lse


def scatter_candidates(k_pool, v_pool, k_new, v_new, slot_cache_loc):
    """This step's candidate KV written at the packed cache references (new pool copies)."""
    k_pool = k_pool.copy()
    v_pool = v_pool.copy()
    for s, loc in enumerate(np.asarray(slot_cache_loc)):
        if loc >= 0:
            k_pool[:, loc, :] = k_new[s]
            v_pool[:, loc, :] = v_new[s]
    return k_pool, v_pool


# --------------------------------------------------------------------------
# Acceptance
# --------------------------------------------------------------------------
def argmax_rows(logits):
    lib = _load()
    logits = _c(logits, np.float32)
    rows, vocab = logits.shape
    out = np.zeros(rows, np.int32)
    _check(lib.oracle_argmax_rows(rows, vocab, _p(logits), _p(out)))
    return out


def accept(logits, slot_tok, offsets, k, W: int) -> dict:
    """Greedy prefix verification.  slot_argmax is computed for slots < offsets[-1] and is -1
    for the tail."""
    lib = _load()
    logits = _c(logits, np.float32)
    m_bs = logits.shape[0]
    offsets = _c(offsets, np.int32)
    k = _c(k, np.int32)
    n_bs = k.shape[0]
    end = int(offsets[n_bs])
    slot_argmax = np.full(m_bs, -1, np.int32)
    if end > 0:
        slot_argmax[:end] = argmax_rows(logits[:end])
    out = dict(
        slot_argmax=slot_argmax,
        accepted=np.zeros(n_bs, np.int32),
        bonus=np.zeros(n_bs, np.int32),
        progress=np.zeros(n_bs, np.int32),
        out_tokens=np.zeros((n_bs, W), np.int32),
    )
    slot_tok = _c(slot_tok, np.int32)
    _check(lib.oracle_accept(n_bs, m_bs, W, _p(offsets), _p(k), _p(slot_tok), _p(slot_argmax),
                             _p(out["accepted"]), _p(out["bonus"]), _p(out["progress"]),
                             _p(out["out_tokens"])))
    return out


def accept_sample(logits, slot_tok, offsets, k, W: int, temperature: float, u_accept, u_draw) -> dict:
    """Sampling-mode prefix verification (DScale Sec. III-D "Prefix verifier") at temperature T
    with the caller's uniforms: u_accept [m_bs] (row s tests the candidate at slot s + 1),
    u_draw [n_bs] (one successor draw per request).  Returns accepted, bonus, progress,
    out_tokens, p_cand (P of the tested candidate per row, -1 on a request's last row) and the
    decision margins acc_margin [m_bs] / draw_margin [n_bs] (NaN where no decision was
    taken)."""
    lib = _load()
    logits = _c(logits, np.float32)
    m_bs, vocab = logits.shape
    offsets = _c(offsets, np.int32)
    k = _c(k, np.int32)
    n_bs = k.shape[0]
    slot_tok = _c(slot_tok, np.int32)
    u_accept = _c(u_accept, np.float32)
    u_draw = _c(u_draw, np.float32)
    assert slot_tok.shape[0] >= m_bs and u_accept.shape[0] >= m_bs and u_draw.shape[0] >= n_bs
    out = dict(
        accepted=np.zeros(n_bs, np.int32),
        bonus=np.zeros(n_bs, np.int32),
        progress=np.zeros(n_bs, np.int32),
        out_tokens=np.zeros((n_bs, W), np.int32),
        p_cand=np.full(m_bs, np.nan),
        acc_margin=np.zeros(m_bs),
        draw_margin=np.zeros(n_bs),
    )
    _check(lib.oracle_accept_sample(
        n_bs, m_bs, W, vocab, _p(logits), float(temperature), _p(offsets), _p(k), _p(slot_tok),
        _p(u_accept), _p(u_draw), _p(out["accepted"]), _p(out["bonus"]), _p(out["progress"]),
        _p(out["out_tokens"]), _p(out["p_cand"]), _p(out["acc_margin"]), _p(out["draw_margin"])))
    return out


def top2_margin(draft_logits):
    """draft_logits [..., vocab] -> (margin float32 [...], top1 int32 [...])."""
    lib = _load()
    x = _c(draft_logits, np.float32)
    lead = x.shape[:-1]
    vocab = x.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    margin = np.zeros(rows, np.float32)
    top1 = np.zeros(rows, np.int32)
    _check(lib.oracle_top2_margin(rows, vocab, _p(x), _p(margin), _p(top1)))
    return margin.reshape(lead), top1.reshape(lead)


def draft_features(draft_logits):
    """draft_logits [..., vocab] (vocab >= 16) -> features float32 [..., 18]: the top logit,
    its gaps to ranks 2..16, the top token's log-probability and the entropy (DScale Sec. III-C,
    Acceptance predictor)."""
    lib = _load()
    x = _c(draft_logits, np.float32)
    lead = x.shape[:-1]
    vocab = x.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    feat = np.zeros((rows, 18), np.float32)
    _check(lib.oracle_draft_features(rows, vocab, _p(x), _p(feat)))
    return feat.reshape(lead + (18,))


def _split128(v):
    v = int(v)
    if v < 0 or v >= 1 << 128:
        raise OracleError("key and counter are 128-bit unsigned integers")
    return v & ((1 << 64) - 1), v >> 64


def philox_raw(key, counter, n):
    """n 64-bit words of Philox4x64-10 (Salmon et al., SC 2011) under a 128-bit key: word i is
    word i % 4 of the block at the 128-bit counter `counter + i // 4`."""
    lib = _load()
    k0, k1 = _split128(key)
    c0, c1 = _split128(counter)
    out = np.zeros(int(n), np.uint64)
    _check(lib.oracle_philox_raw(k0, k1, c0, c1, int(n), _p(out)))
    return out


def philox_uniforms(key, counter, n):
    """float32 uniforms in [0, 1): the top 24 bits of each word of philox_raw, times 2^-24."""
    lib = _load()
    k0, k1 = _split128(key)
    c0, c1 = _split128(counter)
    out = np.zeros(int(n), np.float32)
    _check(lib.oracle_philox_uniforms(k0, k1, c0, c1, int(n), _p(out)))
    return out
