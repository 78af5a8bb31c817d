"""ctypes loader for libdsv.so (the HIP library).  Fails loudly when it is not built."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSV_LIBRARY: another build of the library to load instead (for example a sanitizer build of
# its host code); by default the in-tree libdsv.so
LIB_PATH = os.environ.get("DSV_LIBRARY") or os.path.join(_HERE, "libdsv.so")

DSV_BF16 = 0
DSV_F32 = 1

STATUS_BAD_REQUEST = 1
STATUS_BUDGET = 2
STATUS_NAN = 4
STATUS_POOL = 8
STATUS_PREFILL = 16

MAX_W = 16

P = ctypes.c_void_p
i32 = ctypes.c_int32
i64 = ctypes.c_int64


class AttnArgs(ctypes.Structure):
    """Mirror of `dsv_attn_args` in include/dsv.h (same field order and types)."""

    _fields_ = [
        ("dtype", ctypes.c_int),
        ("hq", i32), ("hkv", i32), ("d", i32),
        ("softmax_scale", ctypes.c_float),
        ("kv_chunk", i32), ("max_ctx", i32),
        ("k_pool", P), ("v_pool", P),
        ("pool_rows", i64), ("stride_head", i64), ("stride_row", i64),
        ("n_bs", i32), ("m_bs", i32), ("W", i32),
        ("offsets", P), ("k", P), ("ctx_len", P), ("kv_base", P), ("slot_cache_loc", P),
        ("q", P), ("k_new", P), ("v_new", P), ("out", P), ("lse", P),
        ("n_pf", i32), ("pf_max_len", i32), ("pf_q_rows", i32),
        ("pf_q_start", P), ("pf_q_len", P), ("pf_ctx_len", P), ("pf_kv_base", P),
        ("pf_q", P), ("pf_k_new", P), ("pf_v_new", P), ("pf_out", P), ("pf_lse", P),
        ("workspace", P), ("workspace_bytes", ctypes.c_size_t), ("status", P),
        ("main_begin", P), ("main_end", P),
        ("kv_index", P), ("kv_index_stride", i64),
    ]


class DsvError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


_lib = None


def load():
    """The loaded library; raises if libdsv.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m block_verification_attention_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    lib.dsv_status_string.argtypes = [ctypes.c_int]
    lib.dsv_status_string.restype = ctypes.c_char_p
    lib.dsv_abi_version.argtypes = []
    lib.dsv_abi_version.restype = ctypes.c_int
    lib.dsv_attn_args_size.argtypes = []
    lib.dsv_attn_args_size.restype = ctypes.c_size_t
    lib.dsv_pack_slots.argtypes = [i32, i32, i32] + [P] * 10 + [P]
    lib.dsv_pack_slots.restype = ctypes.c_int
    lib.dsv_allocate_pack.argtypes = [i32] * 5 + [P] * 12 + [P]
    lib.dsv_allocate_pack.restype = ctypes.c_int
    lib.dsv_verify_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs)]
    lib.dsv_verify_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.dsv_verify_attn.argtypes = [ctypes.POINTER(AttnArgs), P]
    lib.dsv_verify_attn.restype = ctypes.c_int
    lib.dsv_verify_attn_noalloc.argtypes = [ctypes.POINTER(AttnArgs), P]
    lib.dsv_verify_attn_noalloc.restype = ctypes.c_int
    lib.dsv_pack_verify_attn.argtypes = [ctypes.POINTER(AttnArgs)] + [P] * 7
    lib.dsv_pack_verify_attn.restype = ctypes.c_int
    lib.dsv_accept_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.dsv_accept_workspace_bytes.restype = ctypes.c_size_t
    lib.dsv_accept.argtypes = [i32, i32, i32, i32] + [P] * 10 + [i32, i32] + [P, P, P, ctypes.c_size_t, P, P]
    lib.dsv_accept.restype = ctypes.c_int
    lib.dsv_accept_sample_workspace_bytes.argtypes = [i32, i32, i32]
    lib.dsv_accept_sample_workspace_bytes.restype = ctypes.c_size_t
    lib.dsv_accept_sample.argtypes = [i32, i32, i32, i32, P, ctypes.c_float] + [P] * 11 + [ctypes.c_size_t, P, P]
    lib.dsv_accept_sample.restype = ctypes.c_int
    lib.dsv_draft_features_workspace_bytes.argtypes = [ctypes.c_int64, i32]
    lib.dsv_draft_features_workspace_bytes.restype = ctypes.c_size_t
    lib.dsv_draft_features.argtypes = [ctypes.c_int64, i32, P, P, P, ctypes.c_size_t, P, P]
    lib.dsv_draft_features.restype = ctypes.c_int
    u64 = ctypes.c_uint64
    lib.dsv_philox_uniforms.argtypes = [u64, u64, u64, u64, ctypes.c_int64, P, P]
    lib.dsv_philox_uniforms.restype = ctypes.c_int
    lib.dsv_probe_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.dsv_probe_stream_read.restype = ctypes.c_int
    if lib.dsv_attn_args_size() != ctypes.sizeof(AttnArgs):
        raise ImportError("dsv_attn_args layout mismatch between include/dsv.h and the binding")
    _lib = lib
    return lib


def status_string(code: int) -> str:
    try:
        return load().dsv_status_string(code).decode()
    except ImportError:
        return f"status {code}"


def check(code: int, what: str):
    if code != 0:
        raise DsvError(code, what)
