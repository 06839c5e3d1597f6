"""ctypes view of the C ABI declared in ``include/fa.h``.

Argument marshalling only: the structs below mirror ``fa_prefill_params`` and
``fa_decode_params`` field for field, and the functions are the library's own
exports.  The shared library is loaded from the package directory
(``libfa.so``, built by ``make -C transformer_attention_flashattention_amd/csrc``);
if it is missing, importing fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2
FA_KV_PLAIN = 0
FA_KV_FP8_E4M3 = 1

# Every symbol include/fa.h declares.
EXPORTS = ("fa_prefill_fwd", "fa_prefill_workspace_size", "fa_decode_workspace_size",
           "fa_decode_fwd", "fa_decode_fwd_noalloc", "fa_status_str", "fa_last_error_message",
           "fa_abi_version")
# bytes of the device array fa_decode_fwd_noalloc uses (FA_DECODE_NOALLOC_MAX_BYTES)
DECODE_NOALLOC_MAX_BYTES = 32 << 20

_i64x3 = ctypes.c_int64 * 3
_i64x2 = ctypes.c_int64 * 2


class PrefillParams(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("seqlen_k", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("seqlens_q", ctypes.c_void_p),
        ("seqlens_k", ctypes.c_void_p),
        ("q_stride", _i64x3),
        ("k_stride", _i64x3),
        ("v_stride", _i64x3),
        ("o_stride", _i64x3),
        ("alibi_slopes", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p),
        ("rope_sin", ctypes.c_void_p),
        ("rotary_dim", ctypes.c_int32),
        ("rope_max_pos", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
        ("attn_mask", ctypes.c_void_p),
        ("mask_stride", ctypes.c_int64 * 4),
    ]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("chunk_keys", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("reserved0", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("seqlens_k", ctypes.c_void_p),
        ("q_stride", _i64x2),
        ("k_stride", _i64x3),
        ("v_stride", _i64x3),
        ("o_stride", _i64x2),
        ("alibi_slopes", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("reserved1", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p),
        ("rope_sin", ctypes.c_void_p),
        ("rotary_dim", ctypes.c_int32),
        ("rope_max_pos", ctypes.c_int32),
    ]


class FAError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, func: str, message: str):
        self.status = status
        super().__init__(f"{func} -> {status_str(status)}: {message}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build it with "
            "`make -C transformer_attention_flashattention_amd/csrc` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_prefill_fwd.argtypes = [ctypes.POINTER(PrefillParams), ctypes.c_void_p]
    lib.fa_prefill_fwd.restype = ctypes.c_int
    lib.fa_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillParams),
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_prefill_workspace_size.restype = ctypes.c_int
    lib.fa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeParams),
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.fa_decode_workspace_size.restype = ctypes.c_int
    lib.fa_decode_fwd.argtypes = [ctypes.POINTER(DecodeParams), ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_void_p]
    lib.fa_decode_fwd.restype = ctypes.c_int
    lib.fa_decode_fwd_noalloc.argtypes = [ctypes.POINTER(DecodeParams), ctypes.c_void_p]
    lib.fa_decode_fwd_noalloc.restype = ctypes.c_int
    lib.fa_status_str.argtypes = [ctypes.c_int]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_error_message.argtypes = []
    lib.fa_last_error_message.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().fa_status_str(status).decode()


def last_error() -> str:
    return load().fa_last_error_message().decode()


def check(status: int, func: str) -> None:
    if status != FA_OK:
        raise FAError(status, func, last_error())


def prefill_fwd(params: PrefillParams, stream: int) -> int:
    return load().fa_prefill_fwd(ctypes.byref(params), ctypes.c_void_p(stream))


def prefill_workspace_size(params: PrefillParams) -> tuple:
    n = ctypes.c_size_t(0)
    st = load().fa_prefill_workspace_size(ctypes.byref(params), ctypes.byref(n))
    return st, n.value


def decode_workspace_size(params: DecodeParams) -> tuple:
    n = ctypes.c_size_t(0)
    st = load().fa_decode_workspace_size(ctypes.byref(params), ctypes.byref(n))
    return st, n.value


def decode_fwd(params: DecodeParams, workspace: int, workspace_bytes: int, stream: int) -> int:
    return load().fa_decode_fwd(ctypes.byref(params), ctypes.c_void_p(workspace),
                                ctypes.c_size_t(workspace_bytes), ctypes.c_void_p(stream))


def decode_fwd_noalloc(params: DecodeParams, stream: int) -> int:
    return load().fa_decode_fwd_noalloc(ctypes.byref(params), ctypes.c_void_p(stream))
