"""ctypes binding of libvarlen_attn.so (argument marshalling only).

Mirrors include/varlen_attn.h.  Every computation runs in the library's HIP
kernels; this module only turns torch tensors into the plain pointers, sizes
and strides of the C ABI.  It refuses to work without the built library: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# VARLEN_ATTN_LIBRARY names another build of the same library (the host-code
# sanitizer build the CPU tests load); by default the in-tree one.
LIB_PATH = os.environ.get("VARLEN_ATTN_LIBRARY") or os.path.join(HERE, "libvarlen_attn.so")

# host return codes
OK = 0
ERR_NULL, ERR_BATCH, ERR_HEAD_DIM, ERR_HEADS, ERR_ALIGN, ERR_STRIDE = 1, 2, 3, 4, 5, 6
ERR_SPAN, ERR_WORKSPACE, ERR_POLICY, ERR_SCALE, ERR_HIP = 7, 8, 9, 10, 11
ERR_OFFSETS, ERR_WINDOW, ERR_DTYPE, ERR_SCRATCH = 12, 13, 14, 15
NOALLOC_SCRATCH_BYTES = 4 << 20
# element types of the 16-bit tensors
BF16, F16 = 0, 1
# mask policies
PADDING, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT = 0, 1, 2
# device status bits
ST_NEG_LENGTH, ST_BAD_OFFSET, ST_OUT_OF_SPAN, ST_BAD_POLICY, ST_LIST_OVERFLOW = 1, 2, 4, 8, 16
ST_KV_OVERLAP = 32


class varlen_attn_tensor(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("span_elems", c_int64), ("stride_t", c_int64),
                ("stride_h", c_int64), ("ragged", c_void_p), ("ragged_scaled", c_void_p),
                ("ragged_multiplier", c_int64)]


class varlen_attn_problem(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("h_q", c_int32), ("h_kv", c_int32), ("head_dim", c_int32),
                ("scale", c_float), ("cu_seqlens_q", c_void_p), ("cu_seqlens_kv", c_void_p),
                ("mask_policy", c_void_p), ("default_policy", c_int32),
                ("q_causal_offset", c_void_p), ("window_size", c_void_p), ("dtype", c_int32)]


class varlen_attn_layout(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in (
        "total_bytes", "counters_offset", "header_offset", "seq_offset", "seq_i64_offset",
        "fwd_tiles_offset", "fwd_tiles_capacity", "bwd_tiles_offset", "bwd_tiles_capacity",
        "members_offset", "scratch_offset", "delta_offset", "delta_elems", "lse_term_offset")] + \
        [(n, c_int32) for n in ("fwd_block_m", "fwd_block_n", "bwd_block_m", "bwd_block_n")]


class LibraryMissing(RuntimeError):
    pass


class VarlenAttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} (code {code})")
        self.code = code


_lib = None

_T = POINTER(varlen_attn_tensor)
_P = POINTER(varlen_attn_problem)
_L = POINTER(varlen_attn_layout)

_SIGNATURES = {
    "varlen_attn_fwd_workspace_layout": [_P, _T, _L],
    "varlen_attn_bwd_workspace_layout": [_P, _T, _T, _T, _L],
    "varlen_attn_fwd_workspace_size": [_P, _T, POINTER(c_size_t)],
    "varlen_attn_bwd_workspace_size": [_P, _T, _T, _T, POINTER(c_size_t)],
    "varlen_attn_fwd": [_P, _T, _T, _T, _T, _T, c_void_p, c_size_t, c_void_p, c_void_p],
    "varlen_attn_fwd_setup": [_P, _T, _T, _T, _T, _T, c_void_p, c_size_t, c_void_p, c_void_p],
    "varlen_attn_fwd_noalloc": [_P, _T, _T, _T, _T, _T, c_void_p, c_void_p],
    "varlen_attn_bwd": [_P, _T, _T, _T, _T, _T, _T, _T, _T, _T, c_void_p, c_size_t, c_void_p,
                        c_void_p],
    "varlen_attn_bwd_setup": [_P, _T, _T, _T, _T, _T, _T, _T, _T, _T, c_void_p, c_size_t,
                              c_void_p, c_void_p],
    "varlen_attn_fwd_attention": [_P, _T, _T, _T, _T, _T, c_void_p, c_size_t, c_void_p,
                                  c_void_p],
    "varlen_attn_bwd_dkdv": [_P, _T, _T, _T, _T, _T, _T, _T, _T, _T, c_void_p, c_size_t,
                             c_void_p, c_void_p],
    "varlen_attn_bwd_dq": [_P, _T, _T, _T, _T, _T, _T, _T, _T, _T, c_void_p, c_size_t,
                           c_void_p, c_void_p],
    "varlen_attn_status_string": [c_int],
}


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises LibraryMissing if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} is missing: build it with "
                "`python -m variable_length_attention_ragged_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = c_char_p if name == "varlen_attn_status_string" else c_int
        _lib = l
    return _lib


def exported_symbols() -> list:
    return list(_SIGNATURES)


def status_string(code: int) -> str:
    return lib().varlen_attn_status_string(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != OK:
        raise VarlenAttnError(code, what)


def raw_call(name: str, *args) -> int:
    """Call an entry point with already-marshalled ctypes arguments."""
    return getattr(lib(), name)(*args)
