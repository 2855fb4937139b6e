"""Ragged (THD) variable-length attention for MI355X (gfx950).

Python side of the C-ABI library ``libvarlen_attn.so``: the functions below
marshal torch tensors (device memory and the current stream) into the C entry
points of the same names; every step of the computation runs in the library's
HIP kernels.  A tensor argument is a ``Ragged``: a strided view
``[rows, heads, dim]`` (LSE: ``[rows, heads]``) over the caller's buffer plus a
device int64 array of ``batch + 1`` element offsets (one per sequence, entry
``batch`` past-the-end), relative to the view's first element.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _binding as _b
from ._binding import (CAUSAL_BOTTOM_RIGHT, CAUSAL_TOP_LEFT, PADDING, ST_BAD_OFFSET,
                       ST_BAD_POLICY, ST_LIST_OVERFLOW, ST_NEG_LENGTH, ST_OUT_OF_SPAN,
                       LibraryMissing, VarlenAttnError, exported_symbols, lib, status_string,
                       varlen_attn_layout, varlen_attn_problem, varlen_attn_tensor)

__all__ = [
    "Ragged", "Problem", "varlen_attn_fwd", "varlen_attn_bwd", "varlen_attn_fwd_setup",
    "varlen_attn_bwd_setup", "varlen_attn_fwd_attention",
    "varlen_attn_bwd_dkdv", "varlen_attn_bwd_dq", "varlen_attn_fwd_workspace_layout",
    "varlen_attn_bwd_workspace_layout", "varlen_attn_fwd_workspace_size",
    "varlen_attn_bwd_workspace_size", "status_string", "view_span", "PADDING",
    "CAUSAL_TOP_LEFT", "CAUSAL_BOTTOM_RIGHT", "ST_NEG_LENGTH", "ST_BAD_OFFSET",
    "ST_OUT_OF_SPAN", "ST_BAD_POLICY", "ST_LIST_OVERFLOW", "VarlenAttnError", "LibraryMissing",
    "lib", "exported_symbols",
]


def view_span(t: torch.Tensor) -> int:
    """Elements a strided view can reach: every axis counts (not only the
    token axis), so a head-major [h, t] view spans h*t elements."""
    if t.numel() == 0:
        return 0
    return sum((n - 1) * s for n, s in zip(t.shape, t.stride())) + 1


@dataclass
class Ragged:
    """A ragged tensor: strided view + device offsets [batch+1] of each
    sequence's row 0.

    The offsets are either int64 element offsets (``ragged``) or int32
    values in units of ``multiplier`` elements (``scaled``), e.g. one padded
    cu_seqlens array shared by every tensor with multiplier = its token
    stride; give one of them.  ``span`` overrides the addressable element
    count (default: the view's span); use it when the caller's allocation
    extends past the view."""

    view: torch.Tensor
    ragged: torch.Tensor | None = None
    span: int | None = None
    scaled: torch.Tensor | None = None
    multiplier: int = 0

    def c(self) -> varlen_attn_tensor:
        v = self.view
        if self.ragged is not None and self.ragged.dtype != torch.int64:
            raise TypeError("ragged offsets must be int64")
        if self.scaled is not None and self.scaled.dtype != torch.int32:
            raise TypeError("scaled offsets must be int32")
        st, sh = v.stride(0), v.stride(1)
        if v.dim() == 3 and v.stride(2) != 1:
            raise ValueError("the innermost (head_dim) stride must be 1")
        return varlen_attn_tensor(
            v.data_ptr(), self.span if self.span is not None else view_span(v), st, sh,
            self.ragged.data_ptr() if self.ragged is not None else None,
            self.scaled.data_ptr() if self.scaled is not None else None,
            self.multiplier if self.scaled is not None else 0)


_DTYPES = {torch.bfloat16: _b.BF16, torch.float16: _b.F16}


@dataclass
class Problem:
    """Lengths, heads and mask policy (see include/varlen_attn.h)."""

    cu_seqlens_q: torch.Tensor            # int32 [batch+1], device
    cu_seqlens_kv: torch.Tensor           # int32 [batch+1], device
    h_q: int
    h_kv: int
    head_dim: int
    scale: float | None = None            # default 1/sqrt(head_dim)
    mask_policy: torch.Tensor | None = None   # int8 [batch], device
    default_policy: int = PADDING
    q_causal_offset: torch.Tensor | None = None  # int32 [batch], device
    # (left, right) per policy in the order padding, top-left, bottom-right;
    # -1 unbounded.  Host values (six ints, flat or 3 x 2).
    window_size: object | None = None
    dtype: torch.dtype = torch.bfloat16   # of Q, K, V, O, dO, dQ, dK, dV (bf16 or fp16)

    def c(self) -> varlen_attn_problem:
        def ptr(t):
            return None if t is None else t.data_ptr()
        batch = self.cu_seqlens_q.numel() - 1
        scale = self.scale if self.scale is not None else self.head_dim ** -0.5
        win = None
        if self.window_size is not None:
            vals = [int(x) for row in self.window_size for x in
                    (row if hasattr(row, "__len__") else (row,))]
            if len(vals) != 6:
                raise ValueError("window_size needs (left, right) for each of the 3 policies")
            win = (ctypes.c_int32 * 6)(*vals)
        if self.dtype not in _DTYPES:
            raise TypeError("dtype must be torch.bfloat16 or torch.float16")
        prob = varlen_attn_problem(batch, self.h_q, self.h_kv, self.head_dim, scale,
                                   ptr(self.cu_seqlens_q), ptr(self.cu_seqlens_kv),
                                   ptr(self.mask_policy), self.default_policy,
                                   ptr(self.q_causal_offset),
                                   None if win is None else ctypes.addressof(win),
                                   _DTYPES[self.dtype])
        prob._window_keepalive = win  # the library reads it during the call
        return prob


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def varlen_attn_fwd_workspace_layout(p: Problem, o: Ragged) -> varlen_attn_layout:
    L = varlen_attn_layout()
    _b._check(lib().varlen_attn_fwd_workspace_layout(ctypes.byref(p.c()), ctypes.byref(o.c()),
                                                     ctypes.byref(L)), "fwd workspace layout")
    return L


def varlen_attn_bwd_workspace_layout(p: Problem, lse: Ragged, dq: Ragged,
                                     dk: Ragged) -> varlen_attn_layout:
    L = varlen_attn_layout()
    _b._check(lib().varlen_attn_bwd_workspace_layout(
        ctypes.byref(p.c()), ctypes.byref(lse.c()), ctypes.byref(dq.c()), ctypes.byref(dk.c()),
        ctypes.byref(L)), "bwd workspace layout")
    return L


def varlen_attn_fwd_workspace_size(p: Problem, o: Ragged) -> int:
    n = ctypes.c_size_t(0)
    _b._check(lib().varlen_attn_fwd_workspace_size(ctypes.byref(p.c()), ctypes.byref(o.c()),
                                                   ctypes.byref(n)), "fwd workspace size")
    return n.value


def varlen_attn_bwd_workspace_size(p: Problem, lse: Ragged, dq: Ragged, dk: Ragged) -> int:
    n = ctypes.c_size_t(0)
    _b._check(lib().varlen_attn_bwd_workspace_size(
        ctypes.byref(p.c()), ctypes.byref(lse.c()), ctypes.byref(dq.c()), ctypes.byref(dk.c()),
        ctypes.byref(n)), "bwd workspace size")
    return n.value


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _check_dtypes(p, halves, lse):
    """The 16-bit tensors must have the problem's element type, LSE fp32."""
    for r in halves:
        if r.view.dtype != p.dtype:
            raise TypeError(f"tensor dtype {r.view.dtype} differs from the problem's {p.dtype}")
    if lse.view.dtype != torch.float32:
        raise TypeError("lse must be float32")


def _fwd_call(name, p, q, k, v, o, lse, workspace, dev_status, stream):
    _check_dtypes(p, (q, k, v, o), lse)
    if workspace is None:
        workspace = _workspace(varlen_attn_fwd_workspace_size(p, o), o.view.device)
    code = getattr(lib(), name)(
        ctypes.byref(p.c()), ctypes.byref(q.c()), ctypes.byref(k.c()), ctypes.byref(v.c()),
        ctypes.byref(o.c()), ctypes.byref(lse.c()), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _ptr(dev_status), _stream(stream))
    _b._check(code, name)
    return workspace


def varlen_attn_fwd(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged, lse: Ragged, *,
                    workspace: torch.Tensor | None = None, dev_status: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Enqueue the forward; writes o and lse in place.  Returns the workspace
    (allocated with torch if not given).  Raises VarlenAttnError on a host
    error code (nothing enqueued)."""
    return _fwd_call("varlen_attn_fwd", p, q, k, v, o, lse, workspace, dev_status, stream)


def varlen_attn_fwd_setup(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged, lse: Ragged,
                          *, workspace: torch.Tensor | None = None,
                          dev_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Enqueue only the setup kernel of a forward call."""
    return _fwd_call("varlen_attn_fwd_setup", p, q, k, v, o, lse, workspace, dev_status, stream)


def _bwd_call(name, p, q, k, v, o, dout, lse, dq, dk, dv, workspace, dev_status, stream):
    _check_dtypes(p, (q, k, v, o, dout, dq, dk, dv), lse)
    if workspace is None:
        workspace = _workspace(varlen_attn_bwd_workspace_size(p, lse, dq, dk), dq.view.device)
    code = getattr(lib(), name)(
        ctypes.byref(p.c()), ctypes.byref(q.c()), ctypes.byref(k.c()), ctypes.byref(v.c()),
        ctypes.byref(o.c()), ctypes.byref(dout.c()), ctypes.byref(lse.c()),
        ctypes.byref(dq.c()), ctypes.byref(dk.c()), ctypes.byref(dv.c()), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _ptr(dev_status), _stream(stream))
    _b._check(code, name)
    return workspace


def varlen_attn_bwd(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged, dout: Ragged,
                    lse: Ragged, dq: Ragged, dk: Ragged, dv: Ragged, *,
                    workspace: torch.Tensor | None = None, dev_status: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Enqueue the backward; writes dq, dk, dv in place."""
    return _bwd_call("varlen_attn_bwd", p, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                     dev_status, stream)


def varlen_attn_bwd_setup(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged, dout: Ragged,
                          lse: Ragged, dq: Ragged, dk: Ragged, dv: Ragged, *,
                          workspace: torch.Tensor | None = None,
                          dev_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Enqueue only the setup kernel of a backward call."""
    return _bwd_call("varlen_attn_bwd_setup", p, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                     dev_status, stream)


def varlen_attn_fwd_attention(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged,
                              lse: Ragged, *, workspace: torch.Tensor,
                              dev_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Enqueue only the forward kernel (the workspace must hold this call's setup)."""
    return _fwd_call("varlen_attn_fwd_attention", p, q, k, v, o, lse, workspace, dev_status,
                     stream)


def _bwd_stage(name):
    def run(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged, dout: Ragged, lse: Ragged,
            dq: Ragged, dk: Ragged, dv: Ragged, *, workspace: torch.Tensor,
            dev_status: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        return _bwd_call(name, p, q, k, v, o, dout, lse, dq, dk, dv, workspace, dev_status,
                         stream)
    run.__name__ = name
    run.__doc__ = f"Enqueue only {name} (the workspace must hold this call's setup)."
    return run


varlen_attn_bwd_dkdv = _bwd_stage("varlen_attn_bwd_dkdv")
varlen_attn_bwd_dq = _bwd_stage("varlen_attn_bwd_dq")
