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
                       ST_BAD_POLICY, ST_KV_OVERLAP, ST_LIST_OVERFLOW, ST_NEG_LENGTH, ST_OUT_OF_SPAN,
                       LibraryMissing, VarlenAttnError, exported_symbols, lib, status_string,
                       varlen_attn_layout, varlen_attn_problem, varlen_attn_tensor)

__all__ = [
    "Ragged", "Problem", "varlen_attn_fwd", "varlen_attn_bwd", "varlen_attn_fwd_setup",
    "varlen_attn_bwd_setup", "varlen_attn_fwd_attention",
    "varlen_attn_bwd_dkdv", "varlen_attn_bwd_dq", "varlen_attn_fwd_workspace_layout",
    "varlen_attn_bwd_workspace_layout", "varlen_attn_fwd_workspace_size",
    "varlen_attn_bwd_workspace_size", "status_string", "view_span", "PADDING",
    "CAUSAL_TOP_LEFT", "CAUSAL_BOTTOM_RIGHT", "ST_NEG_LENGTH", "ST_BAD_OFFSET",
    "ST_OUT_OF_SPAN", "ST_BAD_POLICY", "ST_LIST_OVERFLOW", "ST_KV_OVERLAP", "VarlenAttnError", "LibraryMissing",
    "lib", "exported_symbols", "VarlenAttention", "varlen_attention", "varlen_attn_fwd_noalloc",
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


def varlen_attn_fwd_noalloc(p: Problem, q: Ragged, k: Ragged, v: Ragged, o: Ragged,
                            lse: Ragged, *, dev_status: torch.Tensor | None = None,
                            stream=None) -> None:
    """Enqueue the forward with the library's static per-GPU workspace instead
    of a workspace argument: nothing is allocated, here or in the library.
    Raises VarlenAttnError (code ERR_SCRATCH) if the problem needs more than
    that workspace holds."""
    _check_dtypes(p, (q, k, v, o), lse)
    code = lib().varlen_attn_fwd_noalloc(
        ctypes.byref(p.c()), ctypes.byref(q.c()), ctypes.byref(k.c()), ctypes.byref(v.c()),
        ctypes.byref(o.c()), ctypes.byref(lse.c()), _ptr(dev_status), _stream(stream))
    _b._check(code, "varlen_attn_fwd_noalloc")


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


# ------------------------------------------------------------------ autograd

def _rows_ragged(t: torch.Tensor, rows: torch.Tensor) -> Ragged:
    """A [rows, heads, dim] (or [rows, heads]) view whose sequences start at
    the int32 row numbers `rows`: the offsets are formed on the device as
    rows * stride_t (the library's scaled-offset form)."""
    return Ragged(t, None, scaled=rows, multiplier=t.stride(0))


class VarlenAttention(torch.autograd.Function):
    """Autograd over varlen_attn_fwd / varlen_attn_bwd.

    forward(q, k, v, problem, rows_q, rows_kv, lse_head_major, status) ->
    (o, lse).  q: [rows_q, h_q, D], k and v: [rows_kv, h_kv, D] (the
    problem's dtype, innermost stride 1); rows_q / rows_kv: device int32
    [batch+1] start rows of the sequences on each side (a padded cu_seqlens).
    o is a new [rows_q, h_q, D] tensor, lse a new fp32 [rows_q, h_q]
    (token-major) or a [rows_q, h_q] view of [h_q, rows_q] storage
    (head-major).  Rows outside every sequence are 0 in o, and their
    gradients are 0.  lse is not differentiable.  Every number comes from the
    library's kernels; this class allocates outputs and workspaces and
    passes pointers."""

    @staticmethod
    def forward(ctx, q, k, v, problem, rows_q, rows_kv, lse_head_major, status):
        o = torch.zeros_like(q, memory_format=torch.contiguous_format)
        if lse_head_major:
            lse = torch.zeros((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device).t()
        else:
            lse = torch.zeros(q.shape[:2], dtype=torch.float32, device=q.device)
        varlen_attn_fwd(problem, _rows_ragged(q, rows_q), _rows_ragged(k, rows_kv),
                        _rows_ragged(v, rows_kv), _rows_ragged(o, rows_q),
                        _rows_ragged(lse, rows_q), dev_status=status)
        ctx.save_for_backward(q, k, v, o, lse, rows_q, rows_kv)
        ctx.problem = problem
        ctx.status = status
        ctx.mark_non_differentiable(lse)
        ctx.set_materialize_grads(False)
        return o, lse

    @staticmethod
    def backward(ctx, grad_o, grad_lse):
        q, k, v, o, lse, rows_q, rows_kv = ctx.saved_tensors
        if grad_o is None:
            return (None,) * 8
        do = grad_o.contiguous()
        dq = torch.zeros_like(q, memory_format=torch.contiguous_format)
        dk = torch.zeros_like(k, memory_format=torch.contiguous_format)
        dv = torch.zeros_like(v, memory_format=torch.contiguous_format)
        varlen_attn_bwd(ctx.problem, _rows_ragged(q, rows_q), _rows_ragged(k, rows_kv),
                        _rows_ragged(v, rows_kv), _rows_ragged(o, rows_q),
                        _rows_ragged(do, rows_q), _rows_ragged(lse, rows_q),
                        _rows_ragged(dq, rows_q), _rows_ragged(dk, rows_kv),
                        _rows_ragged(dv, rows_kv), dev_status=ctx.status)
        return dq, dk, dv, None, None, None, None, None


def varlen_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     cu_seqlens_q: torch.Tensor, cu_seqlens_kv: torch.Tensor, *,
                     seq_rows_q: torch.Tensor | None = None,
                     seq_rows_kv: torch.Tensor | None = None,
                     mask_policy: torch.Tensor | None = None, default_policy: int = PADDING,
                     q_causal_offset: torch.Tensor | None = None, window_size=None,
                     scale: float | None = None, lse_head_major: bool = False,
                     status: torch.Tensor | None = None):
    """Differentiable ragged attention: returns (o, lse).

    cu_seqlens_q / cu_seqlens_kv: device int32 [batch+1] cumulative valid
    lengths.  seq_rows_q / seq_rows_kv: device int32 [batch+1] start row of
    each sequence in q (and o, dO, dQ) and in k, v (and dK, dV), i.e. the
    padded cu_seqlens; default: the cu_seqlens themselves (packed rows).
    The other arguments are those of ``Problem``; ``status`` (device int32
    [1]) receives the device status bits of both passes."""
    rows_q = cu_seqlens_q if seq_rows_q is None else seq_rows_q
    rows_kv = cu_seqlens_kv if seq_rows_kv is None else seq_rows_kv
    for t in (cu_seqlens_q, cu_seqlens_kv, rows_q, rows_kv):
        if t.dtype != torch.int32:
            raise TypeError("cu_seqlens and sequence start rows must be int32")
    problem = Problem(cu_seqlens_q, cu_seqlens_kv, q.shape[1], k.shape[1], q.shape[2], scale,
                      mask_policy, default_policy, q_causal_offset, window_size, q.dtype)
    return VarlenAttention.apply(q, k, v, problem, rows_q, rows_kv, lse_head_major, status)
