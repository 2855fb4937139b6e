"""Device placement of a synthetic batch for the HIP library (no arithmetic).

Copies the bytes of a ``workloads.Batch`` to the GPU, pre-fills output buffers
with NaN payloads, and builds the library's ``Problem`` and ``Ragged``
descriptors over the flat buffers with the batch's layouts.
"""
from __future__ import annotations

import numpy as np
import torch

import variable_length_attention_ragged_amd as va

from . import F32_OUT_NAN, OUT_NAN, TORCH_DTYPE, Batch

OUTPUTS = ("o", "lse", "dq", "dk", "dv")


class DeviceBatch:
    """``scaled_offsets``: pass each tensor's offsets as int32 row numbers times
    a multiplier (its token stride) instead of int64 element offsets; tensors
    on one side (query or key) whose rows start at the same numbers share one
    row array."""

    GUARD_BITS = 0x5AA5   # canary pattern of the guard bands (16-bit words)

    def __init__(self, batch: Batch, device="cuda", with_grad: bool | None = None,
                 scaled_offsets: bool = False, guard_elems: int = 0):
        self.batch = batch
        self.device = device
        self.scaled_offsets = scaled_offsets
        # guard_elems > 0: every output buffer sits between two bands of that
        # many elements holding GUARD_BITS (see guards_intact)
        self.guard_elems = guard_elems
        self.guarded = {}
        with_grad = ("do" in batch.data) if with_grad is None else with_grad
        self.flat = {}
        for n in ("q", "k", "v", "do"):
            if n in batch.data:
                self.flat[n] = torch.from_numpy(batch.data[n].view(np.int16)).to(device) \
                    .view(TORCH_DTYPE[batch.dtype])
        names = ("o", "lse") + (("dq", "dk", "dv") if with_grad else ())
        for n in names:
            self.flat[n] = self.fresh_output(n)
        self.ragged = {n: torch.from_numpy(lay.ragged.astype(np.int64)).to(device)
                       for n, lay in batch.layouts.items()}
        self.rows = {}
        self.multiplier = {n: lay.stride_t for n, lay in batch.layouts.items()}
        if scaled_offsets:
            shared = {}
            for n, lay in batch.layouts.items():
                key = tuple(int(x) for x in lay.start_rows)
                if key not in shared:
                    shared[key] = torch.from_numpy(
                        np.asarray(lay.start_rows, dtype=np.int32)).to(device)
                self.rows[n] = shared[key]
        self.cu_q = torch.from_numpy(batch.cu_q).to(device)
        self.cu_kv = torch.from_numpy(batch.cu_kv).to(device)
        self.policy = None if batch.policy is None else torch.from_numpy(batch.policy).to(device)
        self.qco = None if batch.q_causal_offset is None else \
            torch.from_numpy(batch.q_causal_offset).to(device)
        self.problem = va.Problem(self.cu_q, self.cu_kv, batch.h_q, batch.h_kv, batch.dim,
                                  batch.scale, self.policy, batch.default_policy, self.qco,
                                  None if batch.window is None else batch.window.tolist(),
                                  TORCH_DTYPE[batch.dtype])
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def fresh_output(self, n: str) -> torch.Tensor:
        lay = self.batch.layouts[n]
        g = self.guard_elems
        if n == "lse":
            buf = torch.full((lay.span + 2 * g,), (self.GUARD_BITS << 16) | self.GUARD_BITS,
                             dtype=torch.int32, device=self.device)
            buf[g:g + lay.span] = F32_OUT_NAN - (1 << 32) if F32_OUT_NAN >= 1 << 31 else F32_OUT_NAN
            self.guarded[n] = buf
            return buf[g:g + lay.span].view(torch.float32)
        buf = torch.full((lay.span + 2 * g,), self.GUARD_BITS, dtype=torch.int16,
                         device=self.device)
        out = OUT_NAN[self.batch.dtype]
        buf[g:g + lay.span] = out - (1 << 16) if out >= 1 << 15 else out
        self.guarded[n] = buf
        return buf[g:g + lay.span].view(TORCH_DTYPE[self.batch.dtype])

    def guards_intact(self) -> dict:
        """Per output buffer: True if both guard bands still hold the canary."""
        g = self.guard_elems
        res = {}
        for n, buf in self.guarded.items():
            h = buf.cpu().numpy()
            word = (self.GUARD_BITS << 16) | self.GUARD_BITS if n == "lse" else self.GUARD_BITS
            band = np.concatenate([h[:g], h[h.size - g:]]).view(
                np.uint32 if n == "lse" else np.uint16)
            res[n] = bool(np.all(band == word))
        return res

    def rag(self, n: str) -> va.Ragged:
        lay = self.batch.layouts[n]
        flat = self.flat[n]
        if n == "lse":
            view = torch.as_strided(flat, (lay.rows, lay.heads), (lay.stride_t, lay.stride_h))
        else:
            view = torch.as_strided(flat, (lay.rows, lay.heads, lay.dim),
                                    (lay.stride_t, lay.stride_h, 1))
        if self.scaled_offsets:
            return va.Ragged(view, None, span=lay.span, scaled=self.rows[n],
                             multiplier=self.multiplier[n])
        return va.Ragged(view, self.ragged[n], span=lay.span)

    def fwd(self, **kw):
        return va.varlen_attn_fwd(self.problem, self.rag("q"), self.rag("k"), self.rag("v"),
                                  self.rag("o"), self.rag("lse"), dev_status=self.status, **kw)

    def fwd_setup(self, **kw):
        return va.varlen_attn_fwd_setup(self.problem, self.rag("q"), self.rag("k"), self.rag("v"),
                                        self.rag("o"), self.rag("lse"), dev_status=self.status,
                                        **kw)

    def bwd(self, **kw):
        return va.varlen_attn_bwd(self.problem, self.rag("q"), self.rag("k"), self.rag("v"),
                                  self.rag("o"), self.rag("do"), self.rag("lse"), self.rag("dq"),
                                  self.rag("dk"), self.rag("dv"), dev_status=self.status, **kw)

    def bwd_setup(self, **kw):
        return va.varlen_attn_bwd_setup(self.problem, self.rag("q"), self.rag("k"), self.rag("v"),
                                        self.rag("o"), self.rag("do"), self.rag("lse"),
                                        self.rag("dq"), self.rag("dk"), self.rag("dv"),
                                        dev_status=self.status, **kw)

    def fwd_stage(self, name: str, **kw):
        return getattr(va, name)(self.problem, self.rag("q"), self.rag("k"), self.rag("v"),
                                 self.rag("o"), self.rag("lse"), dev_status=self.status, **kw)

    def bwd_stage(self, name: str, **kw):
        return getattr(va, name)(self.problem, self.rag("q"), self.rag("k"), self.rag("v"),
                                 self.rag("o"), self.rag("do"), self.rag("lse"), self.rag("dq"),
                                 self.rag("dk"), self.rag("dv"), dev_status=self.status, **kw)

    def fwd_layout(self):
        return va.varlen_attn_fwd_workspace_layout(self.problem, self.rag("o"))

    def bwd_layout(self):
        return va.varlen_attn_bwd_workspace_layout(self.problem, self.rag("lse"), self.rag("dq"),
                                                   self.rag("dk"))

    def host(self, n: str) -> np.ndarray:
        """Raw host copy: uint16 bit patterns for 16-bit buffers, float32 for LSE."""
        t = self.flat[n]
        if t.dtype in (torch.bfloat16, torch.float16):
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
