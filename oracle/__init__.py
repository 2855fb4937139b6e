"""CPU oracle for ragged (THD) scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Plain fp64 numpy definitions of what the HIP path
computes, used to check it.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import anything from this
package; the product path (the C-ABI library and its Python binding) never
does and shares no code with it.

Modules:
  attention  forward / backward definitions, per-sequence validation
  worklist   expected outputs of the on-device setup step
  sizing     the span of a strided view, by definition
"""
from .attention import (CAUSAL_BOTTOM_RIGHT, CAUSAL_TOP_LEFT, PADDING, ST_BAD_OFFSET,
                        ST_BAD_POLICY, ST_KV_OVERLAP, ST_LIST_OVERFLOW, ST_NEG_LENGTH,
                        ST_OUT_OF_SPAN, Problem, Tensor, backward, bf16_bits_to_f64,
                        bits_to_f64, forward, forward_rows, kv_overlap, sequence_info)
from . import sizing, worklist

__all__ = [
    "CAUSAL_BOTTOM_RIGHT", "CAUSAL_TOP_LEFT", "PADDING", "ST_BAD_OFFSET", "ST_BAD_POLICY",
    "ST_KV_OVERLAP", "kv_overlap", "ST_LIST_OVERFLOW", "ST_NEG_LENGTH", "ST_OUT_OF_SPAN", "Problem", "Tensor", "backward",
    "bf16_bits_to_f64", "bits_to_f64", "forward", "forward_rows", "sequence_info", "sizing", "worklist",
    "from_batch",
]


def from_batch(batch, outputs: dict | None = None):
    """Oracle Problem and Tensors from a ``workloads.Batch``.

    ``outputs`` maps o/lse/dq/dk/dv to the flat output buffers as they were
    before the call (default: the batch's pre-filled NaN buffers)."""
    import numpy as np
    import workloads

    prob = Problem(batch.h_q, batch.h_kv, batch.dim, batch.scale, batch.cu_q, batch.cu_kv,
                   batch.policy, batch.default_policy, batch.q_causal_offset, batch.window)
    t = {}
    for n, lay in batch.layouts.items():
        if n in batch.data:
            data = batch.data[n]
        elif outputs is not None and n in outputs:
            data = outputs[n]
        else:
            data = workloads.out_buffer(lay, "f32" if n == "lse" else batch.dtype)
        t[n] = Tensor(np.asarray(data), lay.stride_t, lay.stride_h, lay.ragged, lay.heads,
                      lay.dim, batch.dtype)
    return prob, t
