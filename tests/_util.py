"""Helpers shared by the tests (no attention arithmetic here)."""
from __future__ import annotations

import numpy as np

import workloads


def seq_rows(batch: workloads.Batch, name: str, flat: np.ndarray, b: int, length: int):
    """Dense [length, heads, dim] view of sequence b of a flat buffer, located
    with the input generator's layout (start row * stride), not the oracle's
    addressing code."""
    lay = batch.layouts[name]
    s = int(lay.start_rows[b])
    return lay.view(flat)[s:s + length]


def written_rows(batch: workloads.Batch, name: str, mask: np.ndarray) -> np.ndarray:
    """Rows of a buffer with at least one written element."""
    lay = batch.layouts[name]
    return np.nonzero(lay.view(mask).reshape(lay.rows, -1).any(axis=1))[0]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
