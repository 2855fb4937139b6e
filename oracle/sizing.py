"""Oracle of buffer spans: how many elements a strided view can touch.

TEST INFRASTRUCTURE (see ``oracle/attention.py``).  The definition is the
literal one: one past the largest element offset any index of the view
reaches.  cudnn-frontend PR #462 ("Root cause", "The fix (commit 1)") sizes
ragged intermediates from every axis instead of from the token stride alone;
its head-major stats example is a [h, t] tensor with token stride 1, where the
token-stride-only size falls short by a factor h_q.
"""
from __future__ import annotations

import itertools


def span_by_enumeration(shape, strides) -> int:
    """1 + max over every index of sum(index * stride); 0 for an empty view."""
    if any(n == 0 for n in shape):
        return 0
    best = 0
    for idx in itertools.product(*[range(n) for n in shape]):
        best = max(best, sum(i * s for i, s in zip(idx, strides)))
    return best + 1


def span_of_extremes(shape, strides) -> int:
    """Same quantity for non-negative strides, reached at the last index."""
    return sum((n - 1) * s for n, s in zip(shape, strides)) + 1
