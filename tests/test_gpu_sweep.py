"""Seeded sweep of small random problems: HIP path vs the fp64 oracle.

Each case draws its own combination of the features the other GPU tests
exercise one or two at a time: batch and length mix (zero lengths,
cross-length sequences), head counts and GQA ratios, head_dim, element type,
per-sequence policies, q causal offsets, per-policy windows, token-stride
gaps, LSE layout, row-unit offsets with multipliers, shuffled
context-parallel chunks that alias key rows, and an occasional invalid
sequence.  Forward and backward at the plain bars (O 2e-2, LSE 1e-3,
gradients 5e-2), every element outside the written rows untouched.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_common import check_backward, check_forward, oracle_bwd, oracle_fwd, say

pytestmark = pytest.mark.gpu

HEADS = [(1, 1), (2, 1), (4, 2), (4, 4), (8, 2), (8, 1)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import variable_length_attention_ragged_amd as va
    va.lib()


def make_case(seed: int):
    rng = np.random.default_rng(seed)
    h_q, h_kv = HEADS[int(rng.integers(0, len(HEADS)))]
    dim = int(rng.choice([64, 128]))
    dtype = "f16" if rng.random() < 0.3 else "bf16"
    window = "random" if rng.random() < 0.35 else None
    if rng.random() < 0.3:
        b = workloads.aliased_batch(seed, docs=int(rng.integers(1, 4, endpoint=True)),
                                    max_doc=int(rng.integers(40, 400)),
                                    chunks=int(rng.integers(1, 3, endpoint=True)), h_q=h_q,
                                    h_kv=h_kv, dim=dim, dtype=dtype)
        if window is not None:
            b.window = workloads.random_window(rng, 100)
        kind = "aliased"
    else:
        max_len = int(rng.integers(1, 400, endpoint=True)) if rng.random() < 0.8 else \
            int(rng.integers(400, 900, endpoint=True))
        b = workloads.random_batch(seed, batch=int(rng.integers(1, 8, endpoint=True)),
                                   max_len=max_len, h_q=h_q,
                                   h_kv=h_kv, dim=dim, cross=bool(rng.random() < 0.7),
                                   q_causal_offset=bool(rng.random() < 0.4), window=window,
                                   dtype=dtype)
        kind = "random"
    if b.batch > 1 and rng.random() < 0.15:
        pol = (b.policy.copy() if b.policy is not None
               else np.full(b.batch, b.default_policy, np.int8))
        pol[int(rng.integers(0, b.batch))] = 7       # invalid: skipped with a status bit
        b.policy = pol
    scaled = bool(rng.random() < 0.2)
    return b, kind, scaled


@pytest.mark.parametrize("seed", range(5000, 5200))
def test_random_sweep(seed):
    from workloads.device import DeviceBatch
    batch, kind, scaled = make_case(seed)
    say(f"[sweep {seed}] {kind} B={batch.batch} H={batch.h_q}/{batch.h_kv} D={batch.dim} "
        f"{batch.dtype} window={'-' if batch.window is None else batch.window.tolist()} "
        f"scaled={scaled} lq={batch.lq.tolist()} lk={batch.lk.tolist()}")
    dev = DeviceBatch(batch, scaled_offsets=scaled)
    dev.fwd()
    torch.cuda.synchronize()
    fref = oracle_fwd(batch)
    check_forward(batch, dev, fref)
    dev.bwd()
    torch.cuda.synchronize()
    bref = oracle_bwd(batch)
    assert int(dev.status.item()) == fref["status"] | bref["status"]
    check_backward(batch, dev, bref)
