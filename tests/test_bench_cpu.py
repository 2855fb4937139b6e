"""The benchmark's work count against the oracle's mask (no GPU needed)."""
from __future__ import annotations

import numpy as np
import pytest

import bench
import oracle
import workloads


@pytest.mark.parametrize("seed,qco,window", [(700, False, None), (701, True, None),
                                             (702, False, "random"), (703, True, "random"),
                                             (704, True, "random")])
def test_pairs_per_head_counts_the_oracle_mask(seed, qco, window):
    batch = workloads.random_batch(seed, batch=8, max_len=90, q_causal_offset=qco,
                                   window=window, with_grad=False)
    prob, t = oracle.from_batch(batch)
    got = bench.pairs_per_head(batch)
    for b in range(batch.batch):
        info = oracle.sequence_info(prob, [], [], b)
        if info.lq <= 0 or info.lk <= 0:
            assert got[b] == 0
            continue
        mask = oracle.attention.allowed(info, np.arange(info.lq), np.arange(info.lk))
        assert got[b] == int(mask.sum()), b


def test_bench_workloads_are_the_named_configurations():
    full = workloads.packed_causal()
    win = workloads.packed_causal_window()
    assert np.array_equal(full.lq, win.lq) and full.window is None
    assert win.window.tolist() == [[-1, -1], [1024, 0], [-1, -1]]
    # the window removes pairs of rows more than 1024 keys past their sequence start
    assert bench.pairs_per_head(win).sum() < bench.pairs_per_head(full).sum()


def test_long_context_pairs_match_the_closed_form():
    # Each document's two 4096-row chunks start at absolute keys 4096 and
    # 61440; row i of a chunk at offset o sees keys 0 .. o + i, so the chunk
    # contributes sum_{i<4096} (o + 1 + i) pairs per head.
    batch = workloads.long_context_cp(with_grad=False)
    per_chunk = {o: 4096 * (o + 1) + 4095 * 4096 // 2 for o in (4096, 61440)}
    assert per_chunk == {4096: 25_167_872, 61440: 260_048_896}
    assert bench.pairs_per_head(batch).tolist() == [per_chunk[4096], per_chunk[61440]] * 2
    assert int(bench.pairs_per_head(batch).sum()) == 570_433_536


def test_every_bench_workload_resolves_with_its_passes():
    for name, (fn, desc, passes) in bench.WORKLOADS.items():
        assert callable(getattr(workloads, fn)), name
        assert passes in ("fwd", "fwd+bwd") and desc, name
    # the mixed-policy configuration is defined as a forward-only launch
    assert bench.WORKLOADS["mixed_policy"][2] == "fwd"
    assert bench.WORKLOADS["packed_causal"][2] == "fwd+bwd"


def test_kernel_fingerprint_ignores_comments_but_not_code():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no overflow\n check */\n}\n"
    b = "int f(int x) {\n    return 2 * x;\n}"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench._code_tokens(a) == bench._code_tokens(b)
    assert bench._code_tokens(a) != bench._code_tokens(c)
    # the recorded traffic is looked up under the current sources' fingerprint
    assert len(bench.kernel_fingerprint()) == 64
