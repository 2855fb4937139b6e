"""The workspace-free forward (varlen_attn_fwd_noalloc) against varlen_attn_fwd.

Callers that cannot allocate (graph capture, serving loops) get the forward
with the library's static per-GPU workspace.  Two calls in a row, the second
on a smaller problem (so stale metadata of the first call sits in the shared
array), each give bit-identical O, LSE and status to varlen_attn_fwd with its
own workspace, and match the oracle.
"""
from __future__ import annotations

import pytest
import torch

import workloads
from tests.gpu_common import check_forward, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import variable_length_attention_ragged_amd as va
    va.lib()


def _pair(batch):
    from workloads.device import DeviceBatch
    return DeviceBatch(batch, with_grad=False), DeviceBatch(batch, with_grad=False)


def test_noalloc_forward_matches_workspace_forward_twice():
    import variable_length_attention_ragged_amd as va
    big = workloads.random_batch(950, batch=40, max_len=700, h_q=4, h_kv=2, dim=128,
                                 window="random", q_causal_offset=True, with_grad=False)
    small = workloads.random_batch(951, batch=3, max_len=90, h_q=2, h_kv=1, dim=64,
                                   with_grad=False)
    for name, batch in (("big", big), ("small", small)):
        say(f"[noalloc] {name}: B={batch.batch} lq={int(batch.lq.sum())}")
        ref, na = _pair(batch)
        ref.fwd()
        va.varlen_attn_fwd_noalloc(na.problem, na.rag("q"), na.rag("k"), na.rag("v"),
                                   na.rag("o"), na.rag("lse"), dev_status=na.status)
        torch.cuda.synchronize()
        assert int(na.status.item()) == int(ref.status.item())
        for n, view in (("o", torch.int16), ("lse", torch.int32)):
            assert torch.equal(na.flat[n].view(view), ref.flat[n].view(view)), (name, n)
        check_forward(batch, na)


def test_noalloc_forward_refuses_oversized_problem():
    import variable_length_attention_ragged_amd as va
    from variable_length_attention_ragged_amd import _binding as B
    batch = workloads.random_batch(952, batch=30000, max_len=1, max_gap=0, token_gaps=False,
                                   with_grad=False)
    assert min(batch.layouts[n].rows for n in ("q", "k", "o")) > 0
    na, _ = _pair(batch)
    with pytest.raises(va.VarlenAttnError) as e:
        va.varlen_attn_fwd_noalloc(na.problem, na.rag("q"), na.rag("k"), na.rag("v"),
                                   na.rag("o"), na.rag("lse"), dev_status=na.status)
    assert e.value.code == B.ERR_SCRATCH
