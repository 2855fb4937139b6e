"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: the worked layouts
printed on the pages (tests/golden/), PyTorch's own attention, mask and
log-sum-exp routines, closed forms, invariants and finite differences.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right, causal_upper_left

import oracle
import workloads
from tests._util import seq_rows, written_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _run_fwd(batch, outputs=None, **kw):
    prob, t = oracle.from_batch(batch, outputs)
    return oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], **kw)


# ----------------------------------------------------------------- worked example 1

def test_padded_thd_worked_example_addresses_bound_offsets():
    g = _golden("padded_thd_13row.json")
    batch = workloads.tiny_padded_thd(causal=False)
    assert list(batch.cu_q) == g["cu_seqlens"]
    start = batch.layouts["q"].start_rows
    assert list(start) == g["cu_seqlens_padded"]
    res = _run_fwd(batch)
    assert res["status"] == 0
    # rows written: exactly the valid ones; identifier rows untouched
    valid = [r for r in range(13) if r not in g["identifier_rows"]]
    assert list(written_rows(batch, "o", res["o_written"])) == valid
    o = batch.layouts["o"].view(res["o"])
    for r in g["identifier_rows"]:
        raw = batch.layouts["o"].view(workloads.out_buffer(batch.layouts["o"]))[r]
        assert np.all(np.isnan(o[r]))            # still the pre-fill payload
        assert np.all(raw == workloads.BF16_OUT_NAN)
    assert np.all(np.isfinite(o[valid]))         # NaN pads never reached a valid row
    # sequence 1 starts at row 4 (b), not at prefix(lens)[1] = 3 (identifier "1")
    assert int(batch.ragged("q")[1]) == g["sequence_1_start_row"] * batch.layouts["q"].stride_t


def test_padded_thd_worked_example_identifier_rows_do_not_matter():
    g = _golden("padded_thd_13row.json")
    batch = workloads.tiny_padded_thd(causal=True)
    base = _run_fwd(batch)
    # put large finite values into the identifier rows of Q/K/V: nothing changes
    for n in ("q", "k", "v"):
        v = batch.layouts[n].view(batch.data[n])
        for r in g["identifier_rows"]:
            v[r] = 0x4300  # bf16 128.0
    again = _run_fwd(batch)
    np.testing.assert_array_equal(again["o"][again["o_written"]], base["o"][base["o_written"]])
    # changing row 4 (first row of sequence 1) does change sequence 1's output
    kv = batch.layouts["k"].view(batch.data["k"])
    kv[g["sequence_1_start_row"]] = 0x4000  # 2.0
    third = _run_fwd(batch)
    o1 = seq_rows(batch, "o", third["o"], 1, 2)
    o1_base = seq_rows(batch, "o", base["o"], 1, 2)
    assert not np.allclose(o1, o1_base)


def test_prefix_of_lengths_addressing_is_the_defect():
    """The mis-derivation re-addresses sequence 1 at the identifier row 3; the
    NaN there poisons its output.  The oracle must not do that."""
    g = _golden("padded_thd_13row.json")
    batch = workloads.tiny_padded_thd(causal=False)
    prob, t = oracle.from_batch(batch)
    wrong_rows = np.asarray(g["cu_seqlens"], np.int64)
    for n in ("q", "k", "v", "o"):
        t[n].ragged = wrong_rows * t[n].stride_t
    res = oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])
    o = batch.layouts["o"].view(res["o"])
    assert np.isnan(o[3]).any() and g["prefix_of_lengths_start_row"] == 3


# ----------------------------------------------------------------- worked example 2

def _mixed_19(policies, start_rows, lengths, seed=7):
    n = len(lengths)
    return workloads.build("mixed19", seed, 2, 2, 16, lengths, lengths, start_rows, start_rows,
                           default_policy=0, policy=policies, q_rows=19, kv_rows=19)


def test_mixed_policy_equals_sum_of_two_single_policy_passes():
    g = _golden("mixed_policy_19row.json")
    one = g["single_call_reading"]
    pol = [1 if p == "causal" else 0 for p in one["policies"]]
    mixed = _mixed_19(pol, one["start_rows"], one["lengths"])

    def single_pass(cu, padded, policy):
        lens = np.diff(cu)
        b = workloads.build("pass", 7, 2, 2, 16, lens, lens, padded, padded, default_policy=policy,
                            q_rows=19, kv_rows=19)
        for n in ("q", "k", "v"):        # same 19-row buffers as the mixed call
            b.data[n] = mixed.data[n]
        zero_o = np.zeros(b.layouts["o"].span, np.uint16)          # pre-zeroed outputs
        zero_l = np.zeros(b.layouts["lse"].span, np.float32)
        return _run_fwd(b, {"o": zero_o, "lse": zero_l})

    c = single_pass(g["causal_pass"]["cu_seqlens"], g["causal_pass"]["cu_seqlens_padded"], 1)
    p = single_pass(g["padding_pass"]["cu_seqlens"], g["padding_pass"]["cu_seqlens_padded"], 0)
    zero_o = np.zeros(mixed.layouts["o"].span, np.uint16)
    m = _run_fwd(mixed, {"o": zero_o, "lse": np.zeros(mixed.layouts["lse"].span, np.float32)})
    assert m["status"] == c["status"] == p["status"] == 0
    np.testing.assert_array_equal(m["o"], c["o"] + p["o"])
    # the two passes write disjoint rows that together cover all 19
    assert not (c["o_written"] & p["o_written"]).any()
    assert len(written_rows(mixed, "o", m["o_written"])) == 19


# ----------------------------------------------------------------- library routine

def _torch_f64(batch, name):
    """A 16-bit input buffer widened to float64 by torch's own conversion."""
    t = torch.from_numpy(batch.data[name].view(np.int16)).view(workloads.TORCH_DTYPE[batch.dtype])
    return t.double().numpy()


def _torch_ref(batch, b, lq, lk, policy, need_grad=False):
    q = torch.from_numpy(seq_rows(batch, "q", _torch_f64(batch, "q"), b, lq))
    k = torch.from_numpy(seq_rows(batch, "k", _torch_f64(batch, "k"), b, lk))
    v = torch.from_numpy(seq_rows(batch, "v", _torch_f64(batch, "v"), b, lk))
    q, k, v = (x.permute(1, 0, 2)[None].contiguous().requires_grad_(need_grad) for x in (q, k, v))
    if policy == oracle.PADDING:
        mask = torch.ones(lq, lk, dtype=torch.bool)
    elif policy == oracle.CAUSAL_TOP_LEFT:
        mask = causal_upper_left(lq, lk)._materialize()
    else:
        mask = causal_lower_right(lq, lk)._materialize()
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=batch.scale,
                                       enable_gqa=True)
    kk = k.repeat_interleave(batch.h_q // batch.h_kv, dim=1)
    scores = torch.matmul(q, kk.transpose(-1, -2).contiguous()) * batch.scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    return q, k, v, o, lse, mask


@pytest.mark.parametrize("seed,dtype", [(11, "bf16"), (12, "bf16"), (13, "bf16"), (14, "bf16"),
                                        (15, "f16"), (16, "f16")])
def test_forward_matches_torch_sdpa_per_sequence(seed, dtype):
    batch = workloads.random_batch(seed, batch=5, max_len=40, h_q=4, h_kv=2, dim=16,
                                   dtype=dtype)
    res = _run_fwd(batch)
    assert res["status"] == 0
    for b, info in enumerate(res["infos"]):
        if info.lq == 0:
            continue
        o = seq_rows(batch, "o", res["o"], b, info.lq)
        lse = seq_rows(batch, "lse", res["lse"], b, info.lq)[..., 0]
        if info.lk == 0:
            assert np.all(o == 0) and np.all(lse == -np.inf)
            continue
        _, _, _, o_t, lse_t, mask = _torch_ref(batch, b, info.lq, info.lk, info.policy)
        live = mask.any(dim=1).numpy()
        o_t = o_t[0].permute(1, 0, 2).detach().numpy()
        lse_t = lse_t[0].permute(1, 0).detach().numpy()
        np.testing.assert_allclose(o[live], o_t[live], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[live], lse_t[live], rtol=1e-12, atol=1e-12)
        assert np.all(o[~live] == 0) and np.all(lse[~live] == -np.inf)   # dead rows
        assert np.all(o_t[~live] == 0)                                  # torch agrees on O


@pytest.mark.parametrize("seed,dtype", [(21, "bf16"), (22, "bf16"), (23, "bf16"), (24, "f16")])
def test_backward_matches_torch_autograd_per_sequence(seed, dtype):
    batch = workloads.random_batch(seed, batch=4, max_len=24, h_q=4, h_kv=2, dim=8,
                                   zero_lengths=False, dtype=dtype)
    prob, t = oracle.from_batch(batch)
    res = oracle.backward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"],
                          t["dk"], t["dv"])
    assert res["status"] == 0
    for b, info in enumerate(res["infos"]):
        q, k, v, o_t, _, mask = _torch_ref(batch, b, info.lq, info.lk, info.policy, True)
        do = torch.from_numpy(seq_rows(batch, "do", _torch_f64(batch, "do"),
                                       b, info.lq)).permute(1, 0, 2)[None]
        live = mask.any(dim=1)
        (o_t * do * live[None, None, :, None]).sum().backward()
        dq = seq_rows(batch, "dq", res["dq"], b, info.lq)
        dk = seq_rows(batch, "dk", res["dk"], b, info.lk)
        dv = seq_rows(batch, "dv", res["dv"], b, info.lk)
        np.testing.assert_allclose(dq, q.grad[0].permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(dk, k.grad[0].permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(dv, v.grad[0].permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)


# ----------------------------------------------------------------- fp16 inputs

def test_f16_widening_is_exact_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bits_to_f64(bits, "f16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # and bf16 against torch's bfloat16
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    mine = oracle.bits_to_f64(bits, "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and np.array_equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize("seed", [81, 82])
def test_same_values_in_either_format_give_identical_results(seed):
    """The oracle computes in fp64 from exactly widened inputs, so a batch whose
    values are representable in both formats gives bit-identical outputs."""
    a = workloads.random_batch(seed, batch=4, max_len=50, dim=16, window="random",
                               q_causal_offset=True)
    b = workloads.random_batch(seed, batch=4, max_len=50, dim=16, window="random",
                               q_causal_offset=True, dtype="f16")
    for n in ("q", "k", "v", "do"):
        vals = torch.from_numpy(a.data[n].view(np.int16)).view(torch.bfloat16).float()
        # bf16 values below 2^-14 may not be exact in fp16: flush those to 0
        vals = torch.where(vals.abs() < 2.0 ** -14, torch.zeros_like(vals), vals)
        a.data[n] = vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        h = vals.to(torch.float16)
        assert torch.equal(h.float().nan_to_num(7.0), vals.nan_to_num(7.0))  # exact
        b.data[n] = h.view(torch.int16).numpy().view(np.uint16)
    pa, ta = oracle.from_batch(a)
    pb, tb = oracle.from_batch(b)
    fa = oracle.forward(pa, ta["q"], ta["k"], ta["v"], ta["o"], ta["lse"])
    fb = oracle.forward(pb, tb["q"], tb["k"], tb["v"], tb["o"], tb["lse"])
    w = fa["o_written"]
    assert np.array_equal(w, fb["o_written"]) and np.array_equal(fa["o"][w], fb["o"][w])
    lw = fa["lse_written"]
    assert np.array_equal(fa["lse"][lw], fb["lse"][lw])
    ga = oracle.backward(pa, ta["q"], ta["k"], ta["v"], ta["o"], ta["lse"], ta["do"], ta["dq"],
                         ta["dk"], ta["dv"])
    gb = oracle.backward(pb, tb["q"], tb["k"], tb["v"], tb["o"], tb["lse"], tb["do"], tb["dq"],
                         tb["dk"], tb["dv"])
    for n in ("dq", "dk", "dv"):
        w = ga[n + "_written"]
        assert np.array_equal(ga[n][w], gb[n][w]), n


# ----------------------------------------------------------------- closed forms

def _tiny(lq, lk, policy=0, qco=None, dim=8, seed=3):
    return workloads.build("tiny", seed, 1, 1, dim, [lq], [lk], [0, lq], [0, lk],
                           default_policy=policy,
                           q_causal_offset=None if qco is None else [qco])


def test_single_key_closed_form():
    batch = _tiny(1, 1)
    res = _run_fwd(batch)
    q = oracle.bf16_bits_to_f64(batch.data["q"])
    k = oracle.bf16_bits_to_f64(batch.data["k"])
    v = oracle.bf16_bits_to_f64(batch.data["v"])
    np.testing.assert_array_equal(res["o"], v)                       # O = V_0
    assert res["lse"][0] == pytest.approx(batch.scale * float(q @ k), rel=1e-15)


def test_equal_keys_closed_form():
    batch = _tiny(3, 5)
    kb = batch.layouts["k"].view(batch.data["k"])
    kb[:] = kb[0]                                                    # all keys equal
    res = _run_fwd(batch)
    q = batch.layouts["q"].view(oracle.bf16_bits_to_f64(batch.data["q"]))[:, 0]
    k0 = oracle.bf16_bits_to_f64(batch.data["k"])[:8]
    v = batch.layouts["v"].view(oracle.bf16_bits_to_f64(batch.data["v"]))[:, 0]
    o = batch.layouts["o"].view(res["o"])[:, 0]
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=1e-13)
    s = batch.scale * (q @ k0)
    np.testing.assert_allclose(res["lse"], s + np.log(5), rtol=1e-13)


@pytest.mark.parametrize("lq,lk", [(5, 9), (9, 5), (7, 7)])
def test_q_causal_offset_special_cases(lq, lk):
    def out(policy, qco=None):
        return _run_fwd(_tiny(lq, lk, policy, qco))

    tl, br, pad = out(1), out(2), out(0)
    np.testing.assert_array_equal(out(1, 0)["o"], tl["o"])           # offset 0 = top-left
    np.testing.assert_array_equal(out(2, lk - lq)["o"], br["o"])     # Lk-Lq = bottom-right
    np.testing.assert_array_equal(out(1, lk - 1)["o"], pad["o"])     # >= Lk-1 = padding
    np.testing.assert_array_equal(out(2, lk + 5)["o"], pad["o"])
    np.testing.assert_array_equal(out(0, -3)["o"], pad["o"])         # padding ignores it


def test_negative_offset_gives_dead_leading_rows():
    res = _run_fwd(_tiny(6, 6, 1, -2))
    lse = res["lse"]
    assert np.all(lse[:2] == -np.inf) and np.all(np.isfinite(lse[2:]))
    o = res["o"].reshape(6, 8)
    assert np.all(o[:2] == 0)


# ----------------------------------------------------------------- invariants

def test_packed_bound_offsets_equal_derived_offsets():
    rng = np.random.default_rng(5)
    lens = rng.integers(1, 30, size=6)
    start = np.concatenate([[0], np.cumsum(lens)])
    batch = workloads.build("packed", 5, 4, 4, 16, lens, lens, start, start, default_policy=1)
    cu = batch.cu_q.astype(np.int64)
    for n in ("q", "k", "v", "o", "lse"):
        np.testing.assert_array_equal(batch.ragged(n), cu * batch.layouts[n].stride_t)
    res = _run_fwd(batch)
    assert res["o_written"].all()        # packed: every element of O is a valid row


def test_token_major_lse_is_transpose_of_head_major():
    a = workloads.random_batch(31, batch=4, max_len=30, lse_kind="token")
    b = workloads.random_batch(31, batch=4, max_len=30, lse_kind="head")
    ra, rb = _run_fwd(a), _run_fwd(b)
    la = a.layouts["lse"].view(ra["lse"])[:, :, 0]      # [t, h]
    lb = b.layouts["lse"].view(rb["lse"])[:, :, 0]      # [t, h] view of [h, t] storage
    wa = a.layouts["lse"].view(ra["lse_written"])[:, :, 0]
    np.testing.assert_array_equal(la[wa], lb[wa])
    hm = rb["lse"].reshape(b.h_q, -1)                   # raw head-major storage
    np.testing.assert_array_equal(hm.T[wa], la[wa])


def test_gqa_equals_mha_with_repeated_kv_heads():
    g = workloads.random_batch(41, batch=3, max_len=30, h_q=4, h_kv=2, dim=16, token_gaps=False)
    m = workloads.random_batch(41, batch=3, max_len=30, h_q=4, h_kv=4, dim=16, token_gaps=False)
    for n in ("k", "v"):
        src = g.layouts[n].view(g.data[n])
        dst = m.layouts[n].view(m.data[n])
        dst[:] = np.repeat(src, 2, axis=1)
    for n in ("q",):
        m.data[n] = g.data[n]
    rg, rm = _run_fwd(g), _run_fwd(m)
    np.testing.assert_array_equal(rg["o"], rm["o"])
    np.testing.assert_array_equal(rg["lse"], rm["lse"])


def test_permuting_sequences_permutes_outputs():
    batch = workloads.random_batch(51, batch=5, max_len=30, token_gaps=False)
    res = _run_fwd(batch)
    perm = np.array([3, 0, 4, 1, 2])
    p = workloads.random_batch(51, batch=5, max_len=30, token_gaps=False)
    p.lq, p.lk = batch.lq[perm], batch.lk[perm]
    p.policy = batch.policy[perm]
    for n, lay in p.layouts.items():
        src = batch.layouts[n].start_rows
        lay.start_rows = np.concatenate([src[:-1][perm], src[-1:]])
    rp = _run_fwd(p)
    np.testing.assert_array_equal(rp["o"], res["o"])
    np.testing.assert_array_equal(rp["lse"], res["lse"])


def test_explicit_q_offset_equals_bottom_right_with_cropped_keys():
    """A context-parallel query chunk with q[0] at absolute key `off` of an
    L-key document equals bottom-right attention over the first off+Lq keys."""
    L, lq = 96, 16
    for off in (16, 40, 80):
        full = workloads.build("cp", 9, 2, 2, 16, [lq], [L], [0, lq], [0, L], default_policy=1,
                               q_causal_offset=[off])
        crop = workloads.build("crop", 9, 2, 2, 16, [lq], [off + lq], [0, lq], [0, L],
                               default_policy=2)
        for n in ("q", "k", "v"):
            crop.data[n] = full.data[n]
        a, b = _run_fwd(full), _run_fwd(crop)
        np.testing.assert_array_equal(a["o"], b["o"])
        np.testing.assert_array_equal(a["lse"], b["lse"])


# ----------------------------------------------------------------- finite differences

def _fd_problem():
    """3 segments + 1: a dead leading row (negative offset), a bottom-right
    sequence, and two segments binding the same K/V rows (aliasing)."""
    rng = np.random.default_rng(77)
    H_q, H_kv, D = 2, 1, 6
    lq = np.array([3, 2, 2, 3])
    lk = np.array([4, 3, 5, 5])
    q_start = np.array([0, 3, 6, 8, 12])
    kv_start = np.array([0, 4, 8, 8, 14])      # segments 2 and 3 alias K/V rows 8..12
    prob = oracle.Problem(H_q, H_kv, D, 0.7, np.concatenate([[0], np.cumsum(lq)]).astype(np.int32),
                          np.concatenate([[0], np.cumsum(lk)]).astype(np.int32),
                          np.array([1, 2, 1, 1], np.int8), 0, np.array([-1, 1, 1, 3], np.int32))
    # segment 0 (top-left with offset -1) has a dead first row; segment 1 keeps
    # the bottom-right default (1); segments 2, 3 use explicit offsets.
    prob.q_causal_offset = None
    prob.policy = np.array([1, 2, 1, 1], np.int8)

    def mk(rows, heads, start, data=None):
        st = heads * D
        arr = rng.standard_normal(rows * st) if data is None else data
        return oracle.Tensor(arr, st, D, np.asarray(start, np.int64) * st, heads, D)

    q = mk(12, H_q, q_start)
    k = mk(14, H_kv, kv_start)
    v = mk(14, H_kv, kv_start)
    do = mk(12, H_q, q_start)
    o = mk(12, H_q, q_start, np.zeros(12 * H_q * D))
    lse = oracle.Tensor(np.zeros(12 * H_q), H_q, 1, np.asarray(q_start, np.int64) * H_q, H_q, 1)
    dq = mk(12, H_q, q_start, np.zeros(12 * H_q * D))
    dk = mk(14, H_kv, kv_start, np.zeros(14 * H_kv * D))
    dv = mk(14, H_kv, kv_start, np.zeros(14 * H_kv * D))
    return prob, q, k, v, o, lse, do, dq, dk, dv


@pytest.mark.parametrize("use_offsets,windowed", [(False, False), (True, False), (True, True),
                                                  (False, True)])
def test_backward_matches_central_differences(use_offsets, windowed):
    prob, q, k, v, o, lse, do, dq, dk, dv = _fd_problem()
    if use_offsets:
        prob.q_causal_offset = np.array([-1, 1, 1, 3], np.int32)
    if windowed:
        # top-left: one key back; bottom-right: the diagonal and two keys back
        prob.window = np.array([[-1, -1], [1, 0], [2, -1]], np.int32)

    def loss():
        r = oracle.forward(prob, q, k, v, o, lse)
        return float((r["o"][r["o_written"]] * do.data[r["o_written"]]).sum())

    g = oracle.backward(prob, q, k, v, o, lse, do, dq, dk, dv)
    assert g["status"] == 0
    if use_offsets:
        assert g["infos"][0].diag == -1      # a dead leading row in segment 0
    h = 1e-6
    for t, name in ((q, "dq"), (k, "dk"), (v, "dv")):
        written = g[name + "_written"]
        for idx in np.nonzero(written)[0]:
            keep = t.data[idx]
            t.data[idx] = keep + h
            up = loss()
            t.data[idx] = keep - h
            down = loss()
            t.data[idx] = keep
            fd = (up - down) / (2 * h)
            assert g[name][idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, idx)
        # elements outside written rows get no gradient written
        assert not written[~np.isin(np.arange(t.data.size), np.nonzero(written)[0])].any()


def test_aliased_segments_sum_their_kv_gradients():
    prob, q, k, v, o, lse, do, dq, dk, dv = _fd_problem()
    full = oracle.backward(prob, q, k, v, o, lse, do, dq, dk, dv)
    parts = []
    for keep in (2, 3):
        p2 = oracle.Problem(prob.h_q, prob.h_kv, prob.head_dim, prob.scale, prob.cu_q.copy(),
                            prob.cu_kv.copy(), prob.policy.copy(), 0, None)
        p2.policy[[b for b in (0, 1, 2, 3) if b != keep]] = 9    # invalid: skipped
        parts.append(oracle.backward(p2, q, k, v, o, lse, do, dq, dk, dv))
    rows = slice(8 * 6, 13 * 6)
    np.testing.assert_allclose(full["dk"][rows], parts[0]["dk"][rows] + parts[1]["dk"][rows],
                               rtol=1e-13, atol=1e-15)


def _kv_problem(kv_start, lk, seed=5):
    """Four query segments of 3 rows (top-left causal with offsets) over key
    rows placed at ``kv_start`` (start row of each segment's K/V/dK/dV)."""
    rng = np.random.default_rng(seed)
    H, D = 1, 4
    B = len(lk)
    lq = np.full(B, 3)
    q_start = np.arange(B + 1) * 3
    kv_rows = int(max(s + n for s, n in zip(kv_start, lk)))
    prob = oracle.Problem(H, H, D, 0.5, np.concatenate([[0], np.cumsum(lq)]).astype(np.int32),
                          np.concatenate([[0], np.cumsum(lk)]).astype(np.int32),
                          np.ones(B, np.int8), 0, np.full(B, 2, np.int32))

    def mk(rows, start, zero=False):
        arr = np.zeros(rows * D) if zero else rng.standard_normal(rows * D)
        return oracle.Tensor(arr, D, D, np.asarray(list(start) + [0], np.int64) * D, H, D)

    q, do = mk(3 * B, q_start[:-1]), mk(3 * B, q_start[:-1])
    k, v = mk(kv_rows, kv_start), mk(kv_rows, kv_start)
    o, dq = mk(3 * B, q_start[:-1], True), mk(3 * B, q_start[:-1], True)
    dk, dv = mk(kv_rows, kv_start, True), mk(kv_rows, kv_start, True)
    lse = oracle.Tensor(np.zeros(3 * B), 1, 1, np.asarray(q_start, np.int64), H, 1)
    return prob, q, k, v, o, lse, do, dq, dk, dv


def test_partial_kv_overlap_skips_both_groups():
    """Segments 1 and 2 bind different key rows that intersect (rows 4..9 and
    8..13): neither group's dK/dV can be stored, so both are skipped with
    ST_KV_OVERLAP; segments 0 and 3 (disjoint rows) are computed exactly as
    when 1 and 2 are invalid for another reason."""
    prob, q, k, v, o, lse, do, dq, dk, dv = _kv_problem([0, 4, 8, 14], [4, 6, 6, 5])
    g = oracle.backward(prob, q, k, v, o, lse, do, dq, dk, dv)
    assert g["status"] == oracle.ST_KV_OVERLAP
    assert [i.valid for i in g["infos"]] == [True, False, False, True]
    assert not g["dq_written"][3 * 4:9 * 4].any()
    assert not g["dk_written"][4 * 4:14 * 4].any()
    prob.policy = np.array([1, 9, 9, 1], np.int8)
    ref = oracle.backward(prob, q, k, v, o, lse, do, dq, dk, dv)
    assert ref["status"] == oracle.ST_BAD_POLICY
    for n in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(g[n + "_written"], ref[n + "_written"])
        np.testing.assert_array_equal(g[n], ref[n])
    # the forward reads K/V only: no overlap rule there
    f = oracle.forward(prob, q, k, v, o, lse)
    assert not f["status"] & oracle.ST_KV_OVERLAP


def test_touching_kv_ranges_do_not_overlap():
    prob, q, k, v, o, lse, do, dq, dk, dv = _kv_problem([0, 4, 10, 15], [4, 6, 5, 5])
    assert oracle.backward(prob, q, k, v, o, lse, do, dq, dk, dv)["status"] == 0
    assert oracle.kv_overlap(
        [oracle.sequence_info(prob, [q], [k], b) for b in range(4)], k, v, dk, dv) == [False] * 4


def test_interleaved_aliased_segments_sum_like_adjacent_ones():
    """Segments binding identical key rows form one kv group wherever they sit:
    the order A0, B0, A1, B1 gives the dK/dV of A0, A1, B0, B1 (up to the
    order of the fp64 sums)."""
    a = _kv_problem([0, 8, 0, 8], [8, 8, 8, 8])
    prob, q, k, v, o, lse, do, dq, dk, dv = a
    inter = oracle.backward(prob, q, k, v, o, lse, do, dq, dk, dv)
    assert inter["status"] == 0
    # move segment 2 (A1) before segment 1 (B0): permute the query-side rows
    # and the per-segment offsets
    perm = [0, 2, 1, 3]
    q2 = oracle.Tensor(q.data, q.stride_t, q.stride_h, q.ragged.copy(), 1, 4)
    do2 = oracle.Tensor(do.data, do.stride_t, do.stride_h, do.ragged.copy(), 1, 4)
    kv = [oracle.Tensor(t.data, t.stride_t, t.stride_h, t.ragged.copy(), 1, 4)
          for t in (k, v, dk, dv)]
    for t, src in [(q2, q), (do2, do)] + list(zip(kv, (k, v, dk, dv))):
        t.ragged[:4] = src.ragged[perm]
    adj = oracle.backward(prob, q2, kv[0], kv[1], o, lse, do2, dq, kv[2], kv[3])
    assert adj["status"] == 0
    for n in ("dk", "dv"):
        np.testing.assert_allclose(inter[n], adj[n], rtol=1e-13, atol=1e-15)
    # and each document's dK is the sum of its two segments run alone
    parts = []
    for keep in (0, 2):
        p2 = oracle.Problem(1, 1, 4, 0.5, prob.cu_q, prob.cu_kv, prob.policy.copy(), 0,
                            prob.q_causal_offset)
        p2.policy[[b for b in range(4) if b != keep]] = 9
        parts.append(oracle.backward(p2, q, k, v, o, lse, do, dq, dk, dv)["dk"][:8 * 4])
    np.testing.assert_allclose(inter["dk"][:8 * 4], parts[0] + parts[1], rtol=1e-13,
                               atol=1e-15)


@pytest.mark.parametrize("seed,window,qco,lse_kind", [
    (71, None, False, "token"), (72, "random", True, "head"), (73, "random", False, "token"),
    (74, None, True, "head")])
def test_forward_rows_equals_forward(seed, window, qco, lse_kind):
    """The row-by-row oracle used for sampled checks at full size gives the
    same O and LSE as the whole-batch oracle, for every row of every
    sequence and head: random lengths and gaps, per-sequence policies, GQA,
    windows, q causal offsets and both LSE layouts (one row's softmax is the
    same sum whether it sits in a block or alone; only the matrix products'
    summation order may differ)."""
    batch = workloads.random_batch(seed, batch=5, max_len=150, h_q=4, h_kv=2, dim=16,
                                   window=window, q_causal_offset=qco, lse_kind=lse_kind,
                                   with_grad=False)
    prob, t = oracle.from_batch(batch)
    full = oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])
    o_view = batch.layouts["o"].view(full["o"])
    l_view = batch.layouts["lse"].view(full["lse"])[:, :, 0]
    checked = 0
    for b in range(batch.batch):
        lq = int(batch.lq[b])
        if lq == 0 or not full["infos"][b].valid:
            continue
        r0 = int(batch.layouts["o"].start_rows[b])
        rl = int(batch.layouts["lse"].start_rows[b])
        for h in range(batch.h_q):
            o_r, l_r = oracle.forward_rows(prob, t["q"], t["k"], t["v"], b, h, range(lq))
            np.testing.assert_allclose(o_r, o_view[r0:r0 + lq, h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l_r, l_view[rl:rl + lq, h], rtol=1e-12, atol=1e-13)
            checked += lq
    assert checked > 200


# ----------------------------------------------------------------- validation

def test_invalid_sequences_are_skipped_with_status_bits():
    batch = workloads.random_batch(61, batch=4, max_len=20, zero_lengths=False, token_gaps=False)
    prob, t = oracle.from_batch(batch)
    t["k"].ragged = t["k"].ragged.copy()
    t["k"].ragged[1] = -8                                   # negative offset
    t["q"].ragged = t["q"].ragged.copy()
    t["q"].ragged[2] = t["q"].span                          # past the buffer
    prob.policy = prob.policy.copy()
    prob.policy[3] = 5                                      # unknown policy
    res = oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])
    assert res["status"] == oracle.ST_BAD_OFFSET | oracle.ST_OUT_OF_SPAN | oracle.ST_BAD_POLICY
    assert [i.valid for i in res["infos"]] == [True, False, False, False]
    rows = written_rows(batch, "o", res["o_written"])
    s = batch.layouts["o"].start_rows
    assert set(rows) == set(range(s[0], s[0] + batch.lq[0]))
    cu = prob.cu_q.copy()
    cu[1], cu[2] = cu[2], cu[1]
    prob.cu_q = cu
    res2 = oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])
    assert res2["status"] & oracle.ST_NEG_LENGTH


# ----------------------------------------------------------------- sizing pins

def test_head_major_stats_span_pin():
    g = _golden("stats_span.json")
    h, t = g["h_q"], g["t"]
    st = g["stride_stats"]
    assert st[0] == h * t and st[1] == t and st[2] == 1
    span = oracle.sizing.span_by_enumeration((h, t), (st[1], st[2]))
    assert span == g["every_axis_elems"] == 58880
    token_stride_only = t * st[2]
    assert token_stride_only == g["token_stride_only_elems"]
    assert span // token_stride_only == h
    assert (span - token_stride_only) * 4 == g["overrun_bytes"] == (h - 1) * t * 4


@pytest.mark.parametrize("T,h,d", [(5, 3, 4), (7, 2, 8), (1, 4, 2)])
def test_token_major_span_identities(T, h, d):
    # softmax_sum: [T, h] token-major; dQ_accum: [T, h, d] token-major
    assert oracle.sizing.span_by_enumeration((T, h), (h, 1)) == T * h
    assert oracle.sizing.span_by_enumeration((T, h, d), (h * d, d, 1)) == T * h * d
    for shape, strides in (((T, h), (1, T)), ((T, h, d), (d, T * d, 1)), ((T, h, d), (3 * h * d, d, 1))):
        assert oracle.sizing.span_by_enumeration(shape, strides) == \
            oracle.sizing.span_of_extremes(shape, strides)


# ----------------------------------------------------------------- sliding window

NO_WINDOW = np.full((3, 2), -1, np.int32)


def _window(pad=(-1, -1), tl=(-1, -1), br=(-1, -1)):
    return np.array([pad, tl, br], np.int32)


def _tiny_w(lq, lk, policy, window, qco=None, dim=8, seed=3):
    return workloads.build("tiny", seed, 1, 1, dim, [lq], [lk], [0, lq], [0, lk],
                           default_policy=policy,
                           q_causal_offset=None if qco is None else [qco], window=window)


@pytest.mark.parametrize("seed,qco", [(31, False), (32, True), (33, True)])
def test_unbounded_or_wide_window_is_no_window(seed, qco):
    kw = dict(batch=5, max_len=40, dim=16, q_causal_offset=qco)
    ref = _run_fwd(workloads.random_batch(seed, **kw))
    for win in (NO_WINDOW, np.full((3, 2), 10 ** 6, np.int32)):
        res = _run_fwd(workloads.random_batch(seed, window=win, **kw))
        np.testing.assert_array_equal(res["o"], ref["o"])
        np.testing.assert_array_equal(res["lse"], ref["lse"])


def _vrows(batch, name):
    return batch.layouts[name].view(oracle.bf16_bits_to_f64(batch.data[name]))[:, 0]


@pytest.mark.parametrize("lq,lk,policy,window,qco,shift", [
    (7, 7, oracle.PADDING, _window(pad=(0, 0)), None, 0),          # the diagonal only
    (4, 9, oracle.PADDING, _window(pad=(0, 0)), None, 5),          # anchored at Lk - Lq
    (7, 7, oracle.CAUSAL_TOP_LEFT, _window(tl=(0, -1)), None, 0),
    (4, 9, oracle.CAUSAL_TOP_LEFT, _window(tl=(0, 4)), 3, 3),      # anchored at the offset
    (4, 9, oracle.CAUSAL_BOTTOM_RIGHT, _window(br=(0, 0)), None, 5),
    (6, 6, oracle.PADDING, _window(pad=(0, 0)), -2, -2),           # rows 0, 1 dead
])
def test_zero_width_window_selects_one_key(lq, lk, policy, window, qco, shift):
    """A window of width 1: row i sees key i + shift alone, so O_i = V_{i+shift}
    exactly and LSE_i = scale * q_i . k_{i+shift}; rows whose key falls outside
    [0, Lk) are dead."""
    batch = _tiny_w(lq, lk, policy, window, qco)
    res = _run_fwd(batch)
    q, k, v = _vrows(batch, "q"), _vrows(batch, "k"), _vrows(batch, "v")
    o = batch.layouts["o"].view(res["o"])[:, 0]
    lse = batch.layouts["lse"].view(res["lse"])[:, 0, 0]
    for i in range(lq):
        j = i + shift
        if 0 <= j < lk:
            np.testing.assert_array_equal(o[i], v[j])
            assert lse[i] == pytest.approx(batch.scale * float(q[i] @ k[j]), rel=1e-15)
        else:
            assert np.all(o[i] == 0) and lse[i] == -np.inf


def test_zero_width_window_gradients_closed_form():
    """With one visible key per row the softmax is constant (P = 1): dQ = dK = 0
    and dV_j = dO of the row that sees key j."""
    batch = _tiny_w(4, 9, oracle.PADDING, _window(pad=(0, 0)))
    prob, t = oracle.from_batch(batch)
    g = oracle.backward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"],
                        t["dk"], t["dv"])
    assert np.all(g["dq"][g["dq_written"]] == 0) and np.all(g["dk"][g["dk_written"]] == 0)
    dv = batch.layouts["dv"].view(g["dv"])[:, 0]
    do = _vrows(batch, "do")
    np.testing.assert_array_equal(dv[:5], 0)
    np.testing.assert_array_equal(dv[5:], do)


def _band(lq, lk, policy, window, qco):
    """Visibility from torch's band routines: tril(k) keeps j - i <= k and
    triu(k) keeps j - i >= k; the causal part from torch's own causal masks."""
    m = torch.ones(lq, lk, dtype=torch.bool)
    if policy != oracle.PADDING:
        if qco is not None:
            m = m.tril(diagonal=int(qco))
        elif policy == oracle.CAUSAL_TOP_LEFT:
            m = causal_upper_left(lq, lk)._materialize()
        else:
            m = causal_lower_right(lq, lk)._materialize()
    if window is not None:
        left, right = (int(x) for x in window[policy])
        anchor = int(qco) if qco is not None else (0 if policy == oracle.CAUSAL_TOP_LEFT
                                                   else lk - lq)
        if right >= 0:
            m = m.tril(diagonal=anchor + right)
        if left >= 0:
            m = m.triu(diagonal=anchor - left)
    return m


def _torch_band_ref(batch, b, lq, lk, policy, need_grad=False):
    q = torch.from_numpy(seq_rows(batch, "q", _torch_f64(batch, "q"), b, lq))
    k = torch.from_numpy(seq_rows(batch, "k", _torch_f64(batch, "k"), b, lk))
    v = torch.from_numpy(seq_rows(batch, "v", _torch_f64(batch, "v"), b, lk))
    q, k, v = (x.permute(1, 0, 2)[None].contiguous().requires_grad_(need_grad) for x in (q, k, v))
    qco = None if batch.q_causal_offset is None else batch.q_causal_offset[b]
    mask = _band(lq, lk, policy, batch.window, qco)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=batch.scale,
                                       enable_gqa=True)
    kk = k.repeat_interleave(batch.h_q // batch.h_kv, dim=1)
    scores = torch.matmul(q, kk.transpose(-1, -2).contiguous()) * batch.scale
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
    return q, k, v, o, lse, mask


@pytest.mark.parametrize("seed,qco", [(41, False), (42, False), (43, True), (44, True)])
def test_window_forward_matches_torch_sdpa_with_band_mask(seed, qco):
    batch = workloads.random_batch(seed, batch=6, max_len=40, h_q=4, h_kv=2, dim=16,
                                   q_causal_offset=qco, window="random")
    assert batch.window is not None and (batch.window >= 0).any()
    res = _run_fwd(batch)
    assert res["status"] == 0
    for b, info in enumerate(res["infos"]):
        if info.lq == 0:
            continue
        o = seq_rows(batch, "o", res["o"], b, info.lq)
        lse = seq_rows(batch, "lse", res["lse"], b, info.lq)[..., 0]
        if info.lk == 0:
            assert np.all(o == 0) and np.all(lse == -np.inf)
            continue
        _, _, _, o_t, lse_t, mask = _torch_band_ref(batch, b, info.lq, info.lk, info.policy)
        live = mask.any(dim=1).numpy()
        o_t = o_t[0].permute(1, 0, 2).detach().numpy()
        lse_t = lse_t[0].permute(1, 0).detach().numpy()
        np.testing.assert_allclose(o[live], o_t[live], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[live], lse_t[live], rtol=1e-12, atol=1e-12)
        assert np.all(o[~live] == 0) and np.all(lse[~live] == -np.inf)


@pytest.mark.parametrize("seed,qco", [(51, False), (52, True), (53, False)])
def test_window_backward_matches_torch_autograd(seed, qco):
    batch = workloads.random_batch(seed, batch=4, max_len=24, h_q=4, h_kv=2, dim=8,
                                   zero_lengths=False, q_causal_offset=qco, window="random")
    prob, t = oracle.from_batch(batch)
    res = oracle.backward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"],
                          t["dk"], t["dv"])
    assert res["status"] == 0
    for b, info in enumerate(res["infos"]):
        q, k, v, o_t, _, mask = _torch_band_ref(batch, b, info.lq, info.lk, info.policy, True)
        do = torch.from_numpy(seq_rows(batch, "do", _torch_f64(batch, "do"),
                                       b, info.lq)).permute(1, 0, 2)[None]
        live = mask.any(dim=1)
        (o_t * do * live[None, None, :, None]).sum().backward()
        dq = seq_rows(batch, "dq", res["dq"], b, info.lq)
        dk = seq_rows(batch, "dk", res["dk"], b, info.lk)
        dv = seq_rows(batch, "dv", res["dv"], b, info.lk)
        np.testing.assert_allclose(dq, q.grad[0].permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(dk, k.grad[0].permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(dv, v.grad[0].permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-11)


def _pairs(lq, lk, policy, window, qco=None):
    prob = oracle.Problem(1, 1, 8, 1.0, np.array([0, lq], np.int32), np.array([0, lk], np.int32),
                          None, policy, None if qco is None else np.array([qco], np.int32),
                          window)
    info = oracle.sequence_info(prob, [], [], 0)
    return int(oracle.attention.allowed(info, np.arange(lq), np.arange(lk)).sum())


@pytest.mark.parametrize("L,w", [(1, 0), (5, 0), (5, 2), (9, 3), (9, 8), (9, 20)])
def test_window_pair_counts_closed_form(L, w):
    # causal with w keys back: row i sees min(i, w) + 1 keys
    causal = L * (L + 1) // 2 if L <= w + 1 else (w + 1) * (w + 2) // 2 + (L - w - 1) * (w + 1)
    assert _pairs(L, L, oracle.CAUSAL_TOP_LEFT, _window(tl=(w, 0))) == causal
    assert _pairs(L, L, oracle.CAUSAL_BOTTOM_RIGHT, _window(br=(w, -1))) == causal
    # symmetric padding window: 2w + 1 keys per row minus the ones cut off at
    # either end, w(w+1)/2 per end
    sym = L * L if L <= w else L * (2 * w + 1) - w * (w + 1)
    assert _pairs(L, L, oracle.PADDING, _window(pad=(w, w))) == sym
    # a causal right window adds nothing to the diagonal
    assert _pairs(L, L, oracle.CAUSAL_TOP_LEFT, _window(tl=(w, 3))) == causal
