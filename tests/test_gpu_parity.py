"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X)."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import worklist
from tests.gpu_common import (GRAD_TOL, LSE_TOL, O_TOL, check_backward, check_forward,
                              compare_bf16, oracle_bwd, oracle_bwd_heads, oracle_fwd,
                              oracle_fwd_heads, pre_fill, say)
from tests._util import bf16_to_f64

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import variable_length_attention_ragged_amd as va
    va.lib()  # fail loudly if the library is missing


def _dev(batch, with_grad=None, **kw):
    from workloads.device import DeviceBatch
    return DeviceBatch(batch, with_grad=with_grad, **kw)


# ------------------------------------------------------------------ setup kernel

def _read_setup(ws, L, B):
    raw = ws.cpu().numpy().view(np.uint8)
    i32 = lambda off, n: raw[off:off + 4 * n].view(np.int32)
    header = i32(L.header_offset, 16)
    seq = i32(L.seq_offset, 6 * B).reshape(6, B)
    base = raw[L.seq_offset + L.seq_i64_offset:L.seq_offset + L.seq_i64_offset + 72 * B] \
        .view(np.int64).reshape(9, B)
    fwd = i32(L.fwd_tiles_offset, 2 * int(header[0])).reshape(-1, 2)
    bwd = i32(L.bwd_tiles_offset, 4 * int(header[1])).reshape(-1, 4) if header[1] > 0 else \
        np.zeros((0, 4), np.int32)
    counters = i32(L.counters_offset, 64)
    members = i32(L.members_offset, B)
    return header, seq, base, fwd, bwd, counters, members


def _check_setup(batch, backward):
    dev = _dev(batch, with_grad=backward)
    L = dev.bwd_layout() if backward else dev.fwd_layout()
    ws = torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda")
    (dev.bwd_setup if backward else dev.fwd_setup)(workspace=ws)
    torch.cuda.synchronize()
    header, seq, base, fwd, bwd, counters, members = _read_setup(ws, L, batch.batch)
    prob, t = oracle.from_batch(batch)
    if not backward:
        t = {n: t[n] for n in ("q", "k", "v", "o", "lse")}
    exp = worklist.setup(prob, t, backward=backward, bm=L.fwd_block_m, bn=L.fwd_block_n,
                         bm_b=L.bwd_block_m, bn_b=L.bwd_block_n,
                         cap_fwd=L.fwd_tiles_capacity, cap_bwd=L.bwd_tiles_capacity)
    np.testing.assert_array_equal(seq[0], exp["lq"])
    np.testing.assert_array_equal(seq[1], exp["lk"])
    np.testing.assert_array_equal(seq[2], exp["policy"])
    np.testing.assert_array_equal(seq[3], exp["hi"])
    np.testing.assert_array_equal(seq[4], exp["lo"])
    np.testing.assert_array_equal(seq[5], exp["flags"])
    np.testing.assert_array_equal(base, exp["base"])
    np.testing.assert_array_equal(fwd, exp["fwd"])
    if backward:
        np.testing.assert_array_equal(bwd, exp["bwd"])
        np.testing.assert_array_equal(members[:exp["members"].size], exp["members"])
    assert header[2] == exp["status"] == int(dev.status.item())
    assert not counters.any()


SETUP_CASES = [
    ("tiny_padded", lambda: workloads.tiny_padded_thd(causal=True)),
    ("padded_gqa", lambda: workloads.padded_gqa()),
    ("mixed_policy", lambda: workloads.mixed_policy(with_grad=True)),
    ("long_context_small", lambda: workloads.long_context_cp(doc_len=4096, chunk=512, offsets=(512, 3584))),
] + [(f"random{s}", (lambda s=s: workloads.random_batch(s, batch=9, max_len=300,
                                                         q_causal_offset=bool(s % 2))))
     for s in range(100, 106)] + [
    # more sequences (and kv groups) than the setup kernel ranks from LDS, and
    # tile lists longer than one block-scan chunk
    ("random_b1100", lambda: workloads.random_batch(300, batch=1100, max_len=12, max_gap=4)),
    # batches that split the setup kernel's pairwise passes 8, 2 and 1 lanes
    # per sequence (all ranked from LDS), and many aliased kv groups
    ("random_b100", lambda: workloads.random_batch(302, batch=100, max_len=40, max_gap=4)),
    ("random_b300", lambda: workloads.random_batch(303, batch=300, max_len=20, max_gap=4,
                                                   q_causal_offset=True)),
    ("random_b1000", lambda: workloads.random_batch(304, batch=1000, max_len=12, max_gap=3)),
    ("aliased_b120", lambda: workloads.aliased_batch(305, docs=40, max_doc=60, chunks=3)),
    ("random_b2200", lambda: workloads.random_batch(301, batch=2200, max_len=6, max_gap=2,
                                                    cross=False)),
] + [(f"window{s}", (lambda s=s: workloads.random_batch(s, batch=9, max_len=600,
                                                         q_causal_offset=bool(s % 2),
                                                         window="random")))
     for s in range(120, 126)] + [
    ("long_context_small_window", lambda: _windowed(workloads.long_context_cp(doc_len=4096, chunk=512,
                                                              offsets=(512, 3584)),
                                            [[-1, -1], [700, 0], [-1, -1]])),
    ("interleaved_chunks", lambda: _interleaved_chunks()),
    ("partial_kv_overlap", lambda: _partial_kv_overlap()),
    ("overlap_b1100", lambda: _overlap_many()),
]


def _interleaved_chunks(doc=640, chunk=160):
    """Query chunks of documents A and B in the order A0, B0, X, A1, B1; X
    binds A's key rows with an unknown policy (skipped).  A0/A1 and B0/B1
    each form one kv group although they are not adjacent."""
    lq, lk = [chunk] * 5, [doc] * 5
    q_start = [chunk * i for i in range(6)]
    kv_start = [0, doc, 0, 0, doc, 2 * doc]
    qco = [chunk, chunk, chunk, doc - chunk, doc - chunk]
    return workloads.build("interleaved_cp", 801, 4, 2, 128, lq, lk, q_start, kv_start,
                           default_policy=1, policy=[1, 1, 9, 1, 1], q_causal_offset=qco,
                           lse_kind="head")


def _partial_kv_overlap():
    """Sequence 1's key rows (150..299) intersect sequence 0's (0..199):
    both are skipped by the backward; 2 and 3 are disjoint."""
    lq, lk = [100, 90, 120, 80], [200, 150, 170, 60]
    q_start = [0, 100, 190, 310, 390]
    kv_start = [0, 150, 400, 600, 700]
    return workloads.build("partial_overlap", 802, 4, 2, 64, lq, lk, q_start, kv_start,
                           default_policy=0, policy=[0, 1, 2, 0], lse_kind="token")


def _overlap_many():
    """1100 short sequences (more than the setup kernel keeps in LDS): every
    fifth binds the key rows of the one before it (one kv group), and one
    pair of sequences overlaps partially."""
    rng = np.random.default_rng(803)
    B = 1100
    lk = rng.integers(1, 12, size=B, endpoint=True)
    lq = rng.integers(0, 12, size=B, endpoint=True)
    start = np.zeros(B + 1, np.int64)
    row = 0
    for b in range(B):
        if b % 5 == 4:
            lk[b] = lk[b - 1]
            start[b] = start[b - 1]
        else:
            start[b] = row
            row += int(lk[b]) + 1
    start[B] = row
    start[700] = start[699] + 1          # partial overlap of 699 and 700
    lk[700] = max(int(lk[700]), 2)
    q_start = np.concatenate([[0], np.cumsum(lq)])
    return workloads.build("overlap_many", 803, 2, 1, 64, lq, lk, q_start, start,
                           default_policy=2, lse_kind="token", kv_rows=row + 16)


def _windowed(batch, window):
    batch.window = np.asarray(window, np.int32)
    return batch


@pytest.mark.parametrize("name,make", SETUP_CASES, ids=[c[0] for c in SETUP_CASES])
@pytest.mark.parametrize("backward", [False, True])
def test_setup_bit_exact(name, make, backward):
    say(f"[setup] {name} backward={backward}")
    _check_setup(make(), backward)


# ------------------------------------------------------------------ small configs

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lse_kind", ["token", "head"])
def test_config1_fwd_bwd(causal, lse_kind):
    say(f"[tiny padded] causal={causal} lse={lse_kind}")
    batch = workloads.tiny_padded_thd(causal=causal, lse_kind=lse_kind)
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


RANDOM = [(s, d) for s in range(200, 206) for d in (64, 128)]


@pytest.mark.parametrize("seed,dim", RANDOM)
def test_random_fwd_bwd(seed, dim):
    batch = workloads.random_batch(seed, batch=6, max_len=300, h_q=4, h_kv=2, dim=dim,
                                   q_causal_offset=(seed % 3 == 0))
    say(f"[random] seed={seed} D={dim} lq={batch.lq.tolist()} lk={batch.lk.tolist()}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


WINDOWED = [(s, d) for s in range(220, 226) for d in (64, 128)]


@pytest.mark.parametrize("seed,dim", WINDOWED)
def test_window_random_fwd_bwd(seed, dim):
    """Per-policy sliding windows (random sizes, some sides unbounded) on
    random ragged batches, with and without q_causal_offset anchoring them."""
    batch = workloads.random_batch(seed, batch=6, max_len=500, h_q=4, h_kv=2, dim=dim,
                                   q_causal_offset=(seed % 2 == 0), window="random")
    say(f"[window] seed={seed} D={dim} window={batch.window.tolist()} "
        f"lq={batch.lq.tolist()} lk={batch.lk.tolist()}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


@pytest.mark.parametrize("window", [
    [[-1, -1], [256, 0], [-1, -1]],       # causal, 256 keys back
    [[100, 37], [-1, -1], [-1, -1]],      # padding, asymmetric around the row
    [[0, 0], [0, 0], [0, 0]],             # one key per row
])
def test_sliding_window_long_sequences(window):
    """Sequences of up to 2000 rows: the band skips most key tiles of every
    query tile and most query tiles of every key tile."""
    rng = np.random.default_rng(230)
    lens = rng.integers(600, 2000, size=3, endpoint=True)
    pol = np.array([0, 1, 0], np.int8)
    start = np.concatenate([[0], np.cumsum(lens + 8)])
    batch = workloads.build("long_window", 230, 4, 2, 128, lens, lens, start, start,
                            default_policy=0, policy=pol, lse_kind="head", window=window)
    say(f"[long window] {window} lens={lens.tolist()}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


def test_window_with_aliased_kv_segments():
    """Context-parallel chunks of one document with a causal window: the
    caller's offsets anchor each chunk's band, and the chunks' dK/dV sum."""
    batch = _windowed(workloads.long_context_cp(doc_len=1024, chunk=256, offsets=(256, 768)),
                      [[-1, -1], [300, 0], [-1, -1]])
    say("[window alias] long-context shape, doc 1024 chunk 256, window 300")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


FP16 = [(s, d, w) for s, d, w in ((240, 64, None), (241, 128, None), (242, 128, "random"),
                                   (243, 64, "random"), (244, 128, "random"))]


@pytest.mark.parametrize("seed,dim,window", FP16)
def test_fp16_random_fwd_bwd(seed, dim, window):
    """IEEE fp16 inputs and outputs (fp16 MFMAs, P and dS packed as fp16)."""
    batch = workloads.random_batch(seed, batch=6, max_len=400, h_q=4, h_kv=2, dim=dim,
                                   q_causal_offset=(seed % 2 == 0), window=window, dtype="f16")
    say(f"[fp16] seed={seed} D={dim} window={window if window is None else batch.window.tolist()}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


@pytest.mark.timeout(600)
def test_fp16_full_size():
    """The packed causal workload's shape in fp16: complete forward heads,
    sampled rows of random heads and the gradients of two kv heads."""
    b16 = workloads.packed_causal(with_grad=True)
    batch = workloads.build("packed_causal_f16", 1102, 32, 32, 128, b16.lq, b16.lk,
                            b16.layouts["q"].start_rows, b16.layouts["k"].start_rows,
                            default_policy=workloads.CAUSAL_TOP_LEFT, lse_kind="head",
                            dtype="f16")
    say(f"[fp16 full] tokens={int(batch.lq.sum())}")
    dev = _dev(batch, with_grad=True)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    assert int(dev.status.item()) == 0
    _check_fwd_heads(batch, dev, [5, 21])
    _check_sampled_fwd(batch, dev, seed=16)
    _check_bwd_heads(batch, dev, [21, 4])


def test_many_tiny_sequences_fwd_bwd():
    """1100 sequences of 0..12 rows: almost every tile is a ragged tail, and the
    setup ranks more sequences than it keeps in LDS."""
    batch = workloads.random_batch(302, batch=1100, max_len=12, max_gap=3, h_q=4, h_kv=2,
                                   dim=128)
    say(f"[tiny] B={batch.batch} tokens={int(batch.lq.sum())}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


def test_many_queries_over_few_keys_gradients():
    """Padding sequences with up to 244 queries over 3 keys (and the converse):
    every key collects the gradient of every query, so |dK| and |dV| reach
    about 12.  The GPU forms P and dS in fp32, rounds them to bf16 (2^-9
    relative each) for the MFMAs, and takes delta from the bf16 O the forward
    stored; those rounding errors add up over the queries that meet a key in
    the fp32 sums, in proportion to the gradient they build.  The bar is
    therefore 5e-2 + 2^-8 |ref|: the absolute bar for O(1) values plus bf16's
    relative precision, applied to the gradient's magnitude.  O and LSE keep
    their plain bars."""
    lq, lk = [244, 3, 200, 17], [3, 244, 5, 150]
    start_q = np.concatenate([[0], np.cumsum(np.asarray(lq) + 5)])
    start_k = np.concatenate([[0], np.cumsum(np.asarray(lk) + 3)])
    batch = workloads.build("many_queries_few_keys", 250, 4, 2, 64, lq, lk, start_q, start_k,
                            default_policy=0, lse_kind="token")
    say(f"[many queries] lq={lq} lk={lk}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    ref = oracle_bwd(batch)
    mags = {n: float(np.abs(ref[n][ref[n + "_written"]]).max()) for n in ("dq", "dk", "dv")}
    say(f"  max |grad| {mags}")
    assert mags["dk"] > 4.0          # the case this test exists for
    check_backward(batch, dev, ref, rel=2.0 ** -8)


@pytest.mark.timeout(600)
def test_largest_legal_token_stride_fwd_bwd():
    """Every 16-bit tensor with a token stride just below the largest the host
    accepts (a 128-row tile's byte range under 2^31, about 8.45 M elements):
    the kernels' 32-bit offsets inside a tile are then at their largest.  Key
    lengths above 64 fill whole key and query tiles.  Forward and backward
    against the oracle at the plain bars, pads untouched."""
    h, d = 1, 128
    n = ((1 << 30) - 128) // 127 // (h * d) - 1
    st = (1 + n) * h * d
    assert (127 * st + d) * 2 < 1 << 31 <= (127 * (st + h * d) + d) * 2
    lq, lk = [36, 20], [70, 30]
    start_q = np.concatenate([[0], np.cumsum(lq)])
    start_k = np.concatenate([[0], np.cumsum(lk)])
    gaps = {x: n for x in ("q", "k", "v", "o", "do", "dq", "dk", "dv")}
    batch = workloads.build("largest_stride", 260, h, h, d, lq, lk, start_q, start_k,
                            default_policy=2, lse_kind="head", token_gaps=gaps)
    say(f"[largest stride] stride_t={st} elements, lq={lq} lk={lk}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


def test_gqa_groups_of_four_fwd_bwd():
    batch = workloads.random_batch(300, batch=4, max_len=200, h_q=8, h_kv=2, dim=128)
    say(f"[gqa] lq={batch.lq.tolist()}")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


def test_aliased_kv_segments_sum_gradients():
    batch = workloads.long_context_cp(doc_len=1024, chunk=256, offsets=(256, 768))
    say("[alias] long-context shape, doc 1024 chunk 256")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    check_backward(batch, dev)


def test_interleaved_chunks_with_a_skipped_member_sum_gradients():
    """Non-adjacent chunks binding the same key rows form one kv group: their
    dK/dV are the sums, as the oracle defines them; the invalid member in
    between is skipped."""
    batch = _interleaved_chunks()
    say("[interleaved] A0 B0 X A1 B1")
    dev = _dev(batch)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)
    ref = oracle_bwd(batch)
    assert ref["status"] == oracle.ST_BAD_POLICY
    check_backward(batch, dev, ref)


def test_partial_kv_overlap_sets_status_and_leaves_gradients_untouched():
    batch = _partial_kv_overlap()
    say("[overlap] sequences 0 and 1 share key rows 150..199")
    dev = _dev(batch)
    dev.fwd()
    torch.cuda.synchronize()
    check_forward(batch, dev)           # the forward reads K/V only: status 0
    assert int(dev.status.item()) == 0
    dev.bwd()
    torch.cuda.synchronize()
    ref = oracle_bwd(batch)
    assert ref["status"] == oracle.ST_KV_OVERLAP
    assert int(dev.status.item()) == oracle.ST_KV_OVERLAP
    assert [i.valid for i in ref["infos"]] == [False, False, True, True]
    check_backward(batch, dev, ref)     # untouched outside the written rows


def test_autograd_function_matches_oracle():
    """The autograd Function over varlen_attn_fwd / varlen_attn_bwd: inputs as
    strided views of padded buffers (token-stride gaps), sequences located by
    int32 start rows, outputs and gradients in new dense tensors.  O, LSE and
    the gradients torch autograd delivers match the oracle; rows outside every
    sequence are 0."""
    import variable_length_attention_ragged_amd as va
    batch = workloads.random_batch(910, batch=5, max_len=260, h_q=4, h_kv=2, dim=128,
                                   window="random", q_causal_offset=True, lse_kind="head")
    say(f"[autograd] lq={batch.lq.tolist()} lk={batch.lk.tolist()}")
    dev = _dev(batch)
    lay = batch.layouts

    def view(n):
        L = lay[n]
        return torch.as_strided(dev.flat[n], (L.rows, L.heads, L.dim), (L.stride_t, L.stride_h, 1))

    q, k, v = (view(n).detach().requires_grad_() for n in ("q", "k", "v"))
    rows_q = torch.from_numpy(lay["q"].start_rows.astype(np.int32)).cuda()
    rows_kv = torch.from_numpy(lay["k"].start_rows.astype(np.int32)).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, lse = va.varlen_attention(q, k, v, dev.cu_q, dev.cu_kv, seq_rows_q=rows_q,
                                 seq_rows_kv=rows_kv, mask_policy=dev.policy,
                                 default_policy=batch.default_policy, q_causal_offset=dev.qco,
                                 window_size=batch.window.tolist(), scale=batch.scale,
                                 lse_head_major=True, status=status)
    assert not lse.requires_grad and lse.stride() == (1, lse.shape[0])
    do = torch.nan_to_num(view("do").float(), nan=0.0).to(o.dtype)
    o.backward(do)
    torch.cuda.synchronize()
    fref, bref = oracle_fwd(batch), oracle_bwd(batch)
    assert int(status.item()) == fref["status"] | bref["status"]

    def compare(got, ref, written, tol, n):
        got = got.detach().float().cpu().numpy().astype(np.float64)
        w = written.reshape(got.shape[0], -1).any(axis=1)   # rows of some sequence
        assert np.all(got[~w] == 0), f"{n}: rows outside every sequence must be 0"
        err = float(np.abs(got[w] - ref[w]).max()) if w.any() else 0.0
        say(f"  {n}: max abs err {err:.3e}")
        assert err <= tol, n

    def as3(n, arr):
        return lay[n].view(arr)

    compare(o, as3("o", fref["o"]), as3("o", fref["o_written"]), O_TOL, "o")
    l_ref = as3("lse", fref["lse"])[:, :, 0]
    l_w = as3("lse", fref["lse_written"])[:, :, 0]
    got = lse.detach().cpu().numpy().astype(np.float64)
    live = l_w & np.isfinite(l_ref)
    assert np.all(got[l_w & ~np.isfinite(l_ref)] == -np.inf)
    assert float(np.abs(got[live] - l_ref[live]).max()) <= LSE_TOL
    for n, t in (("dq", q), ("dk", k), ("dv", v)):
        compare(t.grad, as3(n, bref[n]), as3(n, bref[n + "_written"]), GRAD_TOL, n)


# ------------------------------------------------------------------ invariants on GPU

def test_mixed_policy_equals_sum_of_two_passes_bitwise():
    with open(os.path.join(GOLDEN, "mixed_policy_19row.json")) as f:
        g = json.load(f)
    one = g["single_call_reading"]
    pol = [1 if p == "causal" else 0 for p in one["policies"]]
    mixed = workloads.build("mixed19", 7, 2, 2, 64, one["lengths"], one["lengths"],
                            one["start_rows"], one["start_rows"], default_policy=0, policy=pol,
                            q_rows=19, kv_rows=19, with_grad=False)

    def run(batch):
        dev = _dev(batch, with_grad=False)
        dev.flat["o"].view(torch.int16).zero_()
        dev.fwd()
        torch.cuda.synchronize()
        return dev.host("o")

    outs = []
    for key, policy in (("causal_pass", 1), ("padding_pass", 0)):
        lens = np.diff(g[key]["cu_seqlens"])
        b = workloads.build("pass", 7, 2, 2, 64, lens, lens, g[key]["cu_seqlens_padded"],
                            g[key]["cu_seqlens_padded"], default_policy=policy, q_rows=19,
                            kv_rows=19, with_grad=False)
        for n in ("q", "k", "v"):
            b.data[n] = mixed.data[n]
        outs.append(bf16_to_f64(run(b)))
    m = bf16_to_f64(run(mixed))
    np.testing.assert_array_equal(m, outs[0] + outs[1])


def test_lse_layouts_agree_bitwise_and_forward_is_deterministic():
    a = workloads.random_batch(400, batch=5, max_len=260, dim=128, lse_kind="token",
                               with_grad=False)
    b = workloads.random_batch(400, batch=5, max_len=260, dim=128, lse_kind="head",
                               with_grad=False)
    da, db = _dev(a), _dev(b)
    da.fwd()
    db.fwd()
    torch.cuda.synchronize()
    la = a.layouts["lse"].view(da.host("lse"))[:, :, 0]
    lb = b.layouts["lse"].view(db.host("lse"))[:, :, 0]
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    assert np.array_equal(da.host("o"), db.host("o"))
    first = da.host("o")
    da.fwd()
    torch.cuda.synchronize()
    assert np.array_equal(first, da.host("o"))


def test_bad_device_arguments_set_status_and_leave_outputs_untouched():
    batch = workloads.random_batch(500, batch=4, max_len=100, zero_lengths=False,
                                   token_gaps=False)
    lay = batch.layouts["k"]
    lay_q = batch.layouts["q"]
    # sequence 1: K offset negative; sequence 2: Q offset past the span;
    # sequence 3: policy 5
    k_start = lay.start_rows.copy()
    q_start = lay_q.start_rows.copy()
    batch.layouts["k"].start_rows = k_start
    dev = _dev(batch)
    rk = dev.ragged["k"].clone()
    rk[1] = -8
    dev.ragged["k"] = rk
    rq = dev.ragged["q"].clone()
    rq[2] = lay_q.span
    dev.ragged["q"] = rq
    pol = dev.policy.clone()
    pol[3] = 5
    dev.policy = pol
    dev.problem.mask_policy = pol
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    prob, t = oracle.from_batch(batch)
    t["k"].ragged = rk.cpu().numpy()
    t["q"].ragged = rq.cpu().numpy()
    prob.policy = pol.cpu().numpy()
    ref = oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])
    expected = oracle.ST_BAD_OFFSET | oracle.ST_OUT_OF_SPAN | oracle.ST_BAD_POLICY
    assert ref["status"] == expected
    assert int(dev.status.item()) == expected
    compare_bf16(batch, "o", dev.host("o"), ref["o"], ref["o_written"], O_TOL)
    bref = oracle.backward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"],
                           t["dk"], t["dv"])
    for n in ("dq", "dk", "dv"):
        compare_bf16(batch, n, dev.host(n), bref[n], bref[n + "_written"], GRAD_TOL)


@pytest.mark.parametrize("seed", [310, 311])
def test_scaled_row_offsets_fwd_bwd(seed):
    """Offsets given as int32 row numbers times each tensor's token stride (one
    row array per side, shared by every tensor on it) address exactly what the
    int64 element offsets address: outputs are bit-identical to the
    element-offset run and match the oracle."""
    batch = workloads.random_batch(seed, batch=7, max_len=300, h_q=4, h_kv=2, dim=128,
                                   q_causal_offset=bool(seed % 2))
    say(f"[scaled] seed={seed}")
    elem = _dev(batch)
    elem.fwd()
    elem.bwd()
    sc = _dev(batch, scaled_offsets=True)
    assert sc.rows["q"] is sc.rows["o"] and sc.rows["k"] is sc.rows["dv"]
    sc.fwd()
    sc.bwd()
    torch.cuda.synchronize()
    assert int(sc.status.item()) == int(elem.status.item()) == 0
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(sc.flat[n].view(torch.int16 if n != "lse" else torch.int32),
                           elem.flat[n].view(torch.int16 if n != "lse" else torch.int32)), n
    check_forward(batch, sc)
    check_backward(batch, sc)


def test_scaled_offset_multiplier_is_applied_on_device():
    """The multiplier is applied by the setup kernel, before its offset checks:
    a Q multiplier of stride + 4 puts every sequence that starts on an odd row
    off the 16-byte grid (status BAD_OFFSET, outputs untouched) and moves the
    others to the rows the product names, exactly as the oracle reads them."""
    # packed rows (no NaN pad rows between sequences): the shifted rows of the
    # sequences that stay valid then read real data
    batch = workloads.random_batch(330, batch=6, max_len=60, zero_lengths=False, max_gap=0,
                                   token_gaps=False, h_q=2, h_kv=2, dim=64)
    lay_q = batch.layouts["q"]
    m = lay_q.stride_t + 4
    starts = lay_q.start_rows[:-1]
    assert (starts % 2 == 1).any() and (starts % 2 == 0).any()
    dev = _dev(batch, scaled_offsets=True)
    dev.rows["q"] = dev.rows["q"].clone()   # Q alone gets the odd multiplier
    dev.multiplier["q"] = m
    dev.fwd()
    torch.cuda.synchronize()
    prob, t = oracle.from_batch(batch)
    t["q"].ragged = lay_q.start_rows.astype(np.int64) * m
    ref = oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])
    assert ref["status"] & oracle.ST_BAD_OFFSET
    assert int(dev.status.item()) == ref["status"]
    compare_bf16(batch, "o", dev.host("o"), ref["o"], ref["o_written"], O_TOL)


def test_graph_capture_replays_match_eager():
    """The full forward and backward calls captured in one HIP graph (they
    allocate nothing and never synchronise): three replays, each on new Q and
    dO values written into the captured buffers, with eager work and a
    synchronisation between replays, each bit-identical to an eager run on
    the same inputs in separate buffers."""
    batch = workloads.random_batch(700, batch=6, max_len=300, h_q=4, h_kv=2, dim=128,
                                   window="random", q_causal_offset=True)
    say(f"[graph] lq={batch.lq.tolist()} window={batch.window.tolist()}")
    cap = _dev(batch)
    fws = torch.empty(cap.fwd_layout().total_bytes, dtype=torch.uint8, device="cuda")
    bws = torch.empty(cap.bwd_layout().total_bytes, dtype=torch.uint8, device="cuda")
    cap.fwd(workspace=fws)  # warm-up outside the capture
    cap.bwd(workspace=bws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap.fwd(workspace=fws)
        cap.bwd(workspace=bws)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(701)
    for rep in range(3):
        for n in ("q", "do"):
            fresh = torch.randn(cap.flat[n].shape, generator=gen, device="cuda")
            src = fresh.to(cap.flat[n].dtype)
            valid = ~torch.isnan(cap.flat[n].float())   # keep the NaN pad rows
            cap.flat[n].copy_(torch.where(valid, src, cap.flat[n]))
        ref = _dev(batch)
        for n in ("q", "do"):
            ref.flat[n].copy_(cap.flat[n])
        g.replay()
        ref.fwd()  # eager work between replays, on its own buffers
        ref.bwd()
        torch.cuda.synchronize()
        for n in ("o", "lse", "dq", "dk", "dv"):
            view = torch.int32 if n == "lse" else torch.int16
            assert torch.equal(cap.flat[n].view(view), ref.flat[n].view(view)), (rep, n)
        assert int(cap.status.item()) == int(ref.status.item()) == 0
    # and the last replay matches the oracle
    for n in ("q", "do"):
        batch.data[n] = cap.flat[n].view(torch.int16).cpu().numpy().view(np.uint16)
    check_forward(batch, cap)
    check_backward(batch, cap)


def test_workspace_and_output_guard_bands():
    """Canary bands of 4096 elements before and after the workspace and every
    output buffer (O, LSE, dQ, dK, dV) survive a forward and a backward
    (cudnn-frontend PR #462, "Why this was never caught (commit 2)": an
    out-of-bounds write past a buffer shows up only in a guard band)."""
    batch = workloads.random_batch(600, batch=5, max_len=300, dim=128)
    dev = _dev(batch, guard_elems=4096)
    for backward in (False, True):
        L = dev.bwd_layout() if backward else dev.fwd_layout()
        guard = 4096
        buf = torch.full((L.total_bytes + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
        ws = buf[guard:guard + L.total_bytes]
        if backward:
            dev.bwd(workspace=ws)
        else:
            dev.fwd(workspace=ws)
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        assert np.all(host[:guard] == 0xA5) and np.all(host[-guard:] == 0xA5), \
            f"workspace guard band overwritten (backward={backward})"
        intact = dev.guards_intact()
        assert all(intact.values()), f"output guard band overwritten: {intact}"
    check_forward(batch, dev)
    check_backward(batch, dev)


# ------------------------------------------------------------------ full-size configs

def _sample_rows(batch, rng, n_seq=6, per_seq=4):
    out = []
    order = rng.permutation(batch.batch)[:n_seq]
    for b in order:
        lq = int(batch.lq[b])
        if lq <= 0:
            continue
        rows = {0, lq - 1} | set(rng.integers(0, lq, size=per_seq - 2).tolist())
        h = int(rng.integers(0, batch.h_q))
        out.append((int(b), h, sorted(rows)))
    return out


def _check_sampled_fwd(batch, dev, seed):
    rng = np.random.default_rng(seed)
    prob, t = oracle.from_batch(batch)
    o_gpu = batch.layouts["o"].view(dev.host("o"))
    lse_gpu = batch.layouts["lse"].view(dev.host("lse"))[:, :, 0]
    worst = 0.0
    for b, h, rows in _sample_rows(batch, rng):
        o_ref, l_ref = oracle.forward_rows(prob, t["q"], t["k"], t["v"], b, h, rows)
        r0 = int(batch.layouts["o"].start_rows[b])
        rl = int(batch.layouts["lse"].start_rows[b])
        g = oracle.bits_to_f64(o_gpu[np.asarray(rows) + r0, h], batch.dtype)
        err = np.abs(g - o_ref).max()
        worst = max(worst, err)
        assert err <= O_TOL, (b, h, rows, err)
        np.testing.assert_allclose(lse_gpu[np.asarray(rows) + rl, h], l_ref, atol=1e-3, rtol=0)
    return worst


def _check_pads_untouched(batch, dev, names):
    for n in names:
        lay = batch.layouts[n]
        valid = workloads.valid_rows(lay, batch.lq if n in ("o", "lse", "dq") else batch.lk)
        got = lay.view(dev.host(n))
        pre = lay.view(pre_fill(batch, n))
        assert np.array_equal(got[~valid].view(np.uint8), pre[~valid].view(np.uint8)), n


def queue_heads(batch, n=8):
    """Query heads whose kv heads sit on n distinct XCD claim queues (queue x
    serves the kv heads g with g mod 8 == x), spread over the kv heads of a
    queue and over the query heads of a GQA group."""
    group = batch.h_q // batch.h_kv
    per_q = max(1, batch.h_kv // 8)
    heads = []
    for x in range(min(8, batch.h_kv)):
        g = x + 8 * ((3 * x) % per_q)
        heads.append(g * group + x % group)
    step = max(1, len(heads) // n)
    return heads[::step][:n]


def _check_fwd_heads(batch, dev, heads):
    """O and LSE of complete query heads (every row of every sequence)
    against the oracle, element by element; pads of every head untouched."""
    ref = oracle_fwd_heads(batch, heads)
    o_w, l_w = ref["o_written"], ref["lse_written"]
    assert o_w.any()
    g = oracle.bits_to_f64(dev.host("o")[o_w], batch.dtype)
    assert np.all(np.isfinite(g))
    err = float(np.abs(g - ref["o"][o_w]).max())
    gl = dev.host("lse")[l_w].astype(np.float64)
    rl = ref["lse"][l_w]
    dead = rl == -np.inf
    assert np.all(gl[dead] == -np.inf)
    lerr = float(np.abs(gl[~dead] - rl[~dead]).max()) if (~dead).any() else 0.0
    say(f"  heads {heads}: O max abs err {err:.3e}, LSE {lerr:.3e} over {int(l_w.sum())} rows")
    assert err <= O_TOL and lerr <= LSE_TOL
    _check_pads_untouched(batch, dev, ("o", "lse"))


def _check_bwd_heads(batch, dev, kv_heads):
    """Complete dQ, dK, dV of whole GQA groups against the oracle."""
    ref = oracle_bwd_heads(batch, kv_heads)
    for n in ("dq", "dk", "dv"):
        w = ref[n + "_written"]
        g = oracle.bits_to_f64(dev.host(n)[w], batch.dtype)
        err = np.abs(g - ref[n][w]).max()
        mag = np.abs(ref[n][w]).max()
        say(f"  {n}: max abs err {err:.3e}, max |ref| {mag:.3e}, over {int(w.sum())} elements")
        assert err <= GRAD_TOL
    _check_pads_untouched(batch, dev, ("dq", "dk", "dv"))


FULL_FWD_HEADS = {"packed_causal": 8, "padded_gqa": 8, "mixed_policy": 16, "long_context_cp": 4}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["packed_causal", "padded_gqa", "mixed_policy", "long_context_cp"])
def test_full_size_forward_complete_heads(name):
    """At full size, in the launch configuration the benchmark times: complete
    query heads spread over the XCD claim queues (the mixed-policy workload:
    every head), plus sampled rows of random heads."""
    batch = workloads.BY_NAME[name](with_grad=False)
    heads = list(range(batch.h_q)) if FULL_FWD_HEADS[name] >= batch.h_q else \
        queue_heads(batch, FULL_FWD_HEADS[name])
    say(f"[full fwd] {name}: B={batch.batch} lq_sum={int(batch.lq.sum())} heads {heads}")
    dev = _dev(batch, with_grad=False)
    dev.fwd()
    torch.cuda.synchronize()
    assert int(dev.status.item()) == 0
    _check_fwd_heads(batch, dev, heads)
    _check_sampled_fwd(batch, dev, seed=batch.seed)


@pytest.mark.timeout(600)
def test_full_size_sliding_window():
    """The benchmark's sliding-window workload at full size, in the launch
    configuration the benchmark times: complete forward heads and the complete
    gradients of kv heads on four queues."""
    batch = workloads.packed_causal_window(with_grad=True)
    say(f"[full window] B={batch.batch} lq_sum={int(batch.lq.sum())} window={batch.window.tolist()}")
    dev = _dev(batch, with_grad=True)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    assert int(dev.status.item()) == 0
    _check_fwd_heads(batch, dev, [7, 12, 21, 30])
    _check_bwd_heads(batch, dev, [7, 12, 21, 30])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,kv_heads", [("packed_causal", [0, 9, 18, 27]),
                                           ("padded_gqa", [0, 3, 5, 6]),
                                           ("long_context_cp", [3, 12])])
def test_full_size_backward_heads(name, kv_heads):
    """Complete gradients of kv heads on distinct XCD claim queues (kv head g
    on queue g mod 8) at full size, in the launch configuration the benchmark
    times (the packed causal workload is its headline)."""
    batch = workloads.BY_NAME[name](with_grad=True)
    say(f"[full bwd] {name} kv heads {kv_heads} (queues {sorted({g % 8 for g in kv_heads})})")
    dev = _dev(batch, with_grad=True)
    dev.fwd()
    dev.bwd()
    torch.cuda.synchronize()
    assert int(dev.status.item()) == 0
    _check_bwd_heads(batch, dev, kv_heads)
