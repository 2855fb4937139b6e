"""Pins of the setup-step oracle (oracle/worklist.py) against hand-computed lists."""
from __future__ import annotations

import numpy as np

import oracle
from oracle import worklist


def _problem(lq, lk, policy, qco=None):
    B = len(lq)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    return oracle.Problem(1, 1, 8, 1.0, cu_q, cu_k, np.asarray(policy, np.int8), 0,
                          None if qco is None else np.asarray(qco, np.int32))


def _tensors(q_start, kv_start, q_rows, kv_rows, lse_rows=None, heads=1, dim=8):
    def t(rows, start, d=dim, st=None):
        st = heads * d if st is None else st
        return oracle.Tensor(np.zeros(rows * st, np.uint16 if d > 1 else np.float32), st, d,
                             np.asarray(start, np.int64) * st, heads, d)
    out = {n: t(q_rows, q_start) for n in ("q", "o", "do", "dq")}
    out.update({n: t(kv_rows, kv_start) for n in ("k", "v", "dk", "dv")})
    out["lse"] = t(q_rows if lse_rows is None else lse_rows, q_start, d=1)
    return out


def test_forward_and_backward_lists_by_hand():
    # lq [5,0,3,9], lk [5,2,7,4], policies [top-left, padding, bottom-right, padding]
    # bm = 4, bn = 2.  Costs (sum over q tiles of max(1, ceil(kv_end/2))):
    #   b0: tiles rows 0-3 -> kv_end 4 -> 2; row 4 -> kv_end 5 -> 3      => 5
    #   b1: no query rows                                                => 0 (not listed)
    #   b2: diag = 7-3 = 4; rows 0-2 -> kv_end min(3+4, 7) = 7 -> 4       => 4
    #   b3: padding, 3 tiles x ceil(4/2)=2                                => 6
    prob = _problem([5, 0, 3, 9], [5, 2, 7, 4], [1, 0, 2, 0])
    t = _tensors([0, 5, 5, 8, 17], [0, 5, 7, 14, 18], 17, 18)
    s = worklist.setup(prob, t, backward=True, bm=4, bn=2, bm_b=4, bn_b=2, cap_fwd=100,
                       cap_bwd=100)
    assert s["status"] == 0
    assert s["fwd"].tolist() == [[3, 2], [3, 1], [3, 0], [0, 1], [0, 0], [2, 0]]
    # kv groups: one per valid sequence with lk > 0 (bases all differ), ordered by
    # the same costs under (bm_b, bn_b) = (4, 2): b3 6, b0 5, b2 4, b1 0.  The
    # member list holds them in that order; an entry names its group's first
    # position in that list.
    assert s["members"].tolist() == [3, 0, 2, 1]
    assert s["bwd"].tolist() == [[0, 1, 0, 4], [0, 1, 1, 4],
                                 [1, 1, 0, 5], [1, 1, 1, 5], [1, 1, 2, 5],
                                 [2, 1, 0, 7], [2, 1, 1, 7], [2, 1, 2, 7], [2, 1, 3, 7],
                                 [3, 1, 0, 2]]
    # band (hi, lo): causal diagonal or lk above, -lq below (no windows)
    assert s["hi"].tolist() == [0, 2, 4, 4]
    assert s["lo"].tolist() == [-5, 0, -3, -9]
    assert s["flags"].tolist() == [1, 1, 1, 1]
    assert s["base"][0].tolist() == [0, 40, 40, 64]          # Q rows 0, 5, 5, 8 (x 8)
    assert s["base"][4].tolist() == [0, 5, 5, 8]             # LSE token stride 1


def test_aliasing_segments_form_one_kv_group():
    # four query chunks; chunks 0,1 bind K/V rows of document 0, chunks 2,3 of doc 1
    prob = _problem([4, 4, 4, 4], [16, 16, 16, 16], [1, 1, 1, 1], qco=[4, 12, 4, 12])
    t = _tensors([0, 4, 8, 12, 16], [0, 0, 16, 16, 32], 16, 32)
    s = worklist.setup(prob, t, backward=True, bm=4, bn=8, bm_b=4, bn_b=8, cap_fwd=100,
                       cap_bwd=100)
    # costs: chunk at offset 4: kv_end = 4+4 = 8 -> 1 tile; offset 12: 16 -> 2 tiles.
    assert s["fwd"].tolist() == [[1, 0], [3, 0], [0, 0], [2, 0]]
    # two groups of 2 members, cost 3 each -> ascending first member; 2 kv tiles each
    assert s["members"].tolist() == [0, 1, 2, 3]
    assert s["bwd"].tolist() == [[0, 2, 0, 16], [0, 2, 1, 16], [2, 2, 0, 16], [2, 2, 1, 16]]
    assert s["status"] == 0


def test_interleaved_chunks_and_a_skipped_member_still_form_one_group():
    # chunks of documents A (K/V rows 0..15) and B (rows 16..31) in the order
    # A0, B0, X, A1, B1, where X binds A's rows but has an unknown policy: the
    # groups are {0, 3} and {1, 4} by their bases, wherever the members sit.
    prob = _problem([4] * 5, [16] * 5, [1, 1, 9, 1, 1], qco=[4, 4, 4, 12, 12])
    t = _tensors([0, 4, 8, 12, 16, 20], [0, 16, 0, 0, 16, 32], 20, 32)
    s = worklist.setup(prob, t, backward=True, bm=4, bn=8, bm_b=4, bn_b=8, cap_fwd=100,
                       cap_bwd=100)
    assert s["status"] == oracle.ST_BAD_POLICY
    assert s["flags"].tolist() == [1, 1, oracle.ST_BAD_POLICY << 8, 1, 1]
    # backward costs (bm_b = 4, bn_b = 8): offset 4 -> 1 tile, offset 12 -> 2
    # tiles; both groups cost 3, so the one whose first member is 0 leads
    assert s["members"].tolist() == [0, 3, 1, 4]
    assert s["bwd"].tolist() == [[0, 2, 0, 16], [0, 2, 1, 16], [2, 2, 0, 16], [2, 2, 1, 16]]
    # forward tiles under (bm, bn) = (4, 8): a chunk at offset 12 reaches keys
    # 0..15 (2 tiles), one at offset 4 keys 0..7 (1 tile); X is not listed
    assert s["fwd"].tolist() == [[3, 0], [4, 0], [0, 0], [1, 0]]


def test_partially_overlapping_kv_groups_are_flagged_and_skipped():
    # b0 binds key rows 0..7, b1 rows 4..11 (different bases, overlapping
    # rows), b2 rows 12..15 (disjoint), b3 rows 16..19 and b4 rows 20..23
    # (touching b3's range, not overlapping it).
    prob = _problem([2] * 5, [8, 8, 4, 4, 4], [0] * 5)
    t = _tensors([0, 2, 4, 6, 8, 10], [0, 4, 12, 16, 20, 24], 10, 24)
    s = worklist.setup(prob, t, backward=True, bm=4, bn=8, bm_b=4, bn_b=8, cap_fwd=100,
                       cap_bwd=100)
    ov = oracle.ST_KV_OVERLAP
    assert s["status"] == ov
    assert s["flags"].tolist() == [ov << 8, ov << 8, 1, 1, 1]
    assert s["hi"].tolist()[:2] == [0, 0] and s["lo"].tolist()[:2] == [0, 0]
    assert s["members"].tolist() == [2, 3, 4]
    assert s["bwd"][:, 0].tolist() == [0, 1, 2] and s["fwd"][:, 0].tolist() == [2, 3, 4]
    # a forward setup does not look at key-side outputs at all
    f = worklist.setup(prob, t, backward=False, bm=4, bn=8, cap_fwd=100)
    assert f["status"] == 0 and f["fwd"][:, 0].tolist() == [0, 1, 2, 3, 4]


def test_same_key_rows_with_different_sources_overlap():
    # identical dK/dV rows but different K inputs: two groups writing the
    # same rows
    prob = _problem([2, 2], [4, 4], [0, 0])
    t = _tensors([0, 2, 4], [0, 0, 4], 4, 8)
    t["k"].ragged = np.array([0, 32, 64], np.int64)
    s = worklist.setup(prob, t, backward=True, bm=4, bn=8, bm_b=4, bn_b=8, cap_fwd=100,
                       cap_bwd=100)
    assert s["status"] == oracle.ST_KV_OVERLAP and s["bwd"].shape == (0, 4)


def test_invalid_and_overflow():
    prob = _problem([4, 4], [4, 4], [0, 7])
    t = _tensors([0, 4, 8], [0, 4, 8], 8, 8)
    s = worklist.setup(prob, t, backward=False, bm=2, bn=2, cap_fwd=100)
    assert s["status"] == oracle.ST_BAD_POLICY
    assert s["flags"].tolist() == [1, oracle.ST_BAD_POLICY << 8]
    assert s["fwd"].tolist() == [[0, 1], [0, 0]]
    s = worklist.setup(prob, t, backward=False, bm=2, bn=2, cap_fwd=1)
    assert s["status"] == oracle.ST_BAD_POLICY | oracle.ST_LIST_OVERFLOW
    assert s["fwd"].shape == (0, 2)


def test_rows_capacity():
    t = oracle.Tensor(np.zeros(13 * 2 * 64, np.uint16), 128, 64, np.zeros(4, np.int64), 2, 64)
    assert worklist.rows_capacity(t) == 13
    hm = oracle.Tensor(np.zeros(8 * 7360, np.float32), 1, 7360, np.zeros(2, np.int64), 8, 1)
    assert worklist.rows_capacity(hm) == 7360


def test_window_bands_and_costs_by_hand():
    # b0: top-left causal, lq = lk = 10, window (3, 0): hi = 0, lo = -3.
    #   bm = 4, bn = 2; tiles: rows 0-3 keys [0, 4) -> 2; rows 4-7 keys [1, 8)
    #   -> 4 - 0 = 4; rows 8-9 keys [5, 10) -> 5 - 2 = 3              => 9
    # b1: padding, lq = lk = 6, window (1, 1) anchored at lk - lq = 0: hi = 1,
    #   lo = -1; rows 0-3 keys [0, 5) -> 3; rows 4-5 keys [3, 6) -> 3 - 1 = 2
    #                                                                  => 5
    # b2: bottom-right, lq = 2, lk = 9, window (-1, 5): the diagonal 7 binds
    #   before the window's upper offset 7 + 5: hi = 7; lo = -lq = -2; rows
    #   0-1 keys [0, 9) -> 5                                            => 5
    prob = _problem([10, 6, 2], [10, 6, 9], [1, 0, 2])
    prob.window = np.array([[1, 1], [3, 0], [-1, 5]], np.int32)
    t = _tensors([0, 10, 16, 18], [0, 10, 16, 25], 18, 25)
    s = worklist.setup(prob, t, backward=False, bm=4, bn=2, cap_fwd=100)
    assert s["status"] == 0
    assert s["hi"].tolist() == [0, 1, 7]
    assert s["lo"].tolist() == [-3, -1, -2]
    assert s["fwd"].tolist() == [[0, 2], [0, 1], [0, 0], [1, 1], [1, 0], [2, 0]]


def test_window_lower_offset_and_clamps_by_hand():
    # One padding sequence lq = 3, lk = 4 with window (0, -1): anchor lk - lq =
    # 1, so row i sees keys >= i + 1: lo = 1, hi = lk = 4.
    prob = _problem([3], [4], [0])
    prob.window = np.array([[0, -1], [-1, -1], [-1, -1]], np.int32)
    t = _tensors([0, 3], [0, 4], 3, 4)
    s = worklist.setup(prob, t, backward=False, bm=4, bn=2, cap_fwd=100)
    assert (s["hi"].tolist(), s["lo"].tolist()) == ([4], [1])
    # A window far past the keys: lo = 100 clamps to lk = 4 (nothing visible);
    # one far before them: hi = -100 clamps to -lq = -3.
    prob.window = np.array([[-1, -1], [-1, -1], [-1, -1]], np.int32)
    prob.q_causal_offset = np.array([103], np.int32)
    prob.window[0] = [3, -1]
    s = worklist.setup(prob, t, backward=False, bm=4, bn=2, cap_fwd=100)
    assert (s["hi"].tolist(), s["lo"].tolist()) == ([4], [4])
    prob.q_causal_offset = np.array([-103], np.int32)
    prob.window[0] = [-1, 3]
    s = worklist.setup(prob, t, backward=False, bm=4, bn=2, cap_fwd=100)
    assert (s["hi"].tolist(), s["lo"].tolist()) == ([-3], [-3])
