"""Oracle of the setup step: per-sequence metadata and tile work lists.

TEST INFRASTRUCTURE (see ``oracle/attention.py``).  This is an independent
restatement of what the on-device setup step must produce, compared with it bit
for bit.  The pages ask for the per-sequence base rows to come from the bound
offsets on device, with no device-to-host read (cudnn-frontend issue on padded
THD, "Proposal": the setup step already writes device metadata and could read
the caller's ragged offsets; validating device prefix sums on the host would
need the read a previous change removed), with one base per tensor (the
metadata must widen beyond one cu_q/cu_k pair).  The list format and its order
are this library's own design:

* Per sequence b: ``lq, lk, policy, hi, lo, flags`` (int32) and one int64
  base per tensor in the order Q, K, V, O, LSE, dO, dQ, dK, dV (backward-only
  bases are 0 in a forward setup).  ``flags`` = 1 if the sequence is valid,
  plus its status bits shifted left by 8.  ``hi`` and ``lo`` fold the causal
  diagonal and the window into one band: key j is visible to row i iff
  ``i + lo <= j <= i + hi`` and ``j < lk``.  ``hi`` is the smallest of the
  causal diagonal (causal policies) and the window's upper offset (when
  bounded), ``lk`` when neither applies; ``lo`` is the window's lower offset,
  ``-lq`` when unbounded; both clamped to [-lq, lk], which changes no
  visibility and keeps them in int32.  Invalid sequences store 0 for both.
* Forward tile list (one int32 pair (b, t) per tile of ``bm`` query rows):
  valid sequences with ``lq > 0``, ordered by descending cost then ascending b,
  each sequence's tiles from last to first.  The cost of a sequence is the sum
  over its tiles of ``max(1, ceil(kv_end / bn) - floor(kv_begin / bn))``, the
  key range of the tile being ``kv_begin = clamp(row_start + lo, 0, lk)`` (its
  first row's lower bound) to ``kv_end = clamp(row_end + hi, 0, lk)`` (its last
  row's upper bound plus one).
* Backward kv groups: the valid sequences with ``lk > 0`` whose K, V, dK and
  dV bases are all equal, wherever they sit in the batch (segments binding the
  same K/V rows, e.g. context-parallel query chunks of one document).  Groups
  whose dK or dV row ranges intersect (``attention.kv_overlap``) are dropped:
  their members get ST_KV_OVERLAP, lose the valid flag, store hi = lo = 0 and
  leave both lists (the forward list of a backward setup feeds the dQ pass).
  The remaining groups are ordered by descending cost (sum of the members'
  costs under the backward tile sizes) then ascending first member.
* Member list (int32 per member): each group's members in ascending index,
  groups in that order.
* Backward kv-tile list (int32 quadruple (m_start, n_members, u, lk_max) per
  tile of ``bn_b`` key rows of a group): ``m_start`` is the position of the
  group's first member in the member list; tiles of a group in ascending u
  over ``ceil(lk_max / bn_b)``.
* If a list would exceed its capacity (more tiles than the output buffer's rows
  can hold, which only happens when sequences overlap), the overflow bit is set
  and both tile counts are 0: nothing is computed.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .attention import (ST_KV_OVERLAP, ST_LIST_OVERFLOW, Problem, SeqInfo, Tensor, kv_overlap,
                        sequence_info)

BASE_ORDER = ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv")


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def rows_capacity(t: Tensor) -> int:
    """Largest row count r such that row r-1 (all heads, all dims) still fits."""
    extra = (t.heads - 1) * t.stride_h + (t.dim - 1)
    return (t.span - 1 - extra) // t.stride_t + 1


def band(info: SeqInfo) -> tuple:
    """(hi, lo) of a sequence as the device table stores them."""
    if not info.valid:
        return 0, 0
    hi = info.lk
    if info.causal:
        hi = min(hi, info.diag)
    if info.win_hi is not None:
        hi = min(hi, info.win_hi)
    lo = -info.lq if info.win_lo is None else info.win_lo
    clamp = lambda x: min(max(x, -info.lq), info.lk)
    return clamp(hi), clamp(lo)


def tile_cost(lq: int, lk: int, hi: int, lo: int, bm: int, bn: int) -> int:
    cost = 0
    for t in range(ceil_div(lq, bm)):
        row_end = min(lq, (t + 1) * bm)
        kv_end = min(max(row_end + hi, 0), lk)
        kv_begin = min(max(t * bm + lo, 0), lk)
        cost += max(1, ceil_div(kv_end, bn) - kv_begin // bn)
    return cost


def setup(prob: Problem, tensors: dict, *, backward: bool, bm: int, bn: int,
          bm_b: int = 0, bn_b: int = 0, cap_fwd: int, cap_bwd: int = 0) -> dict:
    """Expected setup outputs.  ``tensors`` maps q k v o lse (+ do dq dk dv)
    to oracle Tensors."""
    if backward:
        q_side = [tensors[n] for n in ("q", "o", "lse", "do", "dq")]
        kv_side = [tensors[n] for n in ("k", "v", "dk", "dv")]
    else:
        q_side = [tensors[n] for n in ("q", "o", "lse")]
        kv_side = [tensors[n] for n in ("k", "v")]
    B = prob.batch
    lq = np.zeros(B, np.int32)
    lk = np.zeros(B, np.int32)
    pol = np.zeros(B, np.int32)
    hi = np.zeros(B, np.int32)
    lo = np.zeros(B, np.int32)
    flags = np.zeros(B, np.int32)
    base = np.zeros((9, B), np.int64)
    status = 0
    infos = [sequence_info(prob, q_side, kv_side, b) for b in range(B)]
    if backward:
        clash = kv_overlap(infos, *(tensors[n] for n in ("k", "v", "dk", "dv")))
        infos = [dataclasses.replace(i, status=i.status | ST_KV_OVERLAP) if c else i
                 for i, c in zip(infos, clash)]
    for b in range(B):
        info = infos[b]
        lq[b], lk[b], pol[b] = info.lq, info.lk, info.policy
        hi[b], lo[b] = band(info)
        flags[b] = (1 if info.valid else 0) | (info.status << 8)
        status |= info.status
        for i, n in enumerate(BASE_ORDER):
            if n in tensors and (backward or i < 5):
                base[i, b] = int(tensors[n].ragged[b])

    def cost_of(b, tm, tn):
        return tile_cost(infos[b].lq, infos[b].lk, int(hi[b]), int(lo[b]), tm, tn)

    listed = [b for b in range(B) if infos[b].valid and infos[b].lq > 0]
    order = sorted(listed, key=lambda b: (-cost_of(b, bm, bn), b))
    fwd = []
    for b in order:
        for t in range(ceil_div(infos[b].lq, bm) - 1, -1, -1):
            fwd.append((b, t))

    bwd, mlist = [], []
    if backward:
        groups = {}  # (K, V, dK, dV) bases -> members in ascending index
        for b in range(B):
            if infos[b].valid and infos[b].lk > 0:
                groups.setdefault(tuple(int(base[i, b]) for i in (1, 2, 7, 8)), []).append(b)
        glist = list(groups.values())
        gcost = [sum(cost_of(m, bm_b, bn_b) for m in g) for g in glist]
        for gi in sorted(range(len(glist)), key=lambda x: (-gcost[x], glist[x][0])):
            g = glist[gi]
            start = len(mlist)
            mlist.extend(g)
            lmax = max(infos[m].lk for m in g)
            for u in range(ceil_div(lmax, bn_b)):
                bwd.append((start, len(g), u, lmax))

    if len(fwd) > cap_fwd or (backward and len(bwd) > cap_bwd):
        status |= ST_LIST_OVERFLOW
        fwd, bwd, mlist = [], [], []
    return dict(lq=lq, lk=lk, policy=pol, hi=hi, lo=lo, flags=flags, base=base,
                fwd=np.asarray(fwd, np.int32).reshape(-1, 2),
                bwd=np.asarray(bwd, np.int32).reshape(-1, 4),
                members=np.asarray(mlist, np.int32), status=status, infos=infos)
