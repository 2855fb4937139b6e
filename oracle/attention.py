"""Plain fp64 CPU oracle: scaled-dot-product attention over ragged THD batches.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP path and the HIP path never calls it.

What is computed, and where the pages fix it
--------------------------------------------
* Addressing.  Row ``i`` of sequence ``b`` in tensor X, head ``h``, dim ``d``
  sits at element ``X.ragged[b] + i*X.stride_t + h*X.stride_h + d``.  The base
  comes from the caller-bound ragged-offset tensor of *that* tensor, never from
  a prefix sum of lengths (cudnn-frontend issue "THD lowering ignores the bound
  ragged offsets", sections "Concrete failure" and "Proposal: consume the bound
  offsets on device"; per-tensor offsets so Q/O padding may differ from K/V).
  Offsets are in elements (the search answer quoted in the review of
  cudnn-frontend PR #462: offsets count elements, entry B is past-the-end).
* Lengths.  ``Lq = cu_q[b+1]-cu_q[b]``, ``Lk = cu_kv[b+1]-cu_kv[b]``; they
  bound the mask and decide dead rows (issue above, "Proposal": lengths are
  still needed for mask bounds and the dead-row path).
* Mask.  Key j is allowed for row i iff ``j < Lk`` and (policy is padding, or
  ``j <= i + delta_b``).  ``delta_b`` is 0 for top-left causal (Megatron-LM
  PR #14 commit message: top-left keeps j <= i), ``Lk - Lq`` for bottom-right
  (same message: a segment's q[0] sits at doc-local key Lk - Lq), and the
  caller's per-segment ``q_causal_offset[b]`` when given (same message: the
  absolute key index of the segment's local q[0]).  The policy is chosen per
  sequence (TransformerEngine PR #3274, "Description" and the reviewer's
  padding/causal/bottom-right mapping).
* Sliding window (same PR, "Description": a window size per mask type beside
  the per-sequence policy).  Policy p may carry a window (left_p, right_p),
  -1 meaning unbounded on that side.  With the anchor ``a_b`` (the key index
  of the sequence's row 0: ``q_causal_offset[b]`` when given, else 0 for
  top-left and ``Lk - Lq`` for bottom-right and padding), key j is further
  restricted to ``i + a_b - left <= j`` and ``j <= i + a_b + right`` for the
  bounded sides.  The rule intersects with the causal one.
* Forward (textbook definition, no online softmax):
  ``S = scale * Q_b K_bT``; masked entries -inf; ``LSE_i = M_i + ln sum_j
  exp(S_ij - M_i)``; ``P = exp(S - LSE)``; ``O = P V_b``.
* Backward (chain rule of the above): ``delta_i = sum_d dO_id O_id``;
  ``dV = P^T dO``; ``dP = dO V^T``; ``dS = P o (dP - delta)``;
  ``dQ = scale dS K``; ``dK = scale dS^T Q``.  dK/dV of a kv head sum over the
  q heads of its GQA group and over every segment that binds the same K/V
  rows.

Readings where the pages are silent (each listed in the design notes):
  softmax scale is an input (default 1/sqrt(D)); LSE is the natural-log
  log-sum-exp of the scaled, masked scores; a row with no allowed key is dead:
  O = 0, LSE = -inf, dQ = 0 and no dK/dV contribution; elements outside valid
  rows are never written; ``q_causal_offset`` moves the diagonal of causal
  sequences (a padding sequence has none); GQA groups are contiguous (kv head = h // (H_q // H_kv));
  windows of padding sequences anchor bottom-right (so self-attention windows
  are centred on the row), and ``q_causal_offset``, when given, anchors the
  windows of every policy.

The oracle may work on blocks of query rows and skip key columns masked for
every row of the block; each row's softmax is still computed whole, so this is
memory management, not a reformulation.  Sums over segments / q heads / row
blocks are in fp64 and differ from any other order only by rounding.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

PADDING = 0
CAUSAL_TOP_LEFT = 1
CAUSAL_BOTTOM_RIGHT = 2

# Device-data status bits (per sequence, ORed into the call's status word).
ST_NEG_LENGTH = 1 << 0     # Lq < 0 or Lk < 0
ST_BAD_OFFSET = 1 << 1     # ragged offset negative or not 16-byte aligned
ST_OUT_OF_SPAN = 1 << 2    # a row of the sequence would leave the buffer
ST_BAD_POLICY = 1 << 3     # policy value outside {0, 1, 2}
ST_LIST_OVERFLOW = 1 << 4  # more tiles than the output buffer can hold
ST_KV_OVERLAP = 1 << 5     # backward: key-side gradient rows shared with another kv group

ROW_BLOCK = 512


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE binary16 bit patterns (uint16) to float64."""
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit patterns of `dtype` ("bf16" or "f16")."""
    return bf16_bits_to_f64(bits) if dtype == "bf16" else f16_bits_to_f64(bits)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Tensor:
    """A ragged tensor as the caller binds it: flat buffer + strides + offsets."""

    data: np.ndarray        # flat: uint16 bf16/fp16 bits, float32 (LSE) or float64
    stride_t: int
    stride_h: int
    ragged: np.ndarray      # int64 [B+1] element offsets
    heads: int
    dim: int                # D for 16-bit tensors, 1 for LSE
    dtype: str = "bf16"     # element type of uint16 data: "bf16" or "f16"

    @property
    def span(self) -> int:
        return int(self.data.size)

    @property
    def align(self) -> int:
        # 16-bit rows are read 16 bytes at a time: offsets must be multiples of 8
        return 8 if self.data.dtype == np.uint16 else 1

    def index(self, base: int, rows: int, head: int) -> np.ndarray:
        """Element indices [rows, dim] of one head of one sequence."""
        r = np.arange(rows, dtype=np.int64)[:, None] * self.stride_t
        d = np.arange(self.dim, dtype=np.int64)[None, :]
        return base + head * self.stride_h + r + d

    def values(self) -> np.ndarray:
        """Buffer contents as float64 (16-bit patterns widened exactly)."""
        return self.values_at(slice(None))

    def values_at(self, idx) -> np.ndarray:
        """Elements at `idx` as float64 (16-bit patterns widened exactly)."""
        if self.data.dtype == np.uint16:
            return bits_to_f64(self.data[idx], self.dtype)
        return self.data[idx].astype(np.float64)


@dataclass
class Problem:
    h_q: int
    h_kv: int
    head_dim: int
    scale: float
    cu_q: np.ndarray                 # int32 [B+1]
    cu_kv: np.ndarray                # int32 [B+1]
    policy: np.ndarray | None        # int8 [B]
    default_policy: int
    q_causal_offset: np.ndarray | None  # int32 [B]
    window: np.ndarray | None = None    # int32 [3, 2]: (left, right) per policy, -1 unbounded

    @property
    def batch(self) -> int:
        return int(self.cu_q.size) - 1


@dataclass
class SeqInfo:
    lq: int
    lk: int
    policy: int
    diag: int        # causal diagonal delta_b (0 for padding)
    status: int      # OR of ST_* bits for this sequence
    win_lo: int | None = None  # window: keys j >= i + win_lo (None: unbounded)
    win_hi: int | None = None  # window: keys j <= i + win_hi (None: unbounded)

    @property
    def valid(self) -> bool:
        return self.status == 0

    @property
    def causal(self) -> bool:
        return self.policy in (CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT)


def _check_tensor(t: Tensor, base: int, rows: int) -> int:
    if base < 0 or base % t.align != 0:
        return ST_BAD_OFFSET
    last = base + (rows - 1) * t.stride_t + (t.heads - 1) * t.stride_h + (t.dim - 1)
    return ST_OUT_OF_SPAN if last >= t.span else 0


def sequence_info(prob: Problem, q_side: list, kv_side: list, b: int) -> SeqInfo:
    """Lengths, policy, diagonal and validity of sequence b.

    ``q_side``/``kv_side`` are the tensors addressed with the query-side rows
    (Q, O, LSE and in the backward dO, dQ) and the key-side rows (K, V, and in
    the backward dK, dV).  A tensor is checked only when its sequence has rows."""
    lq = int(prob.cu_q[b + 1]) - int(prob.cu_q[b])
    lk = int(prob.cu_kv[b + 1]) - int(prob.cu_kv[b])
    pol = int(prob.policy[b]) if prob.policy is not None else int(prob.default_policy)
    st = 0
    if lq < 0 or lk < 0:
        st |= ST_NEG_LENGTH
    if pol not in (PADDING, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT):
        st |= ST_BAD_POLICY
    if lq > 0:
        for t in q_side:
            st |= _check_tensor(t, int(t.ragged[b]), lq)
    if lk > 0:
        for t in kv_side:
            st |= _check_tensor(t, int(t.ragged[b]), lk)
    diag = 0
    if pol in (CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT):
        if prob.q_causal_offset is not None:
            diag = int(prob.q_causal_offset[b])
        elif pol == CAUSAL_BOTTOM_RIGHT:
            diag = lk - lq
    win_lo = win_hi = None
    if prob.window is not None and pol in (PADDING, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT):
        left, right = (int(x) for x in prob.window[pol])
        if prob.q_causal_offset is not None:
            anchor = int(prob.q_causal_offset[b])
        elif pol == CAUSAL_TOP_LEFT:
            anchor = 0
        else:
            anchor = lk - lq
        if left >= 0:
            win_lo = anchor - left
        if right >= 0:
            win_hi = anchor + right
    return SeqInfo(lq, lk, pol, diag, st, win_lo, win_hi)


def allowed(info: SeqInfo, rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Boolean [len(rows), len(keys)]: the mask rule for one sequence."""
    keep = (keys[None, :] < info.lk) & (keys[None, :] >= 0)
    keep = np.broadcast_to(keep, (rows.size, keys.size))
    if info.causal:
        keep = keep & (keys[None, :] <= rows[:, None] + info.diag)
    if info.win_hi is not None:
        keep = keep & (keys[None, :] <= rows[:, None] + info.win_hi)
    if info.win_lo is not None:
        keep = keep & (keys[None, :] >= rows[:, None] + info.win_lo)
    return keep


def _key_limit(info: SeqInfo, row_end: int) -> int:
    """Keys at or beyond this index are masked for every row < row_end."""
    last = info.lk - 1
    if info.causal:
        last = min(last, row_end - 1 + info.diag)
    if info.win_hi is not None:
        last = min(last, row_end - 1 + info.win_hi)
    return int(np.clip(last + 1, 0, info.lk))


def _key_start(info: SeqInfo, row_start: int) -> int:
    """Keys below this index are masked for every row >= row_start."""
    if info.win_lo is None:
        return 0
    return int(np.clip(row_start + info.win_lo, 0, info.lk))


def _softmax_block(info: SeqInfo, scale: float, qb: np.ndarray, kb: np.ndarray, r0: int,
                   k0: int = 0):
    """Scores, LSE and probabilities for query rows r0.. of one head against
    keys k0.. (the keys outside [k0, k0 + len(kb)) being masked for these rows)."""
    rows = np.arange(r0, r0 + qb.shape[0])
    keys = np.arange(k0, k0 + kb.shape[0])
    s = scale * (qb @ kb.T)
    keep = allowed(info, rows, keys)
    s = np.where(keep, s, -np.inf)
    live = keep.any(axis=1)
    m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(live, m + np.log(np.exp(s - m[:, None]).sum(axis=1)), -np.inf)
    p = np.where(keep, np.exp(s - np.where(live, lse, 0.0)[:, None]), 0.0)
    return lse, p


def _gather(t: Tensor, base: int, rows: int, head: int) -> np.ndarray:
    """Rows [rows, dim] of one head of one sequence, widened to float64."""
    if rows <= 0:
        return np.zeros((0, t.dim))
    return t.values_at(t.index(base, rows, head))


def forward(prob: Problem, q: Tensor, k: Tensor, v: Tensor, o: Tensor, lse: Tensor,
            heads=None, seqs=None):
    """Oracle forward.  Returns a dict with the O and LSE buffers after the
    call (fp64; unwritten elements keep their original value), boolean masks of
    the elements written, the per-sequence info and the OR of status bits.

    ``heads``/``seqs`` restrict the work to a subset (sampling at full size);
    restricted outputs are only meaningful on the written elements."""
    o_out, lse_out = o.values(), lse.values()
    o_w = np.zeros(o.span, bool)
    lse_w = np.zeros(lse.span, bool)
    group = prob.h_q // prob.h_kv
    status = 0
    infos = []
    for b in range(prob.batch):
        info = sequence_info(prob, [q, o, lse], [k, v], b)
        infos.append(info)
        status |= info.status
        if not info.valid or info.lq == 0 or (seqs is not None and b not in seqs):
            continue
        for h in (range(prob.h_q) if heads is None else heads):
            g = h // group
            for r0 in range(0, info.lq, ROW_BLOCK):
                r1 = min(info.lq, r0 + ROW_BLOCK)
                ks, kl = _key_start(info, r0), _key_limit(info, r1)
                kl = max(kl, ks)
                qb = _gather(q, int(q.ragged[b]) + r0 * q.stride_t, r1 - r0, h)
                kb = _gather(k, int(k.ragged[b]) + ks * k.stride_t, kl - ks, g)
                vb = _gather(v, int(v.ragged[b]) + ks * v.stride_t, kl - ks, g)
                lse_b, p = _softmax_block(info, prob.scale, qb, kb, r0, ks)
                ob = p @ vb if kl > ks else np.zeros((r1 - r0, prob.head_dim))
                oi = o.index(int(o.ragged[b]) + r0 * o.stride_t, r1 - r0, h)
                o_out[oi] = ob
                o_w[oi] = True
                li = lse.index(int(lse.ragged[b]) + r0 * lse.stride_t, r1 - r0, h)[:, 0]
                lse_out[li] = lse_b
                lse_w[li] = True
    return dict(o=o_out, o_written=o_w, lse=lse_out, lse_written=lse_w,
                status=status, infos=infos)


def forward_rows(prob: Problem, q: Tensor, k: Tensor, v: Tensor, b: int, h: int, rows):
    """O (fp64 [n, D]) and LSE ([n]) of selected rows of one (sequence, head);
    for sampled checks at sizes where the full oracle would be slow."""
    info = sequence_info(prob, [q], [k, v], b)
    rows = np.asarray(rows, np.int64)
    g = h // (prob.h_q // prob.h_kv)
    out_o = np.zeros((rows.size, prob.head_dim))
    out_l = np.full(rows.size, -np.inf)
    for n, i in enumerate(rows):
        ks, kl = _key_start(info, int(i)), _key_limit(info, int(i) + 1)
        kl = max(kl, ks)
        qi = _gather(q, int(q.ragged[b]) + int(i) * q.stride_t, 1, h)
        kb = _gather(k, int(k.ragged[b]) + ks * k.stride_t, kl - ks, g)
        vb = _gather(v, int(v.ragged[b]) + ks * v.stride_t, kl - ks, g)
        lse_i, p = _softmax_block(info, prob.scale, qi, kb, int(i), ks)
        out_l[n] = lse_i[0]
        if kl > ks:
            out_o[n] = (p @ vb)[0]
    return out_o, out_l


def kv_overlap(infos: list, k: Tensor, v: Tensor, dk: Tensor, dv: Tensor) -> list:
    """Which sequences the backward must skip because their key-side gradient
    rows collide with those of other sequences.

    Several query segments may bind the same key rows: context-parallel query
    chunks of one document share its key prefix (Megatron-LM PR #14, commit
    message), and their dK/dV are the sums over those segments.  Segments
    whose K, V, dK and dV offsets are all identical form one kv group,
    wherever they sit in the batch.  A group owns rows [0, Lk_max) of its dK
    and dV tensors, Lk_max being its members' largest key length, i.e. the
    element range [offset, offset + Lk_max * stride_t) of each.  When two
    groups' ranges intersect in dK or in dV, their gradients cannot both be
    stored (one would overwrite the other without any error: the silent
    mis-service of the cudnn-frontend issue on padded THD, "Concrete
    failure"), so every member of both groups is flagged instead.  Only
    valid sequences with key rows take part.  Returns a list of bools."""
    B = len(infos)
    members = [b for b in range(B) if infos[b].valid and infos[b].lk > 0]
    key = {b: tuple(int(t.ragged[b]) for t in (k, v, dk, dv)) for b in members}
    lk_max = {}
    for b in members:
        lk_max[key[b]] = max(lk_max.get(key[b], 0), infos[b].lk)
    groups = sorted(lk_max)
    hit = set()
    for ga in groups:
        for gb in groups:
            if ga == gb:
                continue
            for pos, t in ((2, dk), (3, dv)):
                a0, b0 = ga[pos], gb[pos]
                a1 = a0 + lk_max[ga] * t.stride_t
                b1 = b0 + lk_max[gb] * t.stride_t
                if a0 < b1 and b0 < a1:
                    hit.add(ga)
    return [b in key and key[b] in hit for b in range(B)]


def backward(prob: Problem, q: Tensor, k: Tensor, v: Tensor, o: Tensor, lse: Tensor,
             do: Tensor, dq: Tensor, dk: Tensor, dv: Tensor, kv_heads=None):
    """Oracle backward: the exact gradients of sum(dO * O) with respect to
    Q, K and V, O being the oracle's own fp64 forward output.

    Returns the dQ/dK/dV buffers after the call (fp64; unwritten elements keep
    their original values), boolean written masks, per-sequence info and the
    status bits.  dK/dV rows of valid key-side rows are written even when no
    query reaches them (their gradient is 0).  ``kv_heads`` restricts the work
    to whole GQA groups.  ``o`` and ``lse`` (the forward's outputs, inputs of
    the backward) take part in the validation of each sequence only; the
    oracle recomputes both in fp64.  Sequences that ``kv_overlap`` flags get
    ST_KV_OVERLAP and are skipped like any invalid sequence."""
    dq_out, dk_out, dv_out = dq.values(), dk.values(), dv.values()
    dq_w = np.zeros(dq.span, bool)
    dk_w = np.zeros(dk.span, bool)
    dv_w = np.zeros(dv.span, bool)
    group = prob.h_q // prob.h_kv
    gsel = range(prob.h_kv) if kv_heads is None else kv_heads
    status = 0
    # Key-side gradients accumulate in fp64 over every segment and q head that
    # reaches them, so that segments binding the same K/V rows sum.
    dk_acc = np.zeros(dk.span)
    dv_acc = np.zeros(dv.span)
    infos = [sequence_info(prob, [q, o, lse, do, dq], [k, v, dk, dv], b)
             for b in range(prob.batch)]
    for b, clash in enumerate(kv_overlap(infos, k, v, dk, dv)):
        if clash:
            infos[b].status |= ST_KV_OVERLAP
    for b in range(prob.batch):
        info = infos[b]
        status |= info.status
        if not info.valid:
            continue
        for g in gsel:
            if info.lk > 0:
                dki = dk.index(int(dk.ragged[b]), info.lk, g)
                dvi = dv.index(int(dv.ragged[b]), info.lk, g)
                dk_w[dki] = True
                dv_w[dvi] = True
            for h in range(g * group, (g + 1) * group):
                if info.lq == 0:
                    continue
                for r0 in range(0, info.lq, ROW_BLOCK):
                    r1 = min(info.lq, r0 + ROW_BLOCK)
                    n = r1 - r0
                    ks, kl = _key_start(info, r0), _key_limit(info, r1)
                    qb = _gather(q, int(q.ragged[b]) + r0 * q.stride_t, n, h)
                    dob = _gather(do, int(do.ragged[b]) + r0 * do.stride_t, n, h)
                    dqi = dq.index(int(dq.ragged[b]) + r0 * dq.stride_t, n, h)
                    dq_w[dqi] = True
                    if kl <= ks:
                        dq_out[dqi] = 0.0
                        continue
                    kb = _gather(k, int(k.ragged[b]) + ks * k.stride_t, kl - ks, g)
                    vb = _gather(v, int(v.ragged[b]) + ks * v.stride_t, kl - ks, g)
                    _, p = _softmax_block(info, prob.scale, qb, kb, r0, ks)
                    ob = p @ vb
                    delta = (dob * ob).sum(axis=1)
                    dp = dob @ vb.T
                    ds = p * (dp - delta[:, None])
                    dq_out[dqi] = prob.scale * (ds @ kb)
                    dk_acc[dk.index(int(dk.ragged[b]) + ks * dk.stride_t, kl - ks, g)] += \
                        prob.scale * (ds.T @ qb)
                    dv_acc[dv.index(int(dv.ragged[b]) + ks * dv.stride_t, kl - ks, g)] += p.T @ dob
    dk_out[dk_w] = dk_acc[dk_w]
    dv_out[dv_w] = dv_acc[dv_w]
    return dict(dq=dq_out, dq_written=dq_w, dk=dk_out, dk_written=dk_w,
                dv=dv_out, dv_written=dv_w, status=status, infos=infos)
