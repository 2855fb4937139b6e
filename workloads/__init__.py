"""Seeded synthetic ragged THD batches shared by the tests, the bench and smoke().

This module only *constructs inputs*: sequence lengths, where each sequence's
rows live in its buffers (the caller-bound ragged offsets), bf16 or fp16 bit
patterns drawn from N(0, 1), and NaN-filled pad rows.  It holds none of the attention
arithmetic, so it can feed both the HIP path and the CPU oracle without
coupling them.

Buffers are flat ``uint16`` arrays of bf16 (default) or fp16 bit patterns
(LSE: ``float32``).  A
buffer layout gives, per tensor, the element strides between tokens and heads
(the dim stride is always 1) and the row at which each sequence starts; the
ragged offsets handed to the library are ``start_row * stride_t`` in elements.

Workloads (seeded, config k uses seed 1000 + k):

1. three sequences [3, 2, 4] in a 13-row buffer, start rows [0, 4, 8, 13]
   (the padded layout with identifier tokens between sequences), H=2, D=64;
2. 16 packed causal sequences, lengths U[128, 4096], H=32, D=128;
3. 32 sequences, lengths U[64, 2048], a U{0..63}-row gap after each sequence,
   drawn separately for the Q/O/dO/dQ buffers and the K/V/dK/dV buffers,
   H_q=32, H_kv=8, D=128, causal;
4. 64 sequences, Lq U[32, 1024], Lk = Lq + U[0, 1024], a per-sequence policy
   U{padding, causal top-left, causal bottom-right}, H=16, D=128;
5. two 65536-key documents, each queried by two 4096-row chunks whose first
   query sits at absolute key 4096 and 61440 (per-segment q causal offsets);
   the two chunks of one document bind the same K/V rows.  H=16, D=128.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

# Mask policy encoding of the library interface.
PADDING = 0
CAUSAL_TOP_LEFT = 1
CAUSAL_BOTTOM_RIGHT = 2

BF16_PAD_NAN = 0x7FC0     # fills pad rows / gap columns of input buffers
BF16_OUT_NAN = 0x7FC1     # pre-fill of bf16 output buffers (distinct payload)
F16_PAD_NAN = 0x7E00      # the same two for fp16 buffers
F16_OUT_NAN = 0x7E01
F32_OUT_NAN = 0x7FC00011  # pre-fill of fp32 LSE buffers
PAD_NAN = {"bf16": BF16_PAD_NAN, "f16": F16_PAD_NAN}
OUT_NAN = {"bf16": BF16_OUT_NAN, "f16": F16_OUT_NAN}
TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}


@dataclass
class Layout:
    """Where the rows of one ragged tensor live inside its flat buffer."""

    rows: int                 # physical rows in the buffer
    heads: int
    dim: int                  # elements per (row, head): D, or 1 for LSE
    stride_t: int             # elements between consecutive rows
    stride_h: int             # elements between consecutive heads
    start_rows: np.ndarray    # int64 [B+1]; entry B is the past-the-end row
    span: int                 # addressable elements of the buffer

    @property
    def ragged(self) -> np.ndarray:
        """Element offset of row 0 of each sequence (entry B: past-the-end)."""
        return (self.start_rows.astype(np.int64) * self.stride_t).astype(np.int64)

    def view(self, flat: np.ndarray) -> np.ndarray:
        """Writable (rows, heads, dim) view of a flat buffer with this layout."""
        assert flat.size >= self.span
        it = flat.itemsize
        return np.lib.stride_tricks.as_strided(
            flat, shape=(self.rows, self.heads, self.dim),
            strides=(self.stride_t * it, self.stride_h * it, it))


def token_major(rows, heads, dim, start_rows, gap_tokens=0) -> Layout:
    """[T, H, D] rows; token stride H*D*(1 + gap_tokens) (gap n = 0..3 models
    the [T, n+1, H, D] interleaved views of a fused projection)."""
    st = heads * dim * (1 + gap_tokens)
    return Layout(rows, heads, dim, st, dim, np.asarray(start_rows, np.int64), rows * st)


def head_major(rows, heads, dim, start_rows) -> Layout:
    """[H, T, D] rows (for LSE, dim=1: the [h, t] softmax-stats layout)."""
    return Layout(rows, heads, dim, dim, rows * dim, np.asarray(start_rows, np.int64),
                  heads * rows * dim)


def lse_layout(kind: str, rows: int, heads: int, start_rows) -> Layout:
    if kind == "token":
        return token_major(rows, heads, 1, start_rows)
    if kind == "head":
        return head_major(rows, heads, 1, start_rows)
    raise ValueError(kind)


def _randn_bits(shape, gen: torch.Generator, dtype: str) -> np.ndarray:
    """N(0, 1) in fp32, rounded to nearest even in `dtype`, as bit patterns."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    return x.to(TORCH_DTYPE[dtype]).view(torch.int16).numpy().view(np.uint16)


def fill_buffer(layout: Layout, lengths: np.ndarray, gen: torch.Generator,
                dtype: str = "bf16") -> np.ndarray:
    """Flat bf16/fp16 buffer: N(0,1) in each sequence's valid rows, NaN elsewhere.

    Values are drawn for every physical row (so they depend on the seed and the
    buffer size only), then every element outside a valid row is NaN."""
    vals = _randn_bits((layout.rows, layout.heads, layout.dim), gen, dtype)
    flat = np.full(layout.span, PAD_NAN[dtype], dtype=np.uint16)
    valid = valid_rows(layout, lengths)
    v = layout.view(flat)
    v[valid] = vals[valid]
    return flat


def valid_rows(layout: Layout, lengths: np.ndarray) -> np.ndarray:
    """Boolean [rows]: True for rows that belong to some sequence."""
    valid = np.zeros(layout.rows, dtype=bool)
    for b, n in enumerate(np.asarray(lengths)):
        s = int(layout.start_rows[b])
        if n > 0:
            valid[s:s + int(n)] = True
    return valid


def out_buffer(layout: Layout, kind: str = "bf16") -> np.ndarray:
    """An output buffer pre-filled with the NaN payload of its kind
    ("bf16", "f16" or "f32")."""
    if kind in OUT_NAN:
        return np.full(layout.span, OUT_NAN[kind], dtype=np.uint16)
    return np.full(layout.span, F32_OUT_NAN, dtype=np.uint32).view(np.float32)


@dataclass
class Batch:
    """One synthetic problem: lengths, policies, layouts and input bytes."""

    name: str
    seed: int
    h_q: int
    h_kv: int
    dim: int
    scale: float
    lq: np.ndarray                  # int64 [B] valid query rows per sequence
    lk: np.ndarray                  # int64 [B] valid key rows per sequence
    default_policy: int
    policy: np.ndarray | None       # int8 [B] or None
    q_causal_offset: np.ndarray | None  # int32 [B] or None
    layouts: dict = field(default_factory=dict)   # q k v o lse do dq dk dv
    data: dict = field(default_factory=dict)      # q k v do -> flat uint16
    window: np.ndarray | None = None  # int32 [3, 2] (left, right) per policy, -1 unbounded
    dtype: str = "bf16"               # element type of Q, K, V, O, dO, dQ, dK, dV

    @property
    def batch(self) -> int:
        return int(self.lq.size)

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lq)]).astype(np.int32)

    @property
    def cu_kv(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lk)]).astype(np.int32)

    def ragged(self, name: str) -> np.ndarray:
        return self.layouts[name].ragged


def _prefix(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int64)


def _with_gaps(lengths, gaps) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64) + np.asarray(gaps, np.int64))])


def build(name, seed, h_q, h_kv, dim, lq, lk, q_start, kv_start, *, default_policy,
          policy=None, q_causal_offset=None, lse_kind="token", scale=None,
          q_rows=None, kv_rows=None, token_gaps=None, with_grad=True, window=None,
          dtype="bf16") -> Batch:
    """Assemble a batch from lengths and start rows.

    ``token_gaps`` maps tensor name -> n, giving that tensor a token stride of
    (1+n)*H*D; the default is packed rows (n=0).  Q, O, dO and dQ share the
    query-side start rows; K, V, dK and dV the key-side ones."""
    lq = np.asarray(lq, np.int64)
    lk = np.asarray(lk, np.int64)
    q_start = np.asarray(q_start, np.int64)
    kv_start = np.asarray(kv_start, np.int64)
    q_rows = int(q_start[-1] if q_rows is None else q_rows)
    kv_rows = int(kv_start[-1] if kv_rows is None else kv_rows)
    gaps = dict(token_gaps or {})
    lay = {}
    for n in ("q", "o", "do", "dq"):
        lay[n] = token_major(q_rows, h_q, dim, q_start, gaps.get(n, 0))
    for n in ("k", "v", "dk", "dv"):
        lay[n] = token_major(kv_rows, h_kv, dim, kv_start, gaps.get(n, 0))
    lay["lse"] = lse_layout(lse_kind, q_rows, h_q, q_start)
    b = Batch(name, seed, h_q, h_kv, dim, float(scale if scale is not None else dim ** -0.5),
              lq, lk, int(default_policy),
              None if policy is None else np.asarray(policy, np.int8),
              None if q_causal_offset is None else np.asarray(q_causal_offset, np.int32),
              lay, {}, None if window is None else np.asarray(window, np.int32).reshape(3, 2),
              dtype)
    g = torch.Generator().manual_seed(seed)
    b.data["q"] = fill_buffer(lay["q"], lq, g, dtype)
    b.data["k"] = fill_buffer(lay["k"], lk, g, dtype)
    b.data["v"] = fill_buffer(lay["v"], lk, g, dtype)
    if with_grad:
        g2 = torch.Generator().manual_seed(seed + 100)
        b.data["do"] = fill_buffer(lay["do"], lq, g2, dtype)
    return b


# ---------------------------------------------------------------- workloads

def tiny_padded_thd(causal: bool = False, lse_kind: str = "token", seed: int = 1001) -> Batch:
    """Three sequences [3, 2, 4] with one identifier row after each:
    rows [a a a 1 b b 2 2 c c c c 3], cu_seqlens [0,3,5,9],
    cu_seqlens_padded [0,4,8,13]."""
    lens = [3, 2, 4]
    start = [0, 4, 8, 13]
    return build("tiny_padded_thd", seed, 2, 2, 64, lens, lens, start, start,
                 default_policy=CAUSAL_TOP_LEFT if causal else PADDING, lse_kind=lse_kind)


def packed_causal(seed: int = 1002, with_grad: bool = False) -> Batch:
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=16, endpoint=True)
    start = _prefix(lens)
    return build("packed_causal_h32_d128", seed, 32, 32, 128, lens, lens, start, start,
                 default_policy=CAUSAL_TOP_LEFT, lse_kind="head", with_grad=with_grad)


def packed_causal_window(seed: int = 1002, with_grad: bool = False, left: int = 1024) -> Batch:
    """The packed causal workload with a bounded causal window: each row sees
    itself and the ``left`` keys before it (the lengths and data of the packed causal workload)."""
    b = packed_causal(seed, with_grad)
    b.name = f"packed_causal_window{left}_h32_d128"
    b.window = np.array([[-1, -1], [left, 0], [-1, -1]], np.int32)
    return b


def packed_causal_f16(seed: int = 1002, with_grad: bool = False) -> Batch:
    """The packed causal workload (same lengths and layout) in IEEE fp16."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=16, endpoint=True)
    start = _prefix(lens)
    return build("packed_causal_f16_h32_d128", seed, 32, 32, 128, lens, lens, start, start,
                 default_policy=CAUSAL_TOP_LEFT, lse_kind="head", with_grad=with_grad,
                 dtype="f16")


def padded_gqa(seed: int = 1003, with_grad: bool = True) -> Batch:
    rng = np.random.default_rng(seed)
    lens = rng.integers(64, 2048, size=32, endpoint=True)
    gq = rng.integers(0, 63, size=32, endpoint=True)
    gk = rng.integers(0, 63, size=32, endpoint=True)
    return build("padded_gqa_causal_h32_8_d128", seed, 32, 8, 128, lens, lens,
                 _with_gaps(lens, gq), _with_gaps(lens, gk),
                 default_policy=CAUSAL_TOP_LEFT, lse_kind="token", with_grad=with_grad)


def mixed_policy(seed: int = 1004, with_grad: bool = False) -> Batch:
    rng = np.random.default_rng(seed)
    lq = rng.integers(32, 1024, size=64, endpoint=True)
    lk = lq + rng.integers(0, 1024, size=64, endpoint=True)
    policy = rng.integers(0, 2, size=64, endpoint=True).astype(np.int8)
    return build("mixed_policy_h16_d128", seed, 16, 16, 128, lq, lk, _prefix(lq), _prefix(lk),
                 default_policy=PADDING, policy=policy, lse_kind="token", with_grad=with_grad)


def long_context_cp(seed: int = 1005, with_grad: bool = True, doc_len: int = 65536,
            chunk: int = 4096, offsets=(4096, 61440)) -> Batch:
    """Two documents of ``doc_len`` keys; each queried by two ``chunk``-row
    segments whose first query sits at absolute key ``offsets[i]``.  Both
    segments of one document bind the same K/V rows (K/V ragged
    [0, 0, L, L, 2L])."""
    lq = [chunk] * 4
    lk = [doc_len] * 4
    q_start = [0, chunk, 2 * chunk, 3 * chunk, 4 * chunk]
    kv_start = [0, 0, doc_len, doc_len, 2 * doc_len]
    qco = [offsets[0], offsets[1], offsets[0], offsets[1]]
    return build("long_context_cp_chunks_h16_d128", seed, 16, 16, 128, lq, lk, q_start, kv_start,
                 default_policy=CAUSAL_TOP_LEFT, q_causal_offset=qco, lse_kind="head",
                 with_grad=with_grad)


# The five measured workloads by name.
BY_NAME = {"tiny_padded_thd": tiny_padded_thd, "packed_causal": packed_causal,
           "padded_gqa": padded_gqa, "mixed_policy": mixed_policy, "long_context_cp": long_context_cp}


def random_batch(seed: int, *, batch: int = 4, max_len: int = 200, h_q: int = 4, h_kv: int = 2,
                 dim: int = 64, cross: bool = True, max_gap: int = 40, token_gaps: bool = True,
                 policies=(PADDING, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT), per_seq_policy=True,
                 q_causal_offset: bool = False, lse_kind: str | None = None,
                 zero_lengths: bool = True, with_grad: bool = True,
                 window=None, dtype: str = "bf16") -> Batch:
    """A small random ragged batch for parity tests: random lengths (some 0;
    a nonzero key length is at least a quarter of the query length), random
    row gaps between sequences (separately for the query-side and
    key-side buffers), random per-tensor token-stride gaps n*H*D (n = 0..3),
    random per-sequence policies and LSE layout.  ``window``: None, an int32
    [3, 2] array of per-policy (left, right) windows, or "random" (each side
    unbounded with probability 1/3, else uniform in [0, max_len // 2])."""
    rng = np.random.default_rng(seed)
    lo = 0 if zero_lengths else 1
    lq = rng.integers(lo, max_len, size=batch, endpoint=True)
    lk = rng.integers(lo, max_len, size=batch, endpoint=True) if cross else lq.copy()
    # at most four query rows per key row, so that no key gathers the
    # gradients of many queries (gradients stay O(1))
    lk = np.where(lk > 0, np.maximum(lk, (lq + 3) // 4), lk)
    lead_q, lead_k = rng.integers(0, max_gap + 1, size=2)
    gq = rng.integers(0, max_gap, size=batch, endpoint=True)
    gk = rng.integers(0, max_gap, size=batch, endpoint=True)
    q_start = _with_gaps(lq, gq) + lead_q
    kv_start = _with_gaps(lk, gk) + lead_k
    gaps = {}
    if token_gaps:
        for n in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
            gaps[n] = int(rng.integers(0, 4))
    pol = rng.choice(np.asarray(policies, np.int8), size=batch)
    if lse_kind is None:
        lse_kind = "token" if rng.integers(0, 2) == 0 else "head"
    qco = None
    if q_causal_offset:
        qco = rng.integers(-max_len // 4, max_len + 1, size=batch).astype(np.int32)
    if isinstance(window, str):
        assert window == "random"
        window = random_window(rng, max_len // 2)
    return build(f"random_{seed}", seed, h_q, h_kv, dim, lq, lk, q_start, kv_start,
                 default_policy=int(pol[0]), policy=pol if per_seq_policy else None,
                 q_causal_offset=qco, lse_kind=lse_kind, token_gaps=gaps,
                 q_rows=int(q_start[-1]) + int(rng.integers(0, 8)),
                 kv_rows=int(kv_start[-1]) + int(rng.integers(0, 8)), with_grad=with_grad,
                 window=window, dtype=dtype)


def random_window(rng: np.random.Generator, max_size: int) -> np.ndarray:
    """Per-policy (left, right) windows: each side -1 (unbounded) with
    probability 1/3, else uniform in [0, max_size]."""
    w = rng.integers(0, max_size, size=(3, 2), endpoint=True)
    w[rng.integers(0, 3, size=(3, 2)) == 0] = -1
    return w.astype(np.int32)


def aliased_batch(seed: int, *, docs: int = 3, max_doc: int = 300, chunks: int = 2,
                  h_q: int = 4, h_kv: int = 2, dim: int = 64, shuffle: bool = True,
                  with_grad: bool = True, dtype: str = "bf16", window=None) -> Batch:
    """Context-parallel style batch: `docs` documents of random length, each
    queried by `chunks` query segments that bind the document's key rows
    (identical K/V/dK/dV offsets) with random per-segment q causal offsets;
    the segments of all documents are shuffled, so aliasing segments need
    not be adjacent.  Top-left causal with offsets; token-major LSE."""
    rng = np.random.default_rng(seed)
    dl = rng.integers(16, max_doc, size=docs, endpoint=True)
    kv_start_doc = _with_gaps(dl, rng.integers(0, 8, size=docs, endpoint=True))
    segs = []
    for d in range(docs):
        for _ in range(chunks):
            lq = int(rng.integers(1, max(2, int(dl[d]) // chunks), endpoint=True))
            off = int(rng.integers(-lq // 2, int(dl[d]) - lq + 1, endpoint=True))
            segs.append((d, lq, off))
    order = rng.permutation(len(segs)) if shuffle else np.arange(len(segs))
    segs = [segs[i] for i in order]
    lq = np.array([s[1] for s in segs], np.int64)
    lk = np.array([int(dl[s[0]]) for s in segs], np.int64)
    q_start = _with_gaps(lq, rng.integers(0, 4, size=len(segs), endpoint=True))
    kv_start = np.array([int(kv_start_doc[s[0]]) for s in segs] + [int(kv_start_doc[-1])],
                        np.int64)
    qco = np.array([s[2] for s in segs], np.int32)
    return build(f"aliased_{seed}", seed, h_q, h_kv, dim, lq, lk, q_start, kv_start,
                 default_policy=CAUSAL_TOP_LEFT, q_causal_offset=qco, lse_kind="token",
                 kv_rows=int(kv_start_doc[-1]), with_grad=with_grad, dtype=dtype,
                 window=window)
