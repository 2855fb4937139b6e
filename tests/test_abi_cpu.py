"""C-ABI checks that need no GPU: exported symbols, host validation codes,
workspace sizing.  Nothing here launches a kernel: every call either fails
host validation or is a host-only sizing query (or batch == 0)."""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

import oracle
import variable_length_attention_ragged_amd as va
from variable_length_attention_ragged_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "varlen_attn.h")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

FAKE = 0x10000  # 256-byte aligned fake device address; never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(varlen_attn_\w+)\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 9
    lib = va.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(va.exported_symbols()) == names


def _t(span, st, sh, data=FAKE, ragged=FAKE, scaled=None, mult=0):
    return B.varlen_attn_tensor(data, span, st, sh, ragged, scaled, mult)


def _p(batch=2, h_q=4, h_kv=2, d=128, scale=0.1, policy=0, mask=None):
    return B.varlen_attn_problem(batch, h_q, h_kv, d, scale, FAKE, FAKE, mask, policy, None)


def _fwd(p, q=None, k=None, v=None, o=None, lse=None, ws=FAKE, ws_bytes=1 << 30):
    d = p.head_dim
    q = q or _t(100 * p.h_q * d, p.h_q * d, d)
    k = k or _t(100 * p.h_kv * d, p.h_kv * d, d)
    v = v or _t(100 * p.h_kv * d, p.h_kv * d, d)
    o = o or _t(100 * p.h_q * d, p.h_q * d, d)
    lse = lse or _t(100 * p.h_q, p.h_q, 1)
    return va.lib().varlen_attn_fwd(ctypes.byref(p), ctypes.byref(q), ctypes.byref(k),
                                    ctypes.byref(v), ctypes.byref(o), ctypes.byref(lse), ws,
                                    ws_bytes, None, None)


@pytest.mark.parametrize("case,code", [
    ("batch", B.ERR_BATCH), ("head_dim", B.ERR_HEAD_DIM), ("heads", B.ERR_HEADS),
    ("heads0", B.ERR_HEADS), ("scale", B.ERR_SCALE), ("policy", B.ERR_POLICY),
    ("null_q", B.ERR_NULL), ("align", B.ERR_ALIGN), ("stride8", B.ERR_STRIDE),
    ("stride_small", B.ERR_STRIDE), ("span", B.ERR_SPAN), ("workspace", B.ERR_WORKSPACE),
    ("ws_align", B.ERR_ALIGN), ("ws_null", B.ERR_WORKSPACE),
    ("no_offsets", B.ERR_NULL), ("both_offsets", B.ERR_OFFSETS),
    ("multiplier0", B.ERR_OFFSETS), ("multiplier_big", B.ERR_OFFSETS),
    ("window", B.ERR_WINDOW), ("dtype", B.ERR_DTYPE),
    ("stride_32bit_tile", B.ERR_STRIDE), ("lse_stride_32bit_tile", B.ERR_STRIDE),
])
def test_host_validation_codes(case, code):
    p = _p()
    kw = {}
    if case == "batch":
        p.batch = -1
    elif case == "head_dim":
        p.head_dim = 96
    elif case == "heads":
        p.h_q, p.h_kv = 6, 4
    elif case == "heads0":
        p.h_kv = 0
    elif case == "scale":
        p.scale = float("nan")
    elif case == "policy":
        p.default_policy = 3
    elif case == "null_q":
        kw["q"] = _t(100 * 512, 512, 128, data=0)
    elif case == "align":
        kw["q"] = _t(100 * 512, 512, 128, data=FAKE + 8)
    elif case == "stride8":
        kw["k"] = _t(100 * 260, 260, 130)
    elif case == "stride_small":
        kw["o"] = _t(100 * 512, 64, 128)
    elif case == "span":
        kw["v"] = _t(200, 128, 128)
    elif case == "workspace":
        kw["ws_bytes"] = 64
    elif case == "ws_align":
        kw["ws"] = FAKE + 64
    elif case == "ws_null":
        kw["ws"] = None
    elif case == "no_offsets":
        kw["k"] = _t(100 * 256, 256, 128, ragged=None)
    elif case == "both_offsets":
        kw["k"] = _t(100 * 256, 256, 128, scaled=FAKE, mult=256)
    elif case == "multiplier0":
        kw["v"] = _t(100 * 256, 256, 128, ragged=None, scaled=FAKE, mult=0)
    elif case == "multiplier_big":
        kw["o"] = _t(100 * 512, 512, 128, ragged=None, scaled=FAKE, mult=1 << 31)
    elif case == "dtype":
        p.dtype = 2
    elif case == "stride_32bit_tile":
        # a legal-looking row stride whose 128-row tile spans 2^31 bytes: the
        # kernels' 32-bit buffer offsets would wrap
        st = ((1 << 30) - 128 + 126) // 127 // 8 * 8 + 8
        assert (127 * st + 128) * 2 >= 1 << 31
        kw["k"] = _t(4 * st, st, 128)
    elif case == "lse_stride_32bit_tile":
        st = ((1 << 29) - 1 + 126) // 127 + 1
        assert (127 * st + 1) * 4 >= 1 << 31
        kw["lse"] = _t(4 * st, st, 1)
    elif case == "window":
        win = (ctypes.c_int32 * 6)(-1, -1, 128, 0, -1, -2)
        p.window_size = ctypes.addressof(win)
    assert _fwd(p, **kw) == code
    assert va.status_string(code) != "unknown status code"


def test_scaled_offsets_pass_host_validation():
    """Row-unit offsets with a multiplier are a complete alternative to
    element offsets: such tensors pass every tensor check, so the call gets
    as far as the workspace check (and, with batch 0, succeeds with no
    launch)."""
    k = _t(100 * 256, 256, 128, ragged=None, scaled=FAKE, mult=256)
    lse = _t(100 * 4, 4, 1, ragged=None, scaled=FAKE, mult=4)
    assert _fwd(_p(), k=k, lse=lse, ws=None) == B.ERR_WORKSPACE
    assert _fwd(_p(batch=0), k=k, lse=lse, ws=None, ws_bytes=0) == B.OK


def test_largest_stride_below_the_32bit_tile_limit_passes():
    """127 * stride_t + D elements of 2 bytes just below 2^31: accepted (the
    call reaches the workspace check); one multiple of 8 more is refused."""
    st = ((1 << 30) - 128) // 127 // 8 * 8
    assert (127 * st + 128) * 2 < 1 << 31
    assert _fwd(_p(), k=_t(4 * st, st, 128), ws=None) == B.ERR_WORKSPACE
    big = st + 8
    while (127 * big + 128) * 2 < 1 << 31:
        big += 8
    assert _fwd(_p(), k=_t(4 * big, big, 128), ws=None) == B.ERR_STRIDE


def test_window_sizes_pass_host_validation():
    """Windows of -1 (unbounded) and any size >= 0 are accepted: the call gets
    as far as the workspace check."""
    for vals in ((-1,) * 6, (0,) * 6, (5, 0, 1 << 30, 0, 0, 7)):
        win = (ctypes.c_int32 * 6)(*vals)
        p = _p()
        p.window_size = ctypes.addressof(win)
        assert _fwd(p, ws=None) == B.ERR_WORKSPACE


def test_empty_batch_is_a_no_op():
    assert _fwd(_p(batch=0), ws=None, ws_bytes=0) == B.OK


def _bwd_layout(lse, dq, dk, p=None):
    p = p or _p(batch=3, h_q=8, h_kv=8, d=128)
    L = B.varlen_attn_layout()
    rc = va.lib().varlen_attn_bwd_workspace_layout(ctypes.byref(p), ctypes.byref(lse),
                                                   ctypes.byref(dq), ctypes.byref(dk),
                                                   ctypes.byref(L))
    assert rc == B.OK
    return L


def test_head_major_stats_workspace_pin():
    """delta mirrors LSE: a head-major [h=8, t=7360] LSE needs 58880 fp32
    elements, not the 7360 a token-stride-only formula gives."""
    with open(os.path.join(GOLDEN, "stats_span.json")) as f:
        g = json.load(f)
    h, t = g["h_q"], g["t"]
    span = oracle.sizing.span_by_enumeration((t, h), (1, t))
    assert span == g["every_axis_elems"]
    lse = _t(span, 1, t)
    dq = _t(t * h * 128, h * 128, 128)
    dk = _t(t * h * 128, h * 128, 128)
    L = _bwd_layout(lse, dq, dk)
    assert L.delta_elems == 58880
    assert L.delta_elems != g["token_stride_only_elems"]
    assert L.total_bytes - L.delta_offset >= 58880 * 4
    # the view-based span the binding computes agrees
    import torch
    view = torch.empty(h, t).t()          # [t, h] view of head-major storage
    assert va.view_span(view) == 58880


@pytest.mark.parametrize("T,h,d", [(7360, 8, 128), (100, 3, 64)])
def test_token_major_workspace_identities(T, h, d):
    lse = _t(T * h, h, 1)
    dq = _t(T * h * d, h * d, d)
    dk = _t(T * h * d, h * d, d)
    L = _bwd_layout(lse, dq, dk, _p(batch=3, h_q=h, h_kv=h, d=d))
    assert L.delta_elems == T * h                 # softmax_sum = maxT * h_q
    assert L.total_bytes >= L.delta_offset + 4 * T * h
    assert L.total_bytes >= L.lse_term_offset + 4 * T * h
    assert L.delta_offset % 256 == 0 and L.lse_term_offset % 256 == 0


def test_regions_are_disjoint_and_ordered():
    lse = _t(1000 * 4, 4, 1)
    dq = _t(1000 * 512, 512, 128)
    dk = _t(2000 * 256, 256, 128)
    L = _bwd_layout(lse, dq, dk, _p(batch=37, h_q=4, h_kv=2))
    regions = [(L.counters_offset, 256), (L.header_offset, 64),
               (L.seq_offset, L.seq_i64_offset + 72 * 37),
               (L.fwd_tiles_offset, 8 * L.fwd_tiles_capacity),
               (L.bwd_tiles_offset, 16 * L.bwd_tiles_capacity),
               (L.members_offset, 4 * 37),
               (L.scratch_offset, 96 * 37), (L.delta_offset, 4 * L.delta_elems),
               (L.lse_term_offset, 4 * L.delta_elems)]
    assert L.seq_i64_offset >= 6 * 4 * 37      # lq, lk, policy, hi, lo, flags
    for (a, n), (b, _) in zip(regions, regions[1:]):
        assert a + n <= b and b % 256 == 0
    assert regions[-1][0] + regions[-1][1] <= L.total_bytes
    # capacities come from the physical rows, plus one partial tile per sequence
    assert L.fwd_tiles_capacity == -(-1000 // L.fwd_block_m) + 37
    assert L.bwd_tiles_capacity == -(-2000 // L.bwd_block_n) + 37


def test_product_path_has_no_oracle_dependency():
    pkg = os.path.join(ROOT, "variable_length_attention_ragged_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracles", ""), f


def _fwd_noalloc(p, **kw):
    d = p.head_dim
    q = kw.get("q") or _t(100 * p.h_q * d, p.h_q * d, d)
    k = kw.get("k") or _t(100 * p.h_kv * d, p.h_kv * d, d)
    v = kw.get("v") or _t(100 * p.h_kv * d, p.h_kv * d, d)
    o = kw.get("o") or _t(100 * p.h_q * d, p.h_q * d, d)
    lse = kw.get("lse") or _t(100 * p.h_q, p.h_q, 1)
    return va.lib().varlen_attn_fwd_noalloc(ctypes.byref(p), ctypes.byref(q), ctypes.byref(k),
                                            ctypes.byref(v), ctypes.byref(o), ctypes.byref(lse),
                                            None, None)


def test_noalloc_forward_host_checks():
    """The workspace-free forward applies the forward's host checks, refuses a
    problem whose workspace exceeds its static 4 MiB with ERR_SCRATCH before
    touching the device, and returns OK for an empty batch."""
    assert _fwd_noalloc(_p(d=96)) == B.ERR_HEAD_DIM
    assert _fwd_noalloc(_p(), q=_t(100 * 512, 512, 128, data=FAKE + 8)) == B.ERR_ALIGN
    assert _fwd_noalloc(_p(batch=0)) == B.OK
    # about 204 bytes per sequence: 30000 sequences need more than 4 MiB
    big = _p(batch=30000)
    size = ctypes.c_size_t(0)
    o = _t(100 * 512, 512, 128)
    assert va.lib().varlen_attn_fwd_workspace_size(ctypes.byref(big), ctypes.byref(o),
                                                   ctypes.byref(size)) == B.OK
    assert size.value > B.NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(big) == B.ERR_SCRATCH
    assert "static scratch" in va.status_string(B.ERR_SCRATCH)
