"""Comparison helpers for the GPU tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads

# Tolerances (max-abs vs fp64) for the HIP path.  Gradients: 5e-2 absolute,
# plus 2^-8 of the magnitude, because a bf16 output cannot come closer to the
# exact value than half an ulp (2^-9 relative) and dS/P enter the bf16 MFMAs
# rounded the same way; e.g. |dK| = 12 (many queries over few keys) has ulp
# 0.0625.  For O(1) gradients the bar is the plain 5e-2.
O_TOL = 2e-2
GRAD_TOL = 5e-2
GRAD_REL = 2.0 ** -8
LSE_TOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pre_fill(batch: workloads.Batch, n: str) -> np.ndarray:
    lay = batch.layouts[n]
    return workloads.out_buffer(lay, "f32" if n == "lse" else batch.dtype)


def compare_bf16(batch, n, gpu_bits, ref_vals, written, tol, what="", rel=0.0):
    """Written elements within `tol + rel*|ref|` of the oracle; all others
    bit-identical to the pre-call contents."""
    pre = pre_fill(batch, n)
    assert gpu_bits.shape == pre.shape
    untouched = ~written
    bad = np.nonzero(gpu_bits[untouched] != pre[untouched])[0]
    assert bad.size == 0, f"{what}{n}: {bad.size} elements outside valid rows were written"
    if written.any():
        g = oracle.bits_to_f64(gpu_bits[written], batch.dtype)
        r = ref_vals[written]
        assert np.all(np.isfinite(g)), f"{what}{n}: non-finite output in a valid row"
        err = np.abs(g - r)
        excess = err - (tol + rel * np.abs(r))
        worst = int(np.argmax(excess))
        assert excess[worst] <= 0, (f"{what}{n}: abs err {err[worst]:.3e} > {tol} + {rel:.4f}"
                                    f"*|ref| (at {worst}, gpu {g[worst]}, ref {r[worst]})")
        return float(err.max())
    return 0.0


def compare_lse(batch, gpu, ref, written, what=""):
    pre = pre_fill(batch, "lse")
    untouched = ~written
    assert np.array_equal(gpu[untouched].view(np.uint32), pre[untouched].view(np.uint32)), \
        f"{what}lse: elements outside valid rows were written"
    if not written.any():
        return 0.0
    g, r = gpu[written].astype(np.float64), ref[written]
    dead = r == -np.inf
    assert np.all(g[dead] == -np.inf), f"{what}lse: dead rows must be -inf"
    assert np.all(np.isfinite(g[~dead])), f"{what}lse: non-finite LSE on a live row"
    err = np.abs(g[~dead] - r[~dead])
    m = float(err.max()) if err.size else 0.0
    assert m <= LSE_TOL, f"{what}lse: max abs err {m:.3e}"
    return m


def oracle_fwd(batch):
    prob, t = oracle.from_batch(batch)
    return oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"])


def oracle_bwd(batch, kv_heads=None):
    prob, t = oracle.from_batch(batch)
    return oracle.backward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"],
                           t["dk"], t["dv"], kv_heads=kv_heads)


def check_forward(batch, dev, ref=None, what=""):
    ref = oracle_fwd(batch) if ref is None else ref
    eo = compare_bf16(batch, "o", dev.host("o"), ref["o"], ref["o_written"], O_TOL, what)
    el = compare_lse(batch, dev.host("lse"), ref["lse"], ref["lse_written"], what)
    assert int(dev.status.item()) == ref["status"], (dev.status.item(), ref["status"])
    return eo, el


def check_backward(batch, dev, ref=None, what=""):
    ref = oracle_bwd(batch) if ref is None else ref
    errs = {}
    for n in ("dq", "dk", "dv"):
        errs[n] = compare_bf16(batch, n, dev.host(n), ref[n], ref[n + "_written"], GRAD_TOL, what,
                               rel=GRAD_REL)
    return errs
