"""Benchmark: ragged THD attention forward + backward on one MI355X.

One step = one pass of the whole hot path over the packed causal workload
(16 sequences with lengths U[128, 4096], seed 1002, H_q = H_kv = 32, D = 128,
top-left causal, head-major LSE): setup + forward (O, LSE), then setup +
dQ (which also forms the dO.O row terms) + dK/dV.  Inputs are
resident in HBM before the timed region; workspaces are preallocated.

Prints one JSON line.  ``value`` is causal-aware TFLOP/s of the whole step:
forward 4*D*pairs and backward 10*D*pairs per head, pairs = allowed
(query, key) pairs counted exactly from the drawn lengths.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0

# --workload: (workloads function, description, passes).  The first is the
# headline configuration; the others time the same kernels on the other
# synthetic configurations, each with the passes its configuration defines.
WORKLOADS = {
    "packed_causal": ("packed_causal", "packed causal THD: 16 sequences, lengths U[128,4096] "
                                 "(seed 1002), H_q=H_kv=32, D=128, top-left causal, "
                                 "head-major LSE; fwd+bwd", "fwd+bwd"),
    "sliding_window": ("packed_causal_window", "packed causal THD with a sliding window: the "
                                         "packed causal lengths (seed 1002), H_q=H_kv=32, "
                                         "D=128, top-left causal, window (1024, 0), "
                                         "head-major LSE; fwd+bwd", "fwd+bwd"),
    "packed_causal_f16": ("packed_causal_f16", "packed causal THD in fp16: the packed causal "
                                         "lengths (seed 1002), H_q=H_kv=32, D=128, top-left "
                                         "causal, head-major LSE; fwd+bwd", "fwd+bwd"),
    "padded_gqa": ("padded_gqa", "padded THD with GQA: 32 sequences, lengths U[64,2048], "
                              "U{0..63} NaN pad rows after each sequence, drawn separately "
                              "for Q/O and K/V (seed 1003), H_q=32, H_kv=8, D=128, "
                              "padding_causal, token-major LSE; fwd+bwd", "fwd+bwd"),
    "mixed_policy": ("mixed_policy", "mixed per-sequence mask policy: 64 sequences, Lq U[32,1024], "
                                "Lk = Lq + U[0,1024], policy U{padding, causal top-left, "
                                "causal bottom-right} as a device int8 tensor (seed 1004), "
                                "H=16, D=128, token-major LSE; fwd", "fwd"),
    "long_context_cp": ("long_context_cp", "long-context causal query chunks: 2 documents of 65536 "
                                   "keys, each queried by two 4096-row chunks at absolute "
                                   "key offsets 4096 and 61440 (per-segment q causal "
                                   "offsets; the two chunks of a document bind the same K/V "
                                   "rows), H=16, D=128, head-major LSE; fwd+bwd", "fwd+bwd"),
}


def pairs_per_head(batch) -> np.ndarray:
    """Allowed (query, key) pairs of each sequence, per head: row i sees the
    keys first(i) .. last(i) of [0, Lk), bounded by the causal diagonal and
    the policy's window."""
    out = np.zeros(batch.batch, np.int64)
    for b in range(batch.batch):
        lq, lk = int(batch.lq[b]), int(batch.lk[b])
        pol = int(batch.policy[b]) if batch.policy is not None else batch.default_policy
        if lq <= 0 or lk <= 0:
            continue
        if batch.q_causal_offset is not None:
            anchor = int(batch.q_causal_offset[b])
        else:
            anchor = 0 if pol == 1 else lk - lq
        i = np.arange(lq, dtype=np.int64)
        first = np.zeros(lq, np.int64)
        last = np.full(lq, lk - 1, np.int64)
        if pol != 0:
            last = np.minimum(last, i + anchor)
        if batch.window is not None:
            left, right = (int(x) for x in batch.window[pol])
            if right >= 0:
                last = np.minimum(last, i + anchor + right)
            if left >= 0:
                first = np.maximum(first, i + anchor - left)
        out[b] = int(np.clip(last - first + 1, 0, None).sum())
    return out


def fwd_bytes(batch) -> int:
    """Compulsory HBM bytes of the forward: Q read + O write (valid rows),
    K and V read once (distinct valid rows), LSE write."""
    q_rows = int(batch.lq.sum())
    kv_rows = int(batch.lk.sum())  # every workload here binds distinct K/V rows
    if batch.name.startswith("long_context"):
        kv_rows = int(batch.layouts["k"].rows)
    D = batch.dim
    return (2 * q_rows * batch.h_q * D * 2 + 2 * kv_rows * batch.h_kv * D * 2
            + q_rows * batch.h_q * 4)


_C_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def _code_tokens(text: str) -> str:
    """C/HIP source with comments removed and whitespace runs collapsed, so
    that a comment-only edit leaves the fingerprint (and the machine code)
    unchanged.  String literals in these sources hold no comment markers."""
    return " ".join(_C_COMMENT.sub(" ", text).split())


def kernel_fingerprint() -> str:
    """sha256 over the code of the HIP sources (comments and layout ignored)
    and the build script (which holds the compiler flags), as recorded next
    to the profiled traffic."""
    import glob
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "variable_length_attention_ragged_amd")
    for p in sorted(glob.glob(os.path.join(pkg, "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, encoding="utf-8") as f:
            h.update(_code_tokens(f.read()).encode())
    with open(os.path.join(pkg, "build.py"), "rb") as f:
        h.update(b"build.py")
        h.update(f.read())
    return h.hexdigest()


def profiled_traffic(kernel: str, workload: str):
    """Calibrated HBM bytes per launch of `kernel` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload, or None when
    the kernel sources have changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic__{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_fingerprint") != kernel_fingerprint():
        return None
    entry = rec.get("per_launch", {}).get(kernel)
    return None if entry is None else entry["total_bytes"]


def cpu_baseline(batch, target_s: float = 15.0):
    """Time the fp64 oracle's forward, as it stands, on a bounded sample of the
    same workload: every sequence for the first n query heads, one head per
    worker thread on every core this process may run on (BLAS held to one
    thread per worker, so the workers do not oversubscribe the cores), n
    chosen from a one-head probe so that the timed run takes about
    `target_s`."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    prob, t = oracle.from_batch(batch)
    pairs = int(pairs_per_head(batch).sum())

    def head(h):
        oracle.forward(prob, t["q"], t["k"], t["v"], t["o"], t["lse"], heads=[h])

    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        head(0)
        probe = time.perf_counter() - t0
        workers = min(cores, batch.h_q)
        n = int(max(1, min(batch.h_q, round(target_s * workers / max(probe, 1e-3)))))
        t0 = time.perf_counter()
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(head, range(n)))
        spent = time.perf_counter() - t0
    flops = 4.0 * batch.dim * pairs * n
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers),
            "kind": "oracle", "blas_threads": 1, "host_cores": int(cores),
            "sample": f"fp64 numpy oracle forward over all {batch.batch} sequences for {n} of "
                      f"{batch.h_q} query heads, one head per thread on {workers} threads "
                      f"({flops / 1e9:.1f} GFLOP causal-aware, {spent:.1f} s wall)"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--warmup-seconds", type=float, default=0.25,
                    help="keep warming up (untimed) until this much wall time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="packed_causal",
                    help="packed_causal (the headline configuration), sliding_window "
                         "(the same lengths with a causal window of 1024 keys back) or "
                         "packed_causal_f16 (the headline configuration in fp16)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times "
                         "(calibrates HBM byte counters against a known size) and exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got "
              f"--gpus {args.gpus}", file=sys.stderr)
        return 2

    import torch

    import workloads
    from workloads.device import DeviceBatch
    import variable_length_attention_ragged_amd as va

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    va.lib()
    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "repeats": 3}), flush=True)
        return 0
    fn, desc, passes = WORKLOADS[args.workload]
    with_bwd = passes == "fwd+bwd"
    batch = getattr(workloads, fn)(with_grad=with_bwd)
    dev = DeviceBatch(batch, with_grad=with_bwd)
    fwd_ws = torch.empty(dev.fwd_layout().total_bytes, dtype=torch.uint8, device="cuda")

    pairs = int(pairs_per_head(batch).sum())
    fwd_flops = 4.0 * batch.dim * batch.h_q * pairs
    bwd_flops = 10.0 * batch.dim * batch.h_q * pairs if with_bwd else 0.0

    # One step, one event between consecutive kernels (all on the current
    # stream, which the library launches on).
    stages = [("setup (fwd)", lambda: dev.fwd_setup(workspace=fwd_ws)),
              ("fwd_kernel", lambda: dev.fwd_stage("varlen_attn_fwd_attention", workspace=fwd_ws))]
    if with_bwd:
        bwd_ws = torch.empty(dev.bwd_layout().total_bytes, dtype=torch.uint8, device="cuda")
        stages += [("setup (bwd)", lambda: dev.bwd_setup(workspace=bwd_ws)),
                   ("bwd_dq_kernel", lambda: dev.bwd_stage("varlen_attn_bwd_dq", workspace=bwd_ws)),
                   ("bwd_dkdv_kernel", lambda: dev.bwd_stage("varlen_attn_bwd_dkdv", workspace=bwd_ws))]

    def step(ev=None):
        for n, (_, run) in enumerate(stages):
            if ev is not None:
                ev[n].record()
            run()
        if ev is not None:
            ev[-1].record()

    # Warm-up: the W steps asked for, and more until the GPU has run the step
    # for args.warmup_seconds, so that the timed steps see the clocks and
    # caches of a GPU under load (a few short steps do not get there: a
    # 0.4 ms step measured 15 % slower after 3 warm-up steps than after 20).
    warm = 0
    t_warm = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_warm < args.warmup_seconds:
        step()
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if int(dev.status.item()) != 0:
        print(f"device status {int(dev.status.item())}", file=sys.stderr)
        return 1

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    stage_ms = {name: float(np.mean([e[n].elapsed_time(e[n + 1]) for e in evs]))
                for n, (name, _) in enumerate(stages)}
    fwd_kernel_ms = stage_ms["fwd_kernel"]
    bwd_ms = sum(v for k, v in stage_ms.items() if k.startswith("bwd") or k == "setup (bwd)")
    fwd_ms = stage_ms["fwd_kernel"] + stage_ms["setup (fwd)"]
    dominant = max(stage_ms, key=stage_ms.get)
    # Algorithmic work per kernel.  The backward's 10*D flops per pair are
    # S, dP, dV, dK (dK/dV pass, 8*D) and dQ (dQ pass, 2*D); the dQ pass also
    # recomputes S and dP, which is not counted as algorithmic work.
    kernel_flops = {"fwd_kernel": fwd_flops, "bwd_dkdv_kernel": 0.8 * bwd_flops,
                    "bwd_dq_kernel": 0.2 * bwd_flops}

    fwd_tflops = fwd_flops / (fwd_kernel_ms * 1e-3) / 1e12
    dom_tflops = kernel_flops.get(dominant, 0.0) / (stage_ms[dominant] * 1e-3) / 1e12
    value = (fwd_flops + bwd_flops) / (ms * 1e-3) / 1e12
    fwd_gb = fwd_bytes(batch) / 1e9
    config = {
        "workload": desc,
        "passes": passes,
        "tokens": int(batch.lq.sum()),
        "pairs_per_head": pairs,
        "fwd_gflop": round(fwd_flops / 1e9, 2),
        "bwd_gflop": round(bwd_flops / 1e9, 2),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_pct_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        # compulsory bytes of the forward (Q, K, V read once, O and LSE
        # written) over the forward kernel's time: the HBM side of its roofline
        "fwd_compulsory_gb": round(fwd_gb, 4),
        "fwd_compulsory_gbs": round(fwd_gb / (fwd_kernel_ms * 1e-3), 1),
    }
    if with_bwd:
        config.update({
            "bwd_ms": round(bwd_ms, 4),
            "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
            "bwd_dkdv_tflops": round(0.8 * bwd_flops / (stage_ms["bwd_dkdv_kernel"] * 1e-3) / 1e12, 2),
            "bwd_dq_tflops": round(0.2 * bwd_flops / (stage_ms["bwd_dq_kernel"] * 1e-3) / 1e12, 2),
        })
    config["step_pct_peak"] = round(100 * value / PEAK_BF16_TFLOPS, 2)
    config["wall_s_timed"] = round(t_wall, 3)
    config["warmup_steps_run"] = warm
    line = {
        "metric": "varlen attention fwd/bwd TFLOP/s (causal-aware) and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": batch.dtype,
        "data": "synthetic",
        "config": config,
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(dom_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": profiled_traffic(dominant, batch.name),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
