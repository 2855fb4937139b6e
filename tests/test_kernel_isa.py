"""Checks on the gfx950 assembly of the persistent kernels (no GPU needed).

Every workgroup of the forward, dQ and dK/dV kernels claims work items in a
loop whose body holds workgroup barriers.  All lanes of a wave must run the
same iterations of that loop: if the compiler turns it into a divergent loop
(lanes leaving at different iterations, kept apart by exec masks), a wave
reaches its barriers a different number of times than the other waves of its
workgroup and the workgroup never finishes.  Such a loop leaves a tell-tale
`s_andn2_b64 exec, exec, ...` at its latch; the kernels here have no other
divergent loops, so none may appear in their code.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from variable_length_attention_ragged_amd import build as B

KERNEL_SOURCES = ("fwd.hip", "bwd.hip")
KERNEL_NAMES = ("fwd_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel")


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = [B.hipcc()] + B.compile_flags() + B.EXTRA_FLAGS.get(src, []) + \
        ["--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{res.stderr}")
    return open(out).read()


def _kernel_bodies(asm: str) -> dict:
    """Mangled kernel symbol -> its instructions (label to s_endpgm)."""
    bodies = {}
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        name = m.group(1)
        if not any(k in name for k in KERNEL_NAMES):
            continue
        end = asm.find("s_endpgm", m.end())
        bodies[name] = asm[m.end():end]
    return bodies


@pytest.fixture(scope="module")
def bodies(tmp_path_factory):
    if not os.path.exists(B.hipcc()):
        pytest.skip("hipcc not installed")
    d = str(tmp_path_factory.mktemp("isa"))
    out = {}
    for src in KERNEL_SOURCES:
        out.update(_kernel_bodies(_device_asm(src, d)))
    return out


def test_every_instantiation_is_found(bodies):
    # 3 kernels x 2 head dims x 2 element types
    assert len(bodies) == 12, sorted(bodies)


def test_item_loops_stay_uniform(bodies):
    for name, body in bodies.items():
        assert "s_barrier" in body, name
        assert not re.search(r"s_andn2_b64\s+exec,\s*exec", body), \
            f"{name}: a loop was compiled as divergent (exec-masked latch)"
