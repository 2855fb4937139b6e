"""Host-sanitizer build of the C-ABI library, for the CPU tier.

The host code of ``api.hip`` (argument checks, workspace layout, launch
setup) is compiled with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side only (``-Xarch_host`` before each sanitizer flag: the gfx950 device
code is built as usual), then linked with the regular objects of the kernel
sources into ``_build/asan/libvarlen_attn_asan.so``.  The tests load it in a
child process with the sanitizer runtime preloaded (Python itself is not
instrumented) and the library path in ``VARLEN_ATTN_LIBRARY``.

Test infrastructure: nothing on the product path uses this build, and no GPU
run needs it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "libvarlen_attn_asan.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def runtime() -> str:
    """Path of the clang AddressSanitizer runtime (it carries the UBSan
    handlers too) that must be preloaded into the child process."""
    from variable_length_attention_ragged_amd import build as b
    clang = os.path.join(os.path.dirname(b.hipcc()), "..", "llvm", "bin", "clang++")
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True,
                         check=True)
    path = os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise FileNotFoundError(path)
    return path


def build() -> str:
    """Compile api.hip with host sanitizers and link it with the regular
    objects of the other sources (built by the library's build()).  Returns
    the library path."""
    from variable_length_attention_ragged_amd import build as b
    objs = [os.path.join(b.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in b.SOURCES
            if s != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError(f"build the library first; missing {missing}")
    os.makedirs(OUT_DIR, exist_ok=True)
    api_obj = os.path.join(OUT_DIR, "api.o")
    flags = [f for f in b.compile_flags() if f != "-O3"] + ["-O1", "-g"]
    cmd = [b.hipcc()] + flags + HOST_SANITIZE + \
        ["-c", os.path.join(b.CSRC, "api.hip"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{res.stderr}")
    cmd = [b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", LIB, api_obj] + \
        objs + HOST_SANITIZE + ["-shared-libsan"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stderr}")
    return LIB
