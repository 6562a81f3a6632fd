"""Compile libmiattn.so for gfx950 with hipcc (in-tree, next to this file).

Usage: ``python -m softmax_attention_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmiattn.so")
SOURCES = ["attn_fwd.hip", "lse_merge.hip", "miattn.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-FP32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Always recompiles; returns the path of the library."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), *[os.path.join(CSRC, s) for s in SOURCES],
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the GPU-only feature: drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    # every symbol must resolve (a kernel whose host-side launch stub was not
    # emitted only shows up here, as an undefined symbol)
    try:
        ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        raise RuntimeError(f"built library does not load: {e}") from None
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
