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
# (source, extra flags): attn_fwd.hip is compiled once per (head dim, logit
# kind) pair, each unit holding that pair's kernels, so the units build in
# parallel.  The D = 256 kernels keep their MFMA results in vector registers:
# with the compiler's default (accumulation registers) their 128 accumulators
# were copied between register files around every tile (~1800 copies per
# kernel; kernel 574 -> 470 us on the wide-group chunked prefill), while the
# same choice made the D <= 128 decode and the backward slower.
_VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
UNITS = [("attn_fwd.hip", [f"-DMIATTN_KD={d}", f"-DMIATTN_KCAP={c}"] + (_VGPR_MFMA if d == 256 else []))
         for d in (64, 128, 256) for c in (0, 1)] + [("lse_merge.hip", []), ("kv_write.hip", []),
                                                  ("attn_bwd.hip", []), ("miattn.hip", [])]
SOURCES = sorted({u[0] for u in UNITS})
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # a variable read before it is written is a bug here (work mappings, plans)
    "-Werror=uninitialized",
    "-Werror=sometimes-uninitialized",
    # keep the compiler from forming packed-FP32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]

# the host pass warns that it does not know the GPU-only feature
_NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if _NOISE not in ln]
    return r.returncode, msgs


def build(verbose: bool = False, extra_flags=None, jobs: int = 0) -> str:
    """Always recompiles (the units in parallel); returns the path of the library."""
    import concurrent.futures
    import tempfile

    jobs = jobs or min(len(UNITS), os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="miattn_build_") as tmpdir:
        cmds = []
        for n, (src, defs) in enumerate(UNITS):
            obj = os.path.join(tmpdir, f"{n}_{os.path.splitext(src)[0]}.o")
            cmds.append([HIPCC, *FLAGS, *(extra_flags or []), *defs, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(_run, cmds))
        for cmd, (rc, msgs) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
                if msgs:
                    print("\n".join(msgs))
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
        tmp = LIB + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", *[c[-1] for c in cmds], "-o", tmp]
        rc, msgs = _run(link)
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
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
