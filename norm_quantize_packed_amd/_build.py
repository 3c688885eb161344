"""Build ``libfrt.so`` (the HIP kernels and the C ABI) for gfx950 in-tree.

Usage: ``python -m norm_quantize_packed_amd._build`` (or ``build()`` from
the repository's entry module). hipcc cross-compiles without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfrt.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["frt_api.hip", "frt_norm.hip", "frt_pack.hip", "frt_gemm.hip", "frt_ffn.hip", "frt_rope.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 VALU instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the frt HIP library cannot be built")


def build(verbose: bool = True, jobs: int = 4) -> str:
    """Compile every source for gfx950 and link libfrt.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print("[frt build]", " ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    tmp = OUT + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print("[frt build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


def _drain(procs):
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        noise = [l for l in out.splitlines()
                 if "packed-fp32-ops" not in l and l.strip()]
        if noise:
            print("\n".join(noise), file=sys.stderr, flush=True)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}")


if __name__ == "__main__":
    print(build())
