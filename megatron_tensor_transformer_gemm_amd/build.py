"""Build libtpshard.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m megatron_tensor_transformer_gemm_amd.build  (or build() from Python).
Every call compiles all sources again; the objects go to ``_build/`` next to
this file and the library to ``libtpshard.so`` in this package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtpshard.so")
SOURCES = ["capi.hip", "gemm_bf16.hip", "gemm_f32.hip", "partial_sum.hip", "attention.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libtpshard")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _check_stubs(objs) -> None:
    """Every kernel a host launcher references must have its launch stub defined."""
    nm = shutil.which("nm")
    if not nm:
        return
    for o in objs:
        out = subprocess.run([nm, "-C", "-u", o], capture_output=True, text=True).stdout
        missing = [ln.strip() for ln in out.splitlines() if "__device_stub__" in ln]
        if missing:
            raise RuntimeError(f"{o}: kernel launch stubs not emitted by the host pass:\n"
                               + "\n".join(missing[:8]))


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    cmds = [[hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out, file=sys.stderr)
    _check_stubs(objs)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
