"""Builds libmoe.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_mixture_experts_06_amd.build

Every .hip file under csrc/ is compiled by hipcc in parallel into
<repo>/_build/, then linked into sparse_mixture_experts_06_amd/libmoe.so.
It always recompiles, so a stale library is never mistaken for a fresh one.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming packed fp32 (v_pk_*_f32) ops; the
# host pass warns that it does not know the feature, which is harmless.
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


# Per-file extra flags. ffn_dma.hip places its MFMAs, fragment reads and
# direct-to-LDS loads by hand (groups closed by scheduling barriers); with the
# machine scheduler on, its reordering makes the register allocator rotate the
# 256 accumulators of a wave through copies every K step.
FILE_FLAGS = {"ffn_dma.hip": ["-mllvm", "-enable-misched=0"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return out


def compile_command(src: str, out: str, extra=()) -> list:
    """The hipcc command build() uses for one source file (plus `extra`)."""
    return [_hipcc(), *HIPFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, src,
            "-o", out]


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = []
    jobs = []
    for src in sources:
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        jobs.append(compile_command(src, obj, ["-c"]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
