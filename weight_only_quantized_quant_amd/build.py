"""Build libwq.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python weight_only_quantized_quant_amd/build.py

(run as a script: importing the package needs the library already built)

Always recompiles.  Each source is compiled to an object of its own in
`_build/` at the repository root, in parallel, then the objects are linked.
The library lands next to this file so that it travels with the source tree;
nothing is installed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libwq.so")

SOURCES = ["wq_quant.hip", "wq_gemm.hip", "wq_moe.hip", "wq_w8a8.hip", "wq_util.hip", "wq_status.cpp"]

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-source additions.  wq_gemm.hip: MFMA results in ordinary VGPRs (the
# compiler otherwise puts the decode GEMV's per-step partial sums in
# accumulation registers and copies each back before the VALU reads it:
# 8 copies per step at M = 1); measured 1-2 % faster for M = 1-4, and the
# prefill kernel, already VGPR-only, compiles to the same code.
SOURCE_FLAGS = {"wq_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
NOISE = "not a recognized feature for this target"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, flush=True)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc(), *HIP_FLAGS, *SOURCE_FLAGS.get(s, []), "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, s),
             "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
