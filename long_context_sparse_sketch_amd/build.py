"""Build libsks.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m long_context_sparse_sketch_amd.build [--attn-valu]

Compiles every csrc/*.hip to an object in parallel with hipcc, then links the
shared library next to this file.  The build always recompiles.
``--attn-valu`` builds the comparison library libsks_attn_valu.so instead,
whose attention computes its Q.K and P.V products on the vector ALUs
(SKS_ATTN_VALU=1; bf16 rows), for timing against the matrix-core
attention (``bench.py --lib``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libsks.so")
ATTN_VALU_LIB_PATH = os.path.join(PKG, "libsks_attn_valu.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs (no argument
    # fetch before a kernel's first loads)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsks)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l
                    and "warning generated when compiling for host" not in l
                    and "warnings generated when compiling for host" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, attn_valu: bool = False) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(BUILD_DIR, "attn_valu") if attn_valu else BUILD_DIR
    lib = ATTN_VALU_LIB_PATH if attn_valu else LIB_PATH
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(bdir, s[:-4] + ".o") for s in srcs]
    flags = HIP_FLAGS + (["-DSKS_ATTN_VALU=1"] if attn_valu else [])

    def compile_one(pair):
        src, obj = pair
        return _run([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])

    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        outs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib + ".tmp"
    outs.append(_run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]))
    os.replace(tmp, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, attn_valu="--attn-valu" in sys.argv))
