"""Builds libpagedkv.so in-tree for gfx950.

HIP sources go through hipcc for gfx950 with packed-FP32 instruction
selection switched off (-Xclang -target-feature -Xclang -packed-fp32-ops);
the host allocator is plain C++17 and goes through g++.  Objects land in
``_build/`` next to this file, the shared library next to this file.  The decode kernels' device
assembly is checked for the discipline their explicitly waited loads rely on
(``verify_waits``); the build fails if it does not hold.

Usage: python -m paged_kv_cache_53_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedkv.so")

ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
HIP_SOURCES = ["api.hip", "scatter.hip", "decode.hip", "span.hip", "probe.hip"]
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # keep a wave's work-claim atomic as written: the optimiser's rewrite reads the result
             # at once, making the wave wait for all of its outstanding loads
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
CXX_SOURCES = ["allocator.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpagedkv)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    common = ["-O3", "-fPIC", "-std=c++17", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, f"--offload-arch={ARCH}", *common, *HIP_FLAGS,
                     "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *common, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # device assembly of the decode kernels, for the static check of their explicit waits
    asm = os.path.join(BUILD, "decode.s")
    cmds.append([hipcc, f"--offload-arch={ARCH}", *common, *HIP_FLAGS, "-S", "--cuda-device-only",
                 os.path.join(CSRC, "decode.hip"), "-o", asm])
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    from .verify_waits import check_file
    bad = {k: v for k, v in check_file(asm).items() if v}
    if bad:
        lines = [f"{k}:\n    " + "\n    ".join(v[:10]) for k, v in bad.items()]
        raise RuntimeError("decode kernels touch registers of in-flight explicitly waited loads:\n" +
                           "\n".join(lines))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
