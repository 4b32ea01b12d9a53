"""Build librrs.so (the C-ABI library of the RRS A4W4 linear) for gfx950.

    python -m rotated_runtime_activation_amd.build

compiles every HIP source under csrc/ with hipcc (one object per source, in
parallel) and links them into lib/librrs.so, in-tree.
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
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "librrs.so")
SOURCES = ["rrs_frontend.hip", "rrs_frontend_kron.hip", "rrs_gemm.hip", "rrs_gemm_small.hip", "rrs_noalloc.hip",
           "rrs_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if os.path.exists(cand):
        return cand
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build librrs")
    return found


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-fvisibility=hidden",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators in VGPRs: the group rescale multiplies them
        # with ordinary VALU instructions
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def compile_cmd(src: str, obj: str) -> list:
    return [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]


def link_cmd(objs: list, out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd: list) -> str:
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    log = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{log}")
    return log


def build(verbose: bool = False) -> str:
    """Compile every source (always, also when a library exists) and link."""
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    cmds = [compile_cmd(src, obj) for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    logs.append(_run(link_cmd(objs, tmp)))
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
