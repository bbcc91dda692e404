"""Build libstq.so (the HIP library behind include/stq.h) in-tree for gfx950.

    python -m linear_attention_recurrent_rule_amd.build

Every kernel is compiled with packed-fp32 instructions disabled and with
floating-point contraction off: each fused multiply-add in the kernels is an
explicit __builtin_fmaf, so the rounding points are the ones written.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libstq.so"
SOURCES = ["decode.hip", "decode128.hip", "aux_kernels.hip", "alloc_kernels.hip", "alloc128.hip",
           "calib_static.hip", "alloc_host.cpp",
           "stq_api.cpp"]

ARCH = os.environ.get("STQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libstq.so")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core results straight into the vector register file (no
        # accumulation-register copies: fewer instructions and registers)
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    """Compile every source and link libstq.so next to this file."""
    cc = hipcc()
    objdir = PKG / "_build"
    objdir.mkdir(exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = objdir / (src + ".o")
        cmds.append([cc, *compile_flags(), *(extra or []), "-c", str(CSRC / src), "-o", str(obj)])
        objs.append(str(obj))
    # the sources are independent translation units: compile them concurrently
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
        for f in [ex.submit(subprocess.run, cmd, check=True) for cmd in cmds]:
            f.result()
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
