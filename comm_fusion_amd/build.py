"""Build libulysses_attn.so in-tree with hipcc for gfx950.

    python -m comm_fusion_amd.build

Compiles every source under ``csrc/`` into ``comm_fusion_amd/lib/``.  The
library is built for MI355X (gfx950) only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libulysses_attn.so")
SOURCES = ["ua_kernels.hip", "ua_api.cpp", "moe_kernels.hip", "moe_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # inputs are finite; lets fmax skip NaN canonicalisation of its operands
        "-fno-honor-nans",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-command-line-argument",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + ["-shared"] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def assembly(source: str = "ua_kernels.hip") -> str:
    """gfx950 assembly of one source (for inspecting waitcnt placement etc.)."""
    cmd = [hipcc()] + compile_flags() + ["--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", "-"]
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True,
                          check=True).stdout


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
