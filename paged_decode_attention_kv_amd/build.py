"""Build libpdakv.so (the HIP kernels + C ABI) for gfx950 with hipcc.

Usage: python paged_decode_attention_kv_amd/build.py [--isa]
(run by path: importing the package itself needs the built library)

--isa additionally keeps the AMD assembly of every kernel under _build/ for
register / occupancy review.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpdakv.so")
SOURCES = ["abi.cpp", "quant_write.hip", "decode.hip", "lifecycle.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # IEEE binary32 division and no denormal flushing: the quantizer's codes
    # and scales must be exact functions of the input.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # no packed-fp32 instructions (only an advisory host-pass warning results)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(isa: bool = False, verbose: bool = False, defines=(), out: str = LIB) -> str:
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += (["-x", "hip", p] if s.endswith(".cpp") else [p])
    cmd = [hipcc()] + FLAGS + [f"-D{d}" for d in defines] + srcs + ["-o", out + ".tmp"]
    cwd = None
    if isa:
        cwd = os.path.join(ROOT, "_build")
        os.makedirs(cwd, exist_ok=True)
        cmd.insert(1, "--save-temps")
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    errs = [ln for ln in r.stderr.splitlines()
            if "warning" in ln and "packed-fp32-ops" not in ln]
    if verbose and errs:
        print("\n".join(errs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(isa="--isa" in sys.argv, verbose=True))
