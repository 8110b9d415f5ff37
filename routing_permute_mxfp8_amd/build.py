"""Build the HIP library libmoe_mx.so in-tree for gfx950 (hipcc, no JIT cache)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmoe_mx.so"
SOURCES = ["csrc/api.cpp", "csrc/routing.hip", "csrc/permute_quant.hip", "csrc/tiles.hip", "csrc/gmm.hip", "csrc/combine.hip", "csrc/peaks.hip"]
ARCH = os.environ.get("MOE_MX_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def lib_path() -> str:
    return os.path.join(HERE, LIB_NAME)


def build(verbose: bool = False) -> str:
    """Compile every source into one shared library; always recompiles."""
    out = lib_path()
    tmp = out + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
        # keep fp32 denormals: MX quantization of subnormal bf16 inputs depends on them
        "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
        *[os.path.join(HERE, s) for s in SOURCES],
        "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
