"""Build the HIP library libmoe_mx.so in-tree for gfx950 (hipcc, no JIT cache)."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmoe_mx.so"
SOURCES = ["csrc/api.cpp", "csrc/routing.hip", "csrc/permute_quant.hip", "csrc/tiles.hip", "csrc/gmm.hip",
           "csrc/gmm_stream.hip", "csrc/combine.hip", "csrc/peaks.hip", "csrc/noalloc.hip"]
ARCH = os.environ.get("MOE_MX_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def lib_path() -> str:
    return os.path.join(HERE, LIB_NAME)


FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    # keep fp32 denormals: MX quantization of subnormal bf16 inputs depends on them
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source (in parallel, one object each) and link them into one shared
    library; always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    out = lib_path()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in SOURCES]
    cmds = [[hipcc(), *FLAGS, *inc, "-c", os.path.join(HERE, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
