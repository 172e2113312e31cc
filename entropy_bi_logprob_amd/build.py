"""Build libbi_logprob.so (HIP, gfx950) in-tree with hipcc, and beside it
libbi_ceilings.so (two plain streaming kernels the benchmark uses to measure
the HBM read and copy ceilings in the same run).

    python -m entropy_bi_logprob_amd.build

The library is a plain C ABI (include/bi_logprob.h) around hand-written HIP
kernels; it links only the HIP runtime.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f)
           for f in ("bi_logprob.hip", "bi_lmhead.hip", "bi_lmhead_bwd.hip")]
LIBS = []
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbi_logprob.so")
CEILINGS_SOURCES = [os.path.join(PKG, "csrc", "bi_ceilings.hip")]
CEILINGS_LIB = os.path.join(PKG, "libbi_ceilings.so")
ARCH = "gfx950"

# -ffp-contract=off: every multiply-add is written out explicitly in the
# kernels, so the arithmetic (and hence every row's bits) is exactly as written.
# The packed-fp32 feature is switched off for the device code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm installation is required to build")


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile the HIP library into ``out`` (and the ceilings library beside the
    default one); returns the library's path."""
    if out == LIB:
        _compile(verbose, (), CEILINGS_LIB, CEILINGS_SOURCES, [])
    return _compile(verbose, extra_flags, out, SOURCES, LIBS)


def _compile(verbose, extra_flags, out, sources, libs) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", INCLUDE, "-o", tmp, *sources, *libs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs:
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-q" not in sys.argv)
    print("built", path)
