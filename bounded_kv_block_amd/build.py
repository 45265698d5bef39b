"""Build libbkv.so (HIP kernels + C-ABI host code) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbkv.so")
SOURCES = [os.path.join(CSRC, "bkv.cpp"), os.path.join(CSRC, "kernels.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libbkv.so")


def command(out: str = LIB) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            # no packed-fp32 VALU forms in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            # an inline-asm diagnostic (e.g. a reserved register in a clobber
            # list) is an error, not a warning to scroll past
            "-Werror=inline-asm",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile every source; always rebuilds.  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (r.stderr or "").splitlines()
            if ln.strip() and "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
