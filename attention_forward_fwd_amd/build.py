"""Build libfa.so (HIP, gfx950 only) in-tree: `python -m attention_forward_fwd_amd.build`."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(PKG, "csrc", "fa_fwd.hip"), os.path.join(PKG, "csrc", "fa_mask.hip")]
LIB = os.path.join(PKG, "libfa.so")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB (always recompiles).  Returns the library path."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
