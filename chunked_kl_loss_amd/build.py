"""Build libckl.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m chunked_kl_loss_amd.build [--debug]

The library is written next to this file; the Python binding loads it from
there.  hipcc cross-compiles for gfx950, so no GPU is needed to build.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("ckl_kernels.hip", "ckl_api.hip")]
LIB = os.path.join(HERE, "libckl.so")
ARCH = os.environ.get("CKL_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(debug: bool = False, verbose: bool = False) -> str:
    flags = [
        f"--offload-arch={ARCH}",
        "-std=c++17",
        "-O1" if debug else "-O3",
        "-fPIC",
        "-shared",
        # packed fp32 ops stay off: the compiler must not form v_pk_*_f32
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
        "-I", os.path.join(ROOT, "include"),
    ]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv, verbose=True))
