"""Build the HIP library libshampoo_mi355x.so in-tree for gfx950.

    python -m blocked_shampoo_preconditioning_amd.build

Compiles the HIP kernels (csrc/kernels.hip, csrc/tensor_kernels.hip) and the
host runtime (csrc/runtime.cpp, roots.cpp, tensor_runtime.cpp) with hipcc into
one shared library next to this file. Packed fp32 instructions are disabled for the
device code (-packed-fp32-ops); hipcc's host pass warns that it does not know
that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libshampoo_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(CSRC, f) for f in ("kernels.hip", "tensor_kernels.hip", "runtime.cpp",
                                            "roots.cpp", "tensor_runtime.cpp")]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose=False):
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with exit code {r.returncode}")
    noise = [ln for ln in (r.stdout + r.stderr).splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "warning generated" not in ln]
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
