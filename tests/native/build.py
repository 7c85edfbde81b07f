"""Builds the test-only matrix-core probe (tests/native/libmfma_probe.so) for gfx950.

    python tests/native/build.py

The probe is test infrastructure: only the tests load it. It is compiled with the same
flags as the selector library, so its instruction behaves as it does there.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_probe.hip")
LIB = os.path.join(HERE, "libmfma_probe.so")
ARCH = os.environ.get("TOPK_OFFLOAD_ARCH", "gfx950")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hipcc = os.path.join(rocm, "bin", "hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc if os.path.exists(hipcc) else "hipcc", "-O3", "-std=c++17", f"--offload-arch={ARCH}",
           "-fPIC", "-shared", "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True), file=sys.stdout)
