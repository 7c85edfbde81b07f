"""Builds the HIP selector library in-tree for gfx950.

    python -m exact_top_selection_stride_amd.build

Produces exact_top_selection_stride_amd/libtopk_exact.so from csrc/topk_exact.hip
(the selector) and csrc/indexer_scores.hip (the FP8 indexer score producer) with
hipcc. Packed FP32 instructions are disabled: the selector does no float math,
and the flag keeps the compiler from emitting them in the score kernel's
ReLU / weighting code.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("topk_exact.hip", "indexer_scores.hip")]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtopk_exact.so")
ARCH = os.environ.get("TOPK_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(out: str, extra=()):
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the score kernel reads every accumulator with VALU
            # ops, which cannot take accumulator registers (each would need a copy).
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INC, *SRCS, "-o", out, *extra]


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
