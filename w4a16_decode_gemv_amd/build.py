"""Build libw4a16.so (gfx950) in-tree with hipcc.

    python -m w4a16_decode_gemv_amd.build
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libw4a16.so")
SOURCES = ["abi.hip", "awq_quantize.hip", "norm_fold.hip", "gemv.hip", "gemm_skinny.hip", "gemm_mfma.hip", "awq_search.hip", "gemm_splitk.hip", "stream_read.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def command(out=LIB, extra=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return [hipcc, *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose=False):
    """Compile every HIP source into one shared library; raises on failure."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
