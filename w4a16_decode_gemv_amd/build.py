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
SOURCES = ["abi.hip", "awq_quantize.hip", "norm_fold.hip", "gemv.hip", "gemm_skinny.hip", "gemm_mfma.hip", "awq_search.hip", "gemm_splitk.hip", "stream_read.hip", "gemm_klane.hip", "gemm_xres.hip"]
# gemm_skinny.hip holds many kernel instances: it compiles as five parts in parallel
PARTS = {"gemm_skinny.hip": 5}
# per-source code generation flags: the tiled MFMA kernels keep their MFMA accumulators in
# ordinary VGPRs (in AGPRs each accumulator read by the scale FMAs costs a v_accvgpr_read)
SOURCE_FLAGS = {"gemm_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "gemm_klane.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
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


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def command(out=LIB, extra=()):
    """The one-step command (every source in one hipcc call); kept for reference builds."""
    return [_hipcc(), *FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def _filter(text):
    noise = "is not a recognized feature for this target"
    return [ln for ln in text.splitlines() if noise not in ln]


def build(verbose=False, jobs=None):
    """Compile every HIP source (one hipcc per source, in parallel) and link them into one
    shared library; raises on failure."""
    import concurrent.futures
    import tempfile

    jobs = jobs or min(8, max(1, len(os.sched_getaffinity(0))))
    compile_flags = [f for f in FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as tmpdir:
        units = []
        for src in SOURCES:
            if src in PARTS:
                units += [(src, f"-DW4A16_SKINNY_PART={p}", f"{os.path.splitext(src)[0]}_{p}.o") for p in range(PARTS[src])]
            else:
                units.append((src, None, os.path.splitext(src)[0] + ".o"))

        def one(unit):
            src, define, objname = unit
            obj = os.path.join(tmpdir, objname)
            cmd = [_hipcc(), *compile_flags, *SOURCE_FLAGS.get(src, []), *([define] if define else []), "-c",
                   f"-I{INCLUDE}", f"-I{CSRC}",
                   "-o", obj, os.path.join(CSRC, src)]
            res = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, res

        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(one, units))
        msgs = []
        for src, _, res in results:
            m = _filter(res.stdout + res.stderr)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(m))
            msgs += m
        tmp = LIB + ".tmp"
        link = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *[obj for _, obj, _ in results]]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(_filter(res.stdout + res.stderr)))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
