"""Build libmm.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

    python -m tiled_gemm_gemv_amd.build        # or build() from Python

The library is written in-tree, next to this file, so it travels with the source
tree. Every HIP source is compiled with packed-fp32 instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmm.so")
SOURCES = ["mm_api.hip", "mm_gemm.hip", "mm_gemm_direct.hip", "mm_gemm_skinny.hip", "mm_gemm_cols.hip",
           "mm_gemm_h16.hip", "mm_gemm_narrow.hip",
           "mm_conv.hip",
           "mm_gemv.hip", "mm_gemv_t.hip", "mm_static_ws.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile libmm.so (always recompiles) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop
    # that note and show anything else.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if msgs and (verbose or r.returncode != 0):
        print("\n".join(msgs), file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
