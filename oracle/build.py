"""Compile the CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure: the oracle is the checker for the GPU library and shares no
code with it. Flags keep the arithmetic exactly as written: no -ffast-math, no
floating-point contraction, no target-specific instruction sets (the library is
built here and may run on a different x86-64 host).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
          "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile `src` (default oracle.c) into the shared library `out` and return its path.

    Always recompiles. The library is written under a temporary name first and then
    renamed, so a concurrent loader never sees a half-written file.
    """
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
