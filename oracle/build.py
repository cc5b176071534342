"""Build the CPU oracle's shared library (liboracle.so) with gcc.

Test infrastructure only.  Run as ``python -m oracle.build`` or through
``__graft_entry__.build()``.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "twell_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No FMA contraction and no fast-math: every sum is evaluated in the order the
# source writes it, so optimisation level and target ISA change no result.
CFLAGS = ["-O3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-shared", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra"]
ARCH_PORTABLE = "-march=x86-64-v3"  # the library that travels with the tree
ARCH_NATIVE = "-march=native"       # a copy built on the machine that times it


def build(verbose: bool = False, native: bool = False, out: str = None) -> str:
    """Build the oracle library: the portable one at oracle/liboracle.so, or
    (native=True, for timing on the machine at hand) one tuned for this CPU at
    `out`."""
    lib = out or (LIB if not native else LIB.replace(".so", "_native.so"))
    tmp = lib + ".tmp"
    cmd = ["gcc", *CFLAGS, ARCH_NATIVE if native else ARCH_PORTABLE, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def build_command(native: bool) -> str:
    return " ".join(["gcc", *CFLAGS, ARCH_NATIVE if native else ARCH_PORTABLE])


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
