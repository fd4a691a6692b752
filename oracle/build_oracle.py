"""Builds the CPU oracle shared library (test infrastructure only).

The oracle is plain single-threaded C++ compiled with the host compiler, with
contraction into fused multiply-adds switched off so that every operation is one
IEEE rounding, as the oracle's arithmetic assumes.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zero_oracle.cpp")
FLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
         "-shared", "-Wall", "-Wextra"]


def lib_path(mutant=0, outdir=None):
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(outdir or HERE, name)


def build(mutant=0, outdir=None, quiet=True):
    """Compile the oracle (or a planted-mistake variant) and return the .so path."""
    out = lib_path(mutant, outdir)
    cmd = ["g++", *FLAGS, f"-DORACLE_MUTANT={int(mutant)}", SRC, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if not quiet and res.stderr:
        sys.stderr.write(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
