"""Builds libzero.so, the C-ABI library of the fused step, for gfx950, and
libzceil.so, the streaming-ceiling kernels that bench.py measures the memory
system with.

The host layer (zero_abi.cpp) is compiled with g++; the kernels
(zero_kernels.hip) and the stream helpers (zero_runtime.hip) with hipcc for
gfx950. Both with multiply-add contraction
off and IEEE division / square root, because the step's result is defined
operation by operation. Packed fp32 instructions are disabled for the device
code.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libzero.so")
CEIL_LIB = os.path.join(HERE, "libzceil.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("ZERO_OFFLOAD_ARCH", "gfx950")

HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math", "-Wall",
              "-Wextra", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res


def build(verbose=False):
    """Compile both translation units and link libzero.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    abi_o = os.path.join(BUILD, "zero_abi.o")
    ker_o = os.path.join(BUILD, "zero_kernels.o")
    rt_o = os.path.join(BUILD, "zero_runtime.o")
    steps = [
        ["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "zero_abi.cpp"), "-o", abi_o],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "zero_kernels.hip"), "-o", ker_o],
        [HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "zero_runtime.hip"), "-o", rt_o],
        [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", abi_o, ker_o, rt_o, "-o",
         LIB + ".tmp"],
    ]
    for cmd in steps:
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
    os.replace(LIB + ".tmp", LIB)
    ceil = [HIPCC, *HIP_FLAGS, "-shared", os.path.join(CSRC, "stream_ceiling.hip"), "-o",
            CEIL_LIB + ".tmp"]
    if verbose:
        print(" ".join(ceil), flush=True)
    _run(ceil)
    os.replace(CEIL_LIB + ".tmp", CEIL_LIB)
    return LIB


def device_asm(out_path):
    """Write the gfx950 assembly of the kernels (for inspecting the instruction mix)."""
    cmd = [HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, "zero_kernels.hip"),
           "-o", out_path]
    _run(cmd)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
    if shutil.which("nm"):
        pass
