"""Builds tests/c_abi/zero_c_consumer, the plain-C consumer of the C ABI (test
infrastructure): gcc, C99, linked against libzero.so, the oracle's
liboracle.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "zero_sharded_optimizer_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "zero_c_consumer")


def build():
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}",
           os.path.join(HERE, "zero_c_consumer.c"), "-o", EXE + ".tmp",
           f"-L{PKG}", "-lzero", f"-L{ORACLE}", "-loracle", f"-L{os.path.join(ROCM, 'lib')}",
           "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../zero_sharded_optimizer_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("C consumer build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
