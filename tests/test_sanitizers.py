"""The host-side C++ under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers are built with g++ and the sanitizers and run as subprocesses:
  * tests/sanitize/host_driver.cpp links the C-ABI host layer (zero_abi.cpp)
    with stub launchers, and drives validation, shard bounds, the memory model
    and the workspace sizes;
  * tests/sanitize/oracle_driver.cpp links the CPU oracle and drives its entry
    points on random shapes, checking the sharded/shard-free and rank-share
    invariants.
Any sanitizer report fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1", "-std=c++17", "-ffp-contract=off"]


def _build_and_run(tmp_path, name, sources, includes=()):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / name)
    cmd = ["g++", *SAN, *[f"-I{i}" for i in includes], *sources, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    return out


def test_host_abi_layer_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "zero_sharded_optimizer_amd", "csrc")
    out = _build_and_run(tmp_path, "host_driver",
                         [os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
                          os.path.join(csrc, "zero_abi.cpp")],
                         includes=[os.path.join(ROOT, "include"), csrc])
    assert "0 failures" in out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "oracle_driver",
                         [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.cpp"),
                          os.path.join(ROOT, "oracle", "zero_oracle.cpp")])
    assert "0 failures" in out
