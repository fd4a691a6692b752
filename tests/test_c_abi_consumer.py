"""The C ABI from plain C (tests/c_abi/zero_c_consumer.c): no Python, no torch.
On the host it checks shard bounds, the memory model, rejection with a message
and the step scalars; on the GPU it allocates with the HIP runtime, runs
init_states and three fused steps in fp64, fp32 and mixed precision, then two
bucketed steps released by events from a producer stream, one clipped step, and
a step that stores the averaged gradient plus the no-allocation mean,
and compares with the oracle library on the same inputs."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "zero_c_consumer")


def _run(mode, timeout):
    if not os.path.exists(EXE):
        pytest.skip("zero_c_consumer not built (run __graft_entry__.build())")
    return subprocess.run([EXE, mode], capture_output=True, text=True, timeout=timeout)


def test_c_consumer_host_checks():
    res = _run("host", 60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host checks: 0 failures" in res.stdout


@pytest.mark.gpu
def test_c_consumer_steps_match_the_oracle():
    print("[case] plain-C consumer, gpu", flush=True)
    res = _run("gpu", 300)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "gpu run: 0 failures" in res.stdout
