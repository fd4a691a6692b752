"""Step scalars in device memory (zero_step_range_dev) and HIP graph capture.

zero_step_range_dev takes the step-dependent scalars (bias corrections, SGD's
first-step flag) from a device buffer, so a launch captured once into a graph
can be replayed for every later step. Checked bit for bit against the eager
zero_step on separate buffers driven by the same gradients:
  * eagerly, bucket by bucket, in every mode, rank mode and SGD;
  * as a captured graph of all buckets, replayed for steps 1..4 with the next
    step's scalars copied in before each replay, eager work and
    synchronisations in between, and every replay compared.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import zero_sharded_optimizer_amd as z  # noqa: E402
from zero_sharded_optimizer_amd import synth  # noqa: E402
from oracle import MODE_F32, MODE_F64, MODE_MIXED, MODE_MIXED_F16  # noqa: E402
from gpu_cases import say, setup  # noqa: E402

W = synth.WORKLOADS
BASE = {MODE_F64: W["fp64-1M-n4"], MODE_F32: W["fp32-320M-n8"], MODE_MIXED: W["mixed-1B-n8"],
        MODE_MIXED_F16: W["mixed-fp16-1B-n8"]}


def _bits(x):
    return x.view({torch.bfloat16: torch.int16, torch.float16: torch.int16, torch.float64: torch.int64,
                   torch.float32: torch.int32}[x.dtype])


def _same_state(p1, s1, p2, s2):
    assert torch.equal(_bits(p1), _bits(p2))
    for a, b in ((s1.m, s2.m), (s1.v, s2.v), (s1.master, s2.master)):
        if a is not None:
            assert torch.equal(_bits(a), _bits(b))


def _buckets(length, size):
    edges = list(range(0, length, size)) + [length]
    return list(reversed(list(zip(edges[:-1], edges[1:]))))


def _scalars_to(dev, hp, t):
    dev.copy_(torch.from_numpy(z.zero_step_scalars(hp, t)))


def _sgd(hp):
    hp.optimizer, hp.momentum, hp.dampening, hp.nesterov = z.ZERO_OPT_SGD, 0.9, 0.0, True
    hp.weight_decay = 0.01
    return hp


CASES = {
    "fp64": (MODE_F64, -1, False), "fp32": (MODE_F32, -1, False),
    "mixed": (MODE_MIXED, -1, False), "mixed-rank3": (MODE_MIXED, 3, False),
    "fp16": (MODE_MIXED_F16, -1, False), "fp16-rank5": (MODE_MIXED_F16, 5, False),
    "fp32-sgd": (MODE_F32, -1, True), "mixed-sgd": (MODE_MIXED, -1, True),
}


def _pair(name):
    mode, rank, sgd = CASES[name]
    wl = synth.scaled(BASE[mode], 400_003, weight_decay=0.05, decay="all",
                      n_workers=8 if mode != MODE_F64 else 4, rank=rank)
    hp, p_ref, s_ref, _ = setup(wl)
    _, p_dev, s_dev, _ = setup(wl)
    if sgd:
        hp = _sgd(hp)
        for s in (s_ref, s_dev):
            s.v = None
    return wl, hp, p_ref, s_ref, p_dev, s_dev


@pytest.mark.parametrize("name", sorted(CASES))
def test_device_scalars_equal_the_eager_step(name):
    wl, hp, p_ref, s_ref, p_dev, s_dev = _pair(name)
    say(f"[case] device scalars, eager, {name}")
    a, b = wl.shard
    scal = torch.empty(z.STEP_SCALARS_BYTES, dtype=torch.uint8, device="cuda")
    for t in (1, 2, 3):
        grads = synth.make_grads(wl, t, "cuda")
        z.zero_step(hp, p_ref, grads, s_ref, t)
        _scalars_to(scal, hp, t)
        for lo, hi in _buckets(b - a, 65_536):
            z.zero_step_range_dev(hp, p_dev, grads, s_dev, scal, lo, hi)
        torch.cuda.synchronize()
        _same_state(p_ref, s_ref, p_dev, s_dev)


@pytest.mark.parametrize("name", ["fp32", "mixed", "fp32-sgd", "mixed-rank3", "fp16"])
def test_captured_buckets_replay_for_later_steps(name):
    wl, hp, p_ref, s_ref, p_dev, s_dev = _pair(name)
    say(f"[case] graph of buckets, {name}")
    a, b = wl.shard
    grads = synth.make_grads(wl, 1, "cuda")
    # the graph reads these buffers; each step copies new gradients into them
    g_buf = [g.clone() for g in grads]
    scal = torch.empty(z.STEP_SCALARS_BYTES, dtype=torch.uint8, device="cuda")
    buckets = _buckets(b - a, 32_768)
    # capture on a side stream (the launches enqueue nothing else)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for lo, hi in buckets:
                z.zero_step_range_dev(hp, p_dev, g_buf, s_dev, scal, lo, hi)
    torch.cuda.synchronize()
    # capture enqueued no work: the buffers are still as set up
    _same_state(p_ref, s_ref, p_dev, s_dev)
    for t in (1, 2, 3, 4):
        grads = synth.make_grads(wl, t, "cuda")
        for dst, src in zip(g_buf, grads):
            dst.copy_(src)
        _scalars_to(scal, hp, t)
        graph.replay()
        torch.cuda.synchronize()
        z.zero_step(hp, p_ref, grads, s_ref, t)  # eager work between the replays
        torch.cuda.synchronize()
        _same_state(p_ref, s_ref, p_dev, s_dev)
        say(f"  replay t={t}: bit-identical to the eager step ({len(buckets)} buckets)")
