"""zero_mean_grad_noalloc against zero_mean_grad: the same kernels, with the
squared norm's partial sums in the library's static device scratch instead of
a caller workspace. Two calls in a row on one GPU, the second on a smaller
input, each must match the workspace entry point's outputs bit for bit (the
mean and the squared norm), and the mean must match the oracle's bit for bit.
The scratch keeps the previous call's contents, so the second call also shows
that nothing stale leaks into its result."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import zero_sharded_optimizer_amd as z  # noqa: E402
from zero_sharded_optimizer_amd import synth  # noqa: E402
from oracle import MODE_F32, MODE_F64, MODE_MIXED, MODE_MIXED_F16  # noqa: E402
from gpu_cases import compare_bits, host, say  # noqa: E402

W = synth.WORKLOADS
BASE = {MODE_F64: W["fp64-1M-n4"], MODE_F32: W["fp32-320M-n8"], MODE_MIXED: W["mixed-1B-n8"],
        MODE_MIXED_F16: W["mixed-fp16-1B-n8"]}


def _one(oracle, mode, n, N, rank, seed):
    wl = synth.scaled(BASE[mode], n, n_workers=N, worker_scale=None, rank=rank,
                      seed=BASE[mode].seed + seed)
    hp = z.HParams(n=n, n_workers=N, mode=mode, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                   eps=wl.eps, rank=rank)
    L = wl.length
    grads = synth.make_grads(wl, 1, "cuda")
    sdt = synth.state_dtype(wl)
    mean_a = torch.full((L,), float("nan"), dtype=sdt, device="cuda")
    mean_b = torch.full((L,), float("nan"), dtype=sdt, device="cuda")
    ss_a = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    ss_b = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    ws = torch.empty(max(1, z.zero_mean_grad_workspace_bytes(hp)), dtype=torch.uint8,
                     device="cuda")
    z.zero_mean_grad_noalloc(hp, grads, mean_a, ss_a)
    z.zero_mean_grad(hp, grads, mean_b, ss_b, ws)
    torch.cuda.synchronize()
    compare_bits("noalloc mean vs workspace mean", host(mean_a), host(mean_b), "exact")
    assert ss_a.item() == ss_b.item(), (ss_a.item(), ss_b.item())
    mean_h, ss_h = oracle.mean_grad(mode, n, N, [host(g) for g in grads], rank=rank)
    compare_bits("noalloc mean vs oracle", host(mean_a), mean_h, "exact")
    assert abs(ss_a.item() - ss_h) <= 2 * L * 2.0 ** -53 * abs(ss_h) + 1e-300
    return ss_a.item()


@pytest.mark.parametrize("mode", [MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16])
def test_noalloc_mean_grad_twice_second_smaller(oracle, mode):
    say(f"[case] zero_mean_grad_noalloc mode={mode}: 3,000,017 x 8, then 40,009 x 5")
    big = _one(oracle, mode, 3_000_017, 8, -1, 1)
    small = _one(oracle, mode, 40_009, 5, -1, 2)
    assert math.isfinite(big) and math.isfinite(small) and small < big


def test_noalloc_mean_grad_rank_mode_and_no_norm(oracle):
    say("[case] zero_mean_grad_noalloc rank mode, then no squared norm")
    _one(oracle, MODE_MIXED, 8 * 250_001 + 5, 8, 3, 3)
    _one(oracle, MODE_MIXED, 8 * 1_001 + 5, 8, 7, 4)
    n, N = 10_007, 3
    wl = synth.scaled(BASE[MODE_F32], n, n_workers=N, worker_scale=None)
    hp = z.HParams(n=n, n_workers=N, mode=MODE_F32, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                   eps=wl.eps)
    grads = synth.make_grads(wl, 1, "cuda")
    mean = torch.empty(n, device="cuda")
    z.zero_mean_grad_noalloc(hp, grads, mean, None)
    torch.cuda.synchronize()
    mean_h, _ = oracle.mean_grad(MODE_F32, n, N, [host(g) for g in grads])
    compare_bits("noalloc mean without norm", host(mean), mean_h, "exact")


def test_noalloc_mean_grad_inside_a_captured_graph(oracle):
    """The reason for the entry point: it can be captured into a HIP graph (no
    allocation during capture). Replayed three times, with eager work and
    synchronisation between replays, each replay's mean and squared norm equal
    the eager workspace call's."""
    n, N = 500_009, 8
    wl = synth.scaled(BASE[MODE_MIXED], n, n_workers=N)
    say("[case] zero_mean_grad_noalloc captured in a graph, 3 replays")
    hp = z.HParams(n=n, n_workers=N, mode=MODE_MIXED, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                   eps=wl.eps)
    grads = synth.make_grads(wl, 1, "cuda")
    mean = torch.empty(n, device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    ref = torch.empty(n, device="cuda")
    ss_ref = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.empty(z.zero_mean_grad_workspace_bytes(hp), dtype=torch.uint8, device="cuda")
    z.zero_mean_grad(hp, grads, ref, ss_ref, ws)
    z.zero_mean_grad_noalloc(hp, grads, mean, ss)  # first call on the device: the lookup
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            z.zero_mean_grad_noalloc(hp, grads, mean, ss, stream=side)
    torch.cuda.synchronize()
    for rep in range(3):
        mean.fill_(float("nan"))
        ss.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(mean.view(torch.int32), ref.view(torch.int32)), rep
        assert ss.item() == ss_ref.item(), rep


def test_noalloc_clipped_step_composition(oracle):
    """A caller that cannot allocate composes the clipped step from the
    no-allocation mean (into its own mean buffer) and zero_step_mean; it must
    equal zero_step_clipped (workspace) bit for bit, with clipping active."""
    n, N = 700_001, 8
    wl = synth.scaled(BASE[MODE_MIXED], n, n_workers=N, weight_decay=0.1, decay="all")
    say("[case] clipped step from zero_mean_grad_noalloc + zero_step_mean")
    from gpu_cases import setup
    hp, p_a, s_a, _ = setup(wl)
    _, p_b, s_b, _ = setup(wl)
    mean = torch.empty(n, device="cuda")
    ss_a = torch.zeros(1, dtype=torch.float64, device="cuda")
    ss_b = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.empty(z.zero_step_clipped_workspace_bytes(hp), dtype=torch.uint8, device="cuda")
    for t in (1, 2, 3):
        grads = synth.make_grads(wl, t, "cuda")
        _, ss_h = oracle.mean_grad(wl.mode, n, N, [host(g) for g in grads])
        max_norm = 0.5 * math.sqrt(ss_h)
        z.zero_mean_grad_noalloc(hp, grads, mean, ss_a)
        z.zero_step_mean(hp, p_a, mean, s_a, t, ss_a, max_norm)
        z.zero_step_clipped(hp, p_b, grads, s_b, t, max_norm, ws, sumsq_out=ss_b)
    torch.cuda.synchronize()
    assert ss_a.item() == ss_b.item()
    for name, x, y in (("param", p_a, p_b), ("master", s_a.master, s_b.master), ("m", s_a.m, s_b.m),
                       ("v", s_a.v, s_b.v)):
        kind = "bf16" if x.dtype == torch.bfloat16 else "exact"
        compare_bits(name, host(x), host(y), kind)
