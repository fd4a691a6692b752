"""GPU parity: the fused HIP step through the C ABI against the CPU oracle.

Bar (oracle/compare.py): fp64 bit-exact; fp32 master/m/v within
1e-6 * max(1, |ref|); bf16 gathered parameters within 1 bf16 ulp.
"""
import json
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import zero_sharded_optimizer_amd as z  # noqa: E402
from zero_sharded_optimizer_amd import synth  # noqa: E402
from oracle import MODE_F32, MODE_F64, MODE_MIXED, MODE_MIXED_F16  # noqa: E402
from gpu_cases import host, run_full, run_sampled, say, setup  # noqa: E402

W = synth.WORKLOADS
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _hp(n, N, mode, lr, **kw):
    d = dict(beta1=0.9, beta2=0.999, eps=1e-8)
    d.update(kw)
    return z.HParams(n=n, n_workers=N, mode=mode, lr=lr, **d)


# -- the pages' worked examples on the device ---------------------------------
def test_p2_worked_example_on_gpu(oracle):
    g = json.load(open(os.path.join(GOLDEN, "p2_worked_example.json")))
    say("[case] p2 worked example")
    param = torch.tensor(g["param"], dtype=torch.float64, device="cuda")
    grads = [torch.tensor(x, dtype=torch.float64, device="cuda") for x in g["grads"]]
    st = z.States(None, torch.empty(5, dtype=torch.float64, device="cuda"),
                  torch.empty(5, dtype=torch.float64, device="cuda"))
    hp = _hp(5, 2, MODE_F64, g["lr"])
    z.zero_init_states(hp, param, st)
    z.zero_step(hp, param, grads, st, 1)
    got = host(param)
    assert np.all(np.abs(got - np.array(g["result"])) <= g["result_tolerance"])
    assert got[3] == 1.0
    ref = oracle.zero_step(MODE_F64, np.array(g["param"]), [np.array(x) for x in g["grads"]],
                           None, np.zeros(5), np.zeros(5), 1, g["lr"])
    assert np.array_equal(got, ref[0]) and np.array_equal(host(st.m), ref[2])
    assert np.array_equal(host(st.v), ref[3])


def test_p1_worked_example_on_gpu(oracle):
    g = json.load(open(os.path.join(GOLDEN, "p1_worked_example.json")))
    say("[case] p1 worked example")
    w = np.arange(10, dtype=np.float64)
    param = torch.tensor(w, device="cuda")
    grads = [torch.tensor(w - r, device="cuda") for r in range(4)]
    st = z.States(None, torch.empty(10, dtype=torch.float64, device="cuda"),
                  torch.empty(10, dtype=torch.float64, device="cuda"))
    hp = _hp(10, 4, MODE_F64, g["lr"])
    z.zero_init_states(hp, param, st)
    z.zero_step(hp, param, grads, st, 1)
    got = host(param)
    assert np.all(np.abs(got - np.array(g["result"])) <= g["result_tolerance"])
    ref = oracle.zero_step(MODE_F64, w, [w - r for r in range(4)], None, np.zeros(10),
                           np.zeros(10), 1, g["lr"])
    assert np.array_equal(got, ref[0])


# -- full-vector parity at oracle-sized inputs --------------------------------
def test_fp64_1M_n4_full_size_every_element(oracle):
    """fp64, n = 1,048,579 over 4 uneven shards, t = 1..10, every element bit-exact."""
    run_full(oracle, W["fp64-1M-n4"], steps=10)


@pytest.mark.parametrize("n", [3_000_017, 1_000_000])
def test_fp32_n8_worker_scales(oracle, n):
    run_full(oracle, synth.scaled(W["fp32-320M-n8"], n), steps=5)


# sizes: 3,000,017 takes the modes' own launch shapes (at least two blocks per
# CU); 4096 and the smaller cases take the small-launch shape
@pytest.mark.parametrize("n", [3_000_017, 4096])
def test_mixed_n8_bf16(oracle, n):
    run_full(oracle, synth.scaled(W["mixed-1B-n8"], n), steps=5)


@pytest.mark.parametrize("n", [3_000_017, 4096])
def test_mixed_n8_fp16(oracle, n):
    run_full(oracle, synth.scaled(W["mixed-fp16-1B-n8"], n), steps=5)


@pytest.mark.parametrize("N", [5, 64])
def test_fp32_any_n_in_its_own_shape(oracle, N):
    """Worker counts other than 1, 2, 4 and 8 at a size that takes the any-N
    kernel's own 128 x 8 shape, with a ragged last tile."""
    wl = synth.scaled(W["fp32-320M-n8"], 3_000_017 if N == 5 else 2_500_011, n_workers=N,
                      worker_scale=None)
    run_full(oracle, wl, steps=3)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_mixed_rank_share_adamw(oracle, rank):
    """One rank's share: chunk gradients and shard-local master/m/v; ragged
    shards make ranks > 0 start at an unaligned slot of the gathered buffer."""
    wl = synth.scaled(W["mixed-rank0-of-8B-n8"], 8 * 250_001 + 5, rank=rank)
    run_full(oracle, wl, steps=4)


@pytest.mark.parametrize("mode", [MODE_F64, MODE_F32, MODE_MIXED_F16])
def test_rank_share_other_modes(oracle, mode):
    base = W["fp32-320M-n8"]
    wl = synth.scaled(base, 5 * 100_003 + 3, rank=2, mode=mode, n_workers=5, weight_decay=0.05,
                      decay="all", worker_scale=None)
    run_full(oracle, wl, steps=3)


def test_gpt2_shaped_tensor_list_n64_decay_mask(oracle):
    """A small GPT-2-shaped tensor list (same structure, smaller widths) with 64
    workers, so shards cut through tensors; decay on 2-D tensors only."""
    shapes = synth.gpt2_small_shapes(vocab=1000, ctx=64, d=96, layers=2)
    wl = synth.scaled(W["gpt2s-fp32-n64"], 0, shapes=shapes)
    starts, n = synth.tensor_starts(shapes)
    cut = sum(1 for r in range(1, 64) for s in starts if
              z.zero_shard_bounds(n, 64, r - 1)[0] < s < z.zero_shard_bounds(n, 64, r - 1)[1])
    assert cut > 0
    run_full(oracle, wl, steps=6, compare_every=2)


# -- edge cases ---------------------------------------------------------------
@pytest.mark.parametrize("mode", [MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16])
@pytest.mark.parametrize("n,N", [(1, 1), (3, 5), (7, 2), (9, 3), (17, 100), (1029, 256),
                                 (100_001, 64), (65_537, 6)])
def test_edge_shapes(oracle, mode, n, N):
    """Tiny and ragged vectors, N > n (empty shards), N not a power of two, and
    the largest N the call accepts."""
    base = {MODE_F64: W["fp64-1M-n4"], MODE_F32: W["fp32-320M-n8"], MODE_MIXED: W["mixed-1B-n8"],
            MODE_MIXED_F16: W["mixed-fp16-1B-n8"]}[mode]
    wl = synth.scaled(base, n, n_workers=N, worker_scale=None, zero_frac=0.0)
    run_full(oracle, wl, steps=3)


def test_zero_mean_gradient_leaves_parameter(oracle):
    """With a zero mean gradient m = v = 0 and the update is 0/(0 + eps) = 0
    ('ZeRO-Sharded Adam Step', section 'The step': the parameter does not move)."""
    say("[case] zero mean gradient")
    n = 4099
    for mode, dt in ((MODE_F64, torch.float64), (MODE_F32, torch.float32)):
        param = torch.randn(n, dtype=dt, device="cuda")
        before = param.clone()
        g0 = torch.randn(n, dtype=dt, device="cuda")
        st = z.States(None, torch.empty(n, dtype=dt, device="cuda"),
                      torch.empty(n, dtype=dt, device="cuda"))
        hp = _hp(n, 2, mode, 0.1)
        z.zero_init_states(hp, param, st)
        z.zero_step(hp, param, [g0, -g0], st, 1)
        torch.cuda.synchronize()
        assert torch.equal(param, before) and not st.m.any() and not st.v.any()


def test_empty_rank_shard_on_gpu():
    say("[case] empty rank shard")
    n, N = 3, 5
    param = torch.arange(n, dtype=torch.float32, device="cuda")
    z0 = torch.empty(0, dtype=torch.float32, device="cuda")
    st = z.States(torch.empty(4, device="cuda"), torch.empty(4, device="cuda"),
                  torch.empty(4, device="cuda"))
    hp = _hp(n, N, MODE_F32, 0.1, rank=4)
    z.zero_init_states(hp, param, st)
    z.zero_step(hp, param, [z0] * N, st, 1)
    torch.cuda.synchronize()
    assert param.tolist() == [0.0, 1.0, 2.0]


def test_resume_from_saved_state_is_bit_exact(tmp_path):
    """The optimizer state (master, m, v, t) is caller-owned: 10 steps equal 5
    steps, a round trip of the state through a file, then 5 more."""
    say("[case] resume equivalence")
    wl = synth.scaled(W["mixed-1B-n8"], 300_007)

    def run(steps, hp, param, st, t0=1):
        for t in range(t0, t0 + steps):
            z.zero_step(hp, param, synth.make_grads(wl, t, "cuda"), st, t)

    hp, pa, sa, _ = setup(wl)
    run(10, hp, pa, sa)
    hp, pb, sb, _ = setup(wl)
    run(5, hp, pb, sb)
    torch.cuda.synchronize()
    f = tmp_path / "state.pt"
    torch.save({"param": pb.cpu(), "master": sb.master.cpu(), "m": sb.m.cpu(), "v": sb.v.cpu(),
                "t": 5}, f)
    del pb, sb
    d = torch.load(f, weights_only=True)
    pc = d["param"].cuda()
    sc = z.States(d["master"].cuda(), d["m"].cuda(), d["v"].cuda())
    run(5, hp, pc, sc, t0=d["t"] + 1)
    torch.cuda.synchronize()
    assert torch.equal(pa.view(torch.int16), pc.view(torch.int16))
    for x, y in ((sa.master, sc.master), (sa.m, sc.m), (sa.v, sc.v)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_stream_ordering_on_a_side_stream(oracle):
    """The step is enqueued on the stream it is given."""
    from oracle.compare import compare
    say("[case] side stream")
    wl = synth.scaled(W["fp32-320M-n8"], 200_003)
    hp, param, st, _ = setup(wl)
    grads = synth.make_grads(wl, 1, "cuda")
    torch.cuda.synchronize()
    p0 = host(param)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        z.zero_step(hp, param, grads, st, 1)
    s.synchronize()
    ref = oracle.zero_step(MODE_F32, p0, [host(g) for g in grads], None,
                           np.zeros(wl.n, np.float32), np.zeros(wl.n, np.float32), 1, wl.lr,
                           wl.beta1, wl.beta2, wl.eps)
    compare("side stream param", host(param), ref[0], "f32")
    compare("side stream m", host(st.m), ref[2], "f32")


# -- full-size workloads, sampled parity, in the launch configuration the
#    benchmark times --------------------------------------------------------
def test_full_size_fp32_320M_n8(oracle):
    run_sampled(oracle, W["fp32-320M-n8"], steps=20, count=1 << 20, compare_steps=[1, 2, 10])


def test_full_size_mixed_1B_n8(oracle):
    run_sampled(oracle, W["mixed-1B-n8"], steps=10, count=1 << 20, compare_steps=[1, 5])


def test_full_size_mixed_fp16_1B_n8(oracle):
    run_sampled(oracle, W["mixed-fp16-1B-n8"], steps=10, count=1 << 20, compare_steps=[1, 5])


def test_full_size_rank0_share_of_8B(oracle):
    run_sampled(oracle, W["mixed-rank0-of-8B-n8"], steps=5, count=1 << 20, compare_steps=[1, 3])


def test_full_size_gpt2s_n64(oracle):
    run_sampled(oracle, W["gpt2s-fp32-n64"], steps=100, count=1 << 18,
                compare_steps=[1, 2, 50])


# -- maximum sizes: byte offsets past 2^32 and element indexes past 2^31 ------
def test_buffers_past_4_GiB_any_N(oracle):
    """fp32 with N = 3 (the any-N kernel): every buffer holds 4.4 GB, so byte
    offsets within one buffer pass 2^32."""
    wl = synth.scaled(W["fp32-320M-n8"], 1_100_000_003, n_workers=3)
    run_sampled(oracle, wl, steps=2, count=1 << 18)


def test_more_than_2_31_elements_mixed(oracle):
    """Mixed precision with N = 2 over 2.2e9 elements: element indexes pass
    2^31 and the fp32 state buffers hold 8.8 GB."""
    wl = synth.scaled(W["mixed-1B-n8"], 2_200_000_005, n_workers=2)
    run_sampled(oracle, wl, steps=2, count=1 << 18)


def test_more_than_2_32_elements_in_two_launches(oracle):
    """Mixed precision with N = 2 over 2^32 + 1001 elements: the library enqueues
    the step as two launches (2^32 elements, then 1001) on offset views. The last
    4096 sampled elements straddle the seam between them."""
    wl = synth.scaled(W["mixed-1B-n8"], (1 << 32) + 1001, n_workers=2)
    run_sampled(oracle, wl, steps=2, count=1 << 18)


def test_last_rank_share_of_8B(oracle):
    """Rank 7 of n = 8e9: its slot in the gathered bf16 buffer starts 14 GB in;
    everything outside the slot stays unchanged."""
    wl = synth.scaled(W["mixed-rank0-of-8B-n8"], 8_000_000_000, rank=7,
                      name="mixed-rank7-of-8B-n8")
    run_sampled(oracle, wl, steps=2, count=1 << 18)
