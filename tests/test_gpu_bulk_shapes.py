"""GPU parity of the bulk launch shapes, every element against the oracle.

The fp32 and mixed-precision steps launch one of two shapes by size: the bulk
shape (one stream in flight per wave, a cap on resident blocks per CU) from
about 12.6 M elements up, the wide shape below. The other parity tests run
either far below that (a few M elements, every element) or at full size
(sampled). Here the bulk shape runs at sizes every element of which the oracle
can check: 13 M elements plus a ragged tail, so the last tile is partial and a
few elements sit past the last whole group; AdamW with and without the decay
bitmask, momentum SGD, a rank share, the mean store and the clipped step from
the materialised mean. The same vector stepped as two
buckets (each below the threshold, so in the wide shape) must match the
one-shot bulk launch bit for bit.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import zero_sharded_optimizer_amd as z  # noqa: E402
from zero_sharded_optimizer_amd import synth  # noqa: E402
from oracle import MODE_F32, MODE_MIXED, MODE_MIXED_F16  # noqa: E402
from gpu_cases import check_all, compare_bits, host, kinds, run_full, say, setup  # noqa: E402
from test_gpu_sgd import run_sgd  # noqa: E402

W = synth.WORKLOADS
BASE = {MODE_F32: W["fp32-320M-n8"], MODE_MIXED: W["mixed-1B-n8"],
        MODE_MIXED_F16: W["mixed-fp16-1B-n8"]}
# above the bulk threshold of every mode on a 256-CU MI355X, not a multiple of 8
N_BULK = 13_000_037


@pytest.mark.parametrize("mode", [MODE_F32, MODE_MIXED, MODE_MIXED_F16])
def test_bulk_shape_every_element(oracle, mode):
    run_full(oracle, synth.scaled(BASE[mode], N_BULK, weight_decay=0.1, decay="all"), steps=3)


def test_bulk_shape_rank_share(oracle):
    """Rank 3's share of 13 M elements: shard-local master/m/v, chunk gradients,
    the bf16 slot written at an unaligned offset of the gathered buffer."""
    run_full(oracle, synth.scaled(W["mixed-rank0-of-8B-n8"], 8 * N_BULK + 5, rank=3), steps=2)


# a GPT-2-shaped tensor list of 13,962,240 elements: 2-D tensors decay, the rest not
MASKED_SHAPES = synth.gpt2_small_shapes(vocab=20000, ctx=512, d=320, layers=6)


@pytest.mark.parametrize("mode", [MODE_F32, MODE_MIXED])
def test_bulk_shape_with_decay_mask(oracle, mode):
    """AdamW with the 2-D decay bitmask read inside the bulk shape's serial loads."""
    wl = synth.scaled(BASE[mode], 0, shapes=MASKED_SHAPES, decay="2d", weight_decay=0.1)
    assert wl.n > N_BULK - 1_000_000
    run_full(oracle, wl, steps=2)


@pytest.mark.parametrize("mode", [MODE_F32, MODE_MIXED])
def test_bulk_shape_momentum_sgd(oracle, mode):
    """The SGD kernel variant (no v stream) in the bulk shape."""
    run_sgd(oracle, synth.scaled(BASE[mode], N_BULK, decay="all", worker_scale=None),
            "nesterov+decay", 3)


@pytest.mark.parametrize("mode", [MODE_F32, MODE_MIXED])
def test_bulk_one_shot_equals_wide_buckets(mode):
    wl = synth.scaled(BASE[mode], N_BULK, weight_decay=0.1, decay="all")
    say(f"[case] bulk vs two wide buckets mode={mode} n={wl.n}")
    hp, p_one, s_one, _ = setup(wl)
    _, p_two, s_two, _ = setup(wl)
    half = (wl.n // 2) // 8 * 8
    for t in (1, 2):
        grads = synth.make_grads(wl, t, "cuda")
        z.zero_step(hp, p_one, grads, s_one, t)
        z.zero_step_range(hp, p_two, grads, s_two, t, half, wl.n)
        z.zero_step_range(hp, p_two, grads, s_two, t, 0, half)
    torch.cuda.synchronize()
    pk, sk = kinds(wl)
    compare_bits("param", host(p_two), host(p_one), pk)
    compare_bits("m", host(s_two.m), host(s_one.m), sk)
    compare_bits("v", host(s_two.v), host(s_one.v), sk)
    if s_one.master is not None:
        compare_bits("master", host(s_two.master), host(s_one.master), sk)


def test_bulk_step_with_mean_store(oracle):
    """zero_step_with_mean in the bulk shape: the stored mean and every output."""
    wl = synth.scaled(BASE[MODE_MIXED], N_BULK, weight_decay=0.1, decay="all")
    say(f"[case] bulk step with mean store n={wl.n}")
    hp, param, st, _ = setup(wl)
    p_h = host(param)
    mst_h, m_h, v_h = oracle.init_states(wl.mode, p_h)
    mean = torch.empty(wl.n, dtype=torch.float32, device="cuda")
    for t in (1, 2):
        grads = synth.make_grads(wl, t, "cuda")
        g_h = [host(g) for g in grads]
        z.zero_step_with_mean(hp, param, grads, st, t, mean)
        mean_h, _ = oracle.mean_grad(wl.mode, wl.n, wl.n_workers, g_h)
        p_h, mst_h, m_h, v_h = oracle.zero_step(wl.mode, p_h, g_h, mst_h, m_h, v_h, t, wl.lr,
                                                wl.beta1, wl.beta2, wl.eps, wl.weight_decay, None)
    torch.cuda.synchronize()
    compare_bits("mean", host(mean), mean_h, "f32")
    check_all("bulk with mean", wl, host(param), st, (p_h, mst_h, m_h, v_h))


def test_bulk_step_from_clipped_mean(oracle):
    """The clipped step's second pass (the step from the materialised fp32 mean)
    in its bulk shape, with the factor at exactly 1 (bit-exact) and below 1 (the
    oracle driven by the device's squared norm, bit-exact too)."""
    wl = synth.scaled(BASE[MODE_MIXED], N_BULK, weight_decay=0.1, decay="all")
    say(f"[case] bulk clipped step n={wl.n}")
    hp, param, st, _ = setup(wl)
    ws = torch.empty(max(1, z.zero_step_clipped_workspace_bytes(hp)), dtype=torch.uint8,
                     device="cuda")
    ss = torch.zeros(1, dtype=torch.float64, device="cuda")
    p_h = host(param)
    mst_h, m_h, v_h = oracle.init_states(wl.mode, p_h)
    for t, scale in ((1, 3.0), (2, 0.3)):
        grads = synth.make_grads(wl, t, "cuda")
        g_h = [host(g) for g in grads]
        mean_h, ss_h = oracle.mean_grad(wl.mode, wl.n, wl.n_workers, g_h)
        max_norm = scale * math.sqrt(ss_h)
        z.zero_step_clipped(hp, param, grads, st, t, max_norm, ws, sumsq_out=ss)
        torch.cuda.synchronize()
        p_h, mst_h, m_h, v_h = oracle.step_mean(wl.mode, wl.n_workers, p_h, mean_h, mst_h, m_h,
                                                v_h, t, wl.lr, wl.beta1, wl.beta2, wl.eps,
                                                wl.weight_decay, None,
                                                clip_sumsq=float(ss.item()), max_norm=max_norm)
    check_all("bulk clipped", wl, host(param), st, (p_h, mst_h, m_h, v_h))
    assert np.isfinite(host(st.m)).all()
