"""Pins for the CPU oracle: each checks it against something other than itself.

Every pin takes an Oracle handle and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix:

  * values the pages print for their worked examples (tests/golden/),
  * closed forms (first-step move, constant-gradient trajectory, memory),
  * special cases that reduce to a library routine (torch.optim.Adam/AdamW with
    one worker, numpy.array_split, torch's bf16 and numpy's fp16 conversions),
  * invariants the pages state (sharded equals shard-free, a rank's share
    equals the shard of the full step).

The same pins run against oracle builds with a planted mistake
(tests/test_oracle_mutants.py) to show each mistake is caught.
"""
import json
import math
import os

import numpy as np

from oracle import MIXED_MODES, MODE_F32, MODE_F64, MODE_MIXED, MODE_MIXED_F16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(x_f32):
    """Round-to-nearest-even bf16 bits of fp32 values, via torch (a library routine)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _fp16_bits(x_f32):
    """Round-to-nearest-even IEEE binary16 bits of fp32 values, via numpy's
    conversion (a library routine)."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x_f32, dtype=np.float32).astype(np.float16).view(np.uint16)


def _fp16_widen(bits):
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------
def pin_p2_worked_example(O):
    """ZeRO-Sharded Adam Step, sections 'The shards' and 'The step'."""
    g = _golden("p2_worked_example.json")
    n, N = g["n"], g["n_workers"]
    shards = [list(range(*O.split_bounds(n, N, r))) for r in range(N)]
    assert shards == g["shards"], shards
    param = np.array(g["param"], np.float64)
    grads = [np.array(x, np.float64) for x in g["grads"]]
    _, m0, v0 = O.init_states(MODE_F64, param)
    assert not m0.any() and not v0.any()
    p1, _, m1, v1 = O.zero_step(MODE_F64, param, grads, None, m0, v0, g["t"], g["lr"])
    res = np.array(g["result"])
    assert np.all(np.abs(p1 - res) <= g["result_tolerance"]), p1
    assert p1[g["exact_unmoved_index"]] == 1.0
    # First-step moments: m = (1-b1) gbar, v = (1-b2) gbar^2 (openlearn L11.3, section
    # '3. Worked example by hand'), with gbar the shard means the page prints.
    means = np.concatenate([np.array(x) for x in g["shard_means"]])
    assert np.allclose(m1, 0.1 * means, rtol=1e-14, atol=1e-17), m1
    assert np.allclose(v1, 0.001 * means * means, rtol=1e-13, atol=1e-19), v1
    # The same example in fp32 and mixed precision lands on the page's values too.
    for mode in (MODE_F32, MODE_MIXED):
        if mode == MODE_F32:
            pp = param.astype(np.float32)
            gg = [x.astype(np.float32) for x in grads]
        else:
            pp = _bf16_bits(param.astype(np.float32))
            gg = [_bf16_bits(x.astype(np.float32)) for x in grads]
        mst, m0, v0 = O.init_states(mode, pp)
        p1, mst1, _, _ = O.zero_step(mode, pp, gg, mst, m0, v0, g["t"], g["lr"])
        w = mst1 if mode == MODE_MIXED else p1
        tol = 1e-6  # the first step moves by lr whatever the gradient's rounding
        assert np.all(np.abs(w.astype(np.float64) - res) <= tol), (mode, w)
        assert w[g["exact_unmoved_index"]] == 1.0


def pin_p1_worked_example(O):
    """openlearn L11.3, section '3. Worked example by hand'."""
    g = _golden("p1_worked_example.json")
    n, N = g["n"], g["n_workers"]
    sizes = [b - a for a, b in (O.split_bounds(n, N, r) for r in range(N))]
    assert sizes == g["chunk_sizes"], sizes
    w = np.array(g["param"], np.float64)
    grads = [w - r for r in range(N)]
    _, m0, v0 = O.init_states(MODE_F64, w)
    p1, _, m1, v1 = O.zero_step(MODE_F64, w, grads, None, m0, v0, g["t"], g["lr"],
                                wd=g["weight_decay"])
    res = np.array(g["result"], np.float64)
    assert np.all(np.abs(p1 - res) <= g["result_tolerance"]), p1
    gbar = w - 1.5
    # entries with a negative mean gradient move up, the others down
    assert np.all(np.sign(p1 - w) == -np.sign(gbar))
    assert np.allclose(m1, 0.1 * gbar, rtol=1e-14), m1
    assert np.allclose(v1, 0.001 * gbar * gbar, rtol=1e-13), v1


def pin_p5_tensor_shards(O):
    """ZeRO One, section 'Sharding Parameters': 291 tensors on 4 ranks."""
    g = _golden("p5_tensor_shards.json")
    got = [list(O.split_bounds(g["n"], g["n_workers"], r)) for r in range(g["n_workers"])]
    assert got == g["bounds"], got


# ---------------------------------------------------------------------------
# Shard bounds: numpy's own array_split, brute force
# ---------------------------------------------------------------------------
def pin_split_bounds_numpy(O, n_max=300, N_max=70):
    for n in range(0, n_max + 1, 7 if n_max > 100 else 1):
        for N in range(1, N_max + 1):
            parts = np.array_split(np.arange(n), N)
            start = 0
            for r, part in enumerate(parts):
                a, b = O.split_bounds(n, N, r)
                assert (a, b) == (start, start + len(part)), (n, N, r, a, b)
                if len(part):
                    assert a == part[0] and b == part[-1] + 1
                start += len(part)
            for i in range(n):
                r = O.owner(n, N, i)
                a, b = O.split_bounds(n, N, r)
                assert a <= i < b, (n, N, i, r)


# ---------------------------------------------------------------------------
# Closed forms of the step
# ---------------------------------------------------------------------------
def _rand_case(rng, n, N, scale=1.0):
    w = rng.standard_normal(n)
    grads = [scale * rng.standard_normal(n) for _ in range(N)]
    return w, grads


def pin_first_step_closed_form(O):
    """At t = 1 bias correction gives mh = gbar and sqrt(vh) = |gbar| exactly in real
    arithmetic, so w1 = w0 - lr*gbar/(|gbar| + eps), m1 = (1-b1) gbar, v1 = (1-b2) gbar^2
    (openlearn L11.3, section '3. Worked example by hand'), for any inputs."""
    rng = np.random.default_rng(11)
    for n, N, lr, scale in ((1000, 4, 1e-2, 1.0), (257, 3, 0.5, 1e-3), (64, 64, 3e-4, 1e-3)):
        w, grads = _rand_case(rng, n, N, scale)
        gbar = np.mean(np.stack(grads), axis=0)
        _, m0, v0 = O.init_states(MODE_F64, w)
        for b1, b2 in ((0.9, 0.999), (0.8, 0.95)):
            p1, _, m1, v1 = O.zero_step(MODE_F64, w, grads, None, m0, v0, 1, lr, b1, b2, 1e-8)
            ref = w - lr * gbar / (np.abs(gbar) + 1e-8)
            assert np.all(np.abs(p1 - ref) <= 1e-14 * (np.abs(w) + lr)), np.max(np.abs(p1 - ref))
            assert np.allclose(m1, (1 - b1) * gbar, rtol=1e-13, atol=0)
            assert np.allclose(v1, (1 - b2) * gbar * gbar, rtol=1e-13, atol=0)


def pin_constant_gradient_trajectory(O):
    """With the same mean gradient c every step, m_t = (1-b1^t) c and v_t = (1-b2^t) c^2,
    so mh = c and vh = c^2 exactly in real arithmetic and
    w_t = w0 - t*lr*c/(|c| + eps)."""
    rng = np.random.default_rng(12)
    n, N, T, lr, b1, b2, eps = 513, 4, 30, 1e-3, 0.9, 0.95, 1e-8
    w0 = rng.standard_normal(n)
    c = 1e-3 * rng.standard_normal(n)
    # worker 0 holds N*c (exact: N is a power of two), the rest hold 0, so the mean is c
    grads = [N * c] + [np.zeros(n) for _ in range(N - 1)]
    _, m, v = O.init_states(MODE_F64, w0)
    w = w0
    for t in range(1, T + 1):
        w, _, m, v = O.zero_step(MODE_F64, w, grads, None, m, v, t, lr, b1, b2, eps)
        assert np.allclose(m, (1 - b1 ** t) * c, rtol=1e-12, atol=0), t
        assert np.allclose(v, (1 - b2 ** t) * c * c, rtol=1e-12, atol=0), t
    ref = w0 - T * lr * c / (np.abs(c) + eps)
    assert np.all(np.abs(w - ref) <= 1e-12 * (np.abs(w0) + T * lr)), np.max(np.abs(w - ref))


# ---------------------------------------------------------------------------
# Special case N = 1: plain Adam / AdamW, checked against torch.optim on CPU fp64
# ---------------------------------------------------------------------------
def _torch_trajectory(w0, grad_seq, lr, b1, b2, eps, wd, adamw, dtype="float64"):
    import torch
    dt = getattr(torch, dtype)
    p = torch.nn.Parameter(torch.tensor(w0, dtype=dt))
    cls = torch.optim.AdamW if adamw else torch.optim.Adam
    kw = dict(lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    opt = cls([p], **kw)
    for g in grad_seq:
        p.grad = torch.tensor(g, dtype=dt)
        opt.step()
    st = opt.state[p]
    return (p.detach().numpy().copy(), st["exp_avg"].numpy().copy(),
            st["exp_avg_sq"].numpy().copy())


def pin_torch_adam_single_worker(O):
    rng = np.random.default_rng(13)
    n, T = 300, 8
    for lr, b1, b2, wd in ((1e-2, 0.9, 0.999, 0.0), (3e-4, 0.9, 0.95, 0.1), (0.05, 0.7, 0.9, 0.3)):
        w0 = rng.standard_normal(n)
        gseq = [rng.standard_normal(n) for _ in range(T)]
        tw, tm, tv = _torch_trajectory(w0, gseq, lr, b1, b2, 1e-8, wd, adamw=wd > 0)
        _, m, v = O.init_states(MODE_F64, w0)
        w = w0
        for t, g in enumerate(gseq, 1):
            w, _, m, v = O.zero_step(MODE_F64, w, [g], None, m, v, t, lr, b1, b2, 1e-8, wd)
        assert np.allclose(w, tw, rtol=1e-12, atol=1e-14), np.max(np.abs(w - tw))
        assert np.allclose(m, tm, rtol=1e-12, atol=1e-16)
        assert np.allclose(v, tv, rtol=1e-12, atol=1e-18)


def pin_torch_adam_mean_of_workers(O):
    """Several workers: the step equals torch Adam driven by the mean gradient. The
    workers' gradients are chosen so that their sum is exact in fp64 (integers times a
    power of two), so the mean itself carries no rounding."""
    rng = np.random.default_rng(14)
    n, N, T, lr = 200, 4, 5, 1e-2
    w0 = rng.standard_normal(n)
    gseqs = [[rng.integers(-512, 512, n).astype(np.float64) / 1024.0 for _ in range(N)]
             for _ in range(T)]
    means = [sum(gs) / N for gs in gseqs]  # exact: integer numerators
    tw, tm, tv = _torch_trajectory(w0, means, lr, 0.9, 0.999, 1e-8, 0.0, adamw=False)
    _, m, v = O.init_states(MODE_F64, w0)
    w = w0
    for t, gs in enumerate(gseqs, 1):
        w, _, m, v = O.zero_step(MODE_F64, w, gs, None, m, v, t, lr)
    assert np.allclose(w, tw, rtol=1e-12, atol=1e-14)
    assert np.allclose(m, tm, rtol=1e-12, atol=1e-16)
    assert np.allclose(v, tv, rtol=1e-12, atol=1e-18)


def pin_decay_mask(O):
    """Elements whose flag is set follow AdamW, the others plain Adam (torch, N = 1)."""
    rng = np.random.default_rng(15)
    n, T, lr, wd = 400, 6, 1e-2, 0.1
    w0 = rng.standard_normal(n)
    gseq = [rng.standard_normal(n) for _ in range(T)]
    flags = (rng.random(n) < 0.5).astype(np.uint8)
    aw, _, _ = _torch_trajectory(w0, gseq, lr, 0.9, 0.95, 1e-8, wd, adamw=True)
    pw, _, _ = _torch_trajectory(w0, gseq, lr, 0.9, 0.95, 1e-8, 0.0, adamw=False)
    ref = np.where(flags != 0, aw, pw)
    _, m, v = O.init_states(MODE_F64, w0)
    w = w0
    for t, g in enumerate(gseq, 1):
        w, _, m, v = O.zero_step(MODE_F64, w, [g], None, m, v, t, lr, 0.9, 0.95, 1e-8, wd,
                                 decay=flags)
    assert np.allclose(w, ref, rtol=1e-12, atol=1e-14), np.max(np.abs(w - ref))


def pin_torch_adam_f32(O):
    """fp32 mode against torch fp32 Adam/AdamW (different operation order, so a
    tolerance: a few fp32 roundings per step)."""
    rng = np.random.default_rng(16)
    n, T = 500, 10
    for lr, wd in ((3e-4, 0.0), (3e-4, 0.1)):
        w0 = (0.02 * rng.standard_normal(n)).astype(np.float32)
        gseq = [(1e-3 * rng.standard_normal(n)).astype(np.float32) for _ in range(T)]
        tw, tm, tv = _torch_trajectory(w0, gseq, lr, 0.9, 0.95, 1e-8, wd, adamw=wd > 0,
                                       dtype="float32")
        _, m, v = O.init_states(MODE_F32, w0)
        w = w0
        for t, g in enumerate(gseq, 1):
            w, _, m, v = O.zero_step(MODE_F32, w, [g], None, m, v, t, lr, 0.9, 0.95, 1e-8, wd)
        assert np.all(np.abs(w - tw) <= 1e-6 * np.maximum(1, np.abs(tw))), np.max(np.abs(w - tw))
        # m cancels towards zero: a few fp32 ulps of its largest terms, not of itself
        assert np.allclose(m, tm, rtol=1e-5, atol=2e-6 * np.abs(tm).max())
        assert np.allclose(v, tv, rtol=1e-5, atol=1e-16)


# ---------------------------------------------------------------------------
# Invariants the pages state
# ---------------------------------------------------------------------------
def _case_for_mode(rng, mode, n, N):
    if mode == MODE_F64:
        w = rng.standard_normal(n)
        grads = [rng.standard_normal(n) for _ in range(N)]
        return w, grads
    w = (0.02 * rng.standard_normal(n)).astype(np.float32)
    grads = [(1e-3 * rng.standard_normal(n)).astype(np.float32) for _ in range(N)]
    if mode == MODE_MIXED:
        return _bf16_bits(w), [_bf16_bits(g) for g in grads]
    if mode == MODE_MIXED_F16:
        return _fp16_bits(w), [_fp16_bits(g) for g in grads]
    return w, grads


def pin_sharded_equals_shard_free(O):
    """ZeRO-Sharded Adam Step, 'Requirements': the sharded result equals ordinary Adam
    over the whole vector driven by the averaged gradient, bit for bit, for every
    shard count."""
    rng = np.random.default_rng(17)
    for mode in (MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16):
        for n, N in ((1, 1), (3, 5), (10, 4), (1031, 7), (4096, 64), (777, 2)):
            w, _ = _case_for_mode(rng, mode, n, 1)
            mst, m, v = O.init_states(mode, w)
            ws, ms, vs, msts = w, m, v, mst
            wf, mf, vf, mstf = w, m, v, mst
            flags = (rng.random(n) < 0.7).astype(np.uint8)
            for t in (1, 2, 3):
                _, grads = _case_for_mode(rng, mode, n, N)
                ws, msts, ms, vs = O.zero_step(mode, ws, grads, msts, ms, vs, t, 1e-3, 0.9, 0.95,
                                               1e-8, 0.1, decay=flags)
                wf, mstf, mf, vf = O.full_step(mode, wf, grads, mstf, mf, vf, t, 1e-3, 0.9, 0.95,
                                               1e-8, 0.1, decay=flags)
                assert np.array_equal(ws.view(np.uint8), wf.view(np.uint8)), (mode, n, N, t)
                assert np.array_equal(ms, mf) and np.array_equal(vs, vf), (mode, n, N, t)
                if mode in MIXED_MODES:
                    assert np.array_equal(msts, mstf)


def pin_rank_share_equals_shard(O):
    """One rank's share (chunk gradients, shard-local state) equals the full sharded
    step restricted to that rank's shard (openlearn L11.3, section '2. Principles',
    stage 2), and leaves every other element of the gathered vector as it was."""
    rng = np.random.default_rng(18)
    for mode in (MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16):
        for n, N in ((1031, 8), (10, 4), (3, 5)):
            w, grads = _case_for_mode(rng, mode, n, N)
            mst, m, v = O.init_states(mode, w)
            # one step to get non-zero state, then compare the next one
            w, mst, m, v = O.zero_step(mode, w, grads, mst, m, v, 1, 1e-3)
            _, grads = _case_for_mode(rng, mode, n, N)
            flags = (rng.random(n) < 0.5).astype(np.uint8)
            full_w, full_mst, full_m, full_v = O.zero_step(mode, w, grads, mst, m, v, 2, 1e-3,
                                                           0.9, 0.95, 1e-8, 0.1, decay=flags)
            for r in range(N):
                a, b = O.split_bounds(n, N, r)
                master_r = (mst if mode in MIXED_MODES else w)[a:b]
                if mode not in MIXED_MODES:
                    master_r = master_r.astype(w.dtype)
                chunks = [g[a:b] for g in grads]
                pw, pm, rm, rv = O.rank_step(mode, N, r, w, chunks, master_r, m[a:b], v[a:b], 2,
                                             1e-3, 0.9, 0.95, 1e-8, 0.1, decay=flags)
                assert np.array_equal(pw[a:b].view(np.uint8), full_w[a:b].view(np.uint8))
                assert np.array_equal(pw[:a].view(np.uint8), w[:a].view(np.uint8))
                assert np.array_equal(pw[b:].view(np.uint8), w[b:].view(np.uint8))
                assert np.array_equal(rm, full_m[a:b]) and np.array_equal(rv, full_v[a:b])
                full_master = full_mst if mode in MIXED_MODES else full_w
                assert np.array_equal(pm.view(np.uint8),
                                      full_master[a:b].astype(pm.dtype).view(np.uint8))


# ---------------------------------------------------------------------------
# Mixed precision
# ---------------------------------------------------------------------------
def pin_bf16_rounding(O):
    """The oracle's bf16 rounding equals torch's round-to-nearest-even conversion."""
    rng = np.random.default_rng(19)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (1e-3 * rng.standard_normal(20000)).astype(np.float32),
        np.ldexp(rng.standard_normal(5000), rng.integers(-140, 127, 5000)).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45,
                  1.1754942e-38], np.float32),
    ])
    # exact ties: bf16 value plus half a bf16 ulp, both mantissa parities
    base = rng.integers(0x0080, 0x7F00, 4000).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    near = np.concatenate([(base | 0x7FFF).view(np.float32), (base | 0x8001).view(np.float32)])
    x = np.concatenate([x, ties, -ties, near])
    got = O.bf16_round(x)
    ref = _bf16_bits(x)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]
    nan = O.bf16_round(np.array([np.nan], np.float32))
    assert nan[0] == 0x7FC0


def pin_mixed_precision(O):
    """Mixed mode: the master starts as the exact widening of the bf16 parameters, the
    gathered output is the bf16 rounding of the master, and the master follows the fp64
    trajectory within fp32 rounding."""
    rng = np.random.default_rng(20)
    n, N, T = 2048, 8, 5
    p_bits = _bf16_bits((0.02 * rng.standard_normal(n)).astype(np.float32))
    mst, m, v = O.init_states(MODE_MIXED, p_bits)
    assert np.array_equal(mst, _widen(p_bits)) and not m.any() and not v.any()
    w64 = _widen(p_bits).astype(np.float64)
    _, m64, v64 = O.init_states(MODE_F64, w64)
    p = p_bits
    for t in range(1, T + 1):
        gb = [_bf16_bits((1e-3 * rng.standard_normal(n)).astype(np.float32)) for _ in range(N)]
        p, mst, m, v = O.zero_step(MODE_MIXED, p, gb, mst, m, v, t, 1e-4, 0.9, 0.95, 1e-8)
        w64, _, m64, v64 = O.zero_step(MODE_F64, w64, [_widen(g).astype(np.float64) for g in gb],
                                       None, m64, v64, t, 1e-4, 0.9, 0.95, 1e-8)
        assert np.array_equal(p, _bf16_bits(mst))
        assert np.all(np.abs(mst - w64) <= 1e-6 * np.maximum(1, np.abs(w64)))
        assert np.allclose(m, m64, rtol=1e-5, atol=2e-6 * np.abs(m64).max())


def pin_fp16_rounding(O):
    """The oracle's fp16 rounding equals numpy's round-to-nearest-even float32 ->
    float16 conversion (gradual underflow, overflow to infinity), and its widening
    equals numpy's float16 -> float32 for all 65536 bit patterns."""
    rng = np.random.default_rng(21)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (1e-3 * rng.standard_normal(20000)).astype(np.float32),
        np.ldexp(rng.standard_normal(8000), rng.integers(-30, 18, 8000)).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.0, 65520.0, 65536.0, -65520.0,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
                  1e-45, 3.4028235e38], np.float32),
    ])
    # exact ties: a finite fp16 value plus half its ulp, both parities, normal and subnormal
    h = rng.integers(1, 0x7BFF, 6000).astype(np.uint16)
    lo = _fp16_widen(h).astype(np.float64)
    hi = _fp16_widen(h + 1).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    x = np.concatenate([x, ties, -ties, np.nextafter(ties, np.float32(0)),
                        np.nextafter(ties, np.float32(np.inf))])
    got = O.fp16_round(x)
    ref = _fp16_bits(x)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]
    assert O.fp16_round(np.array([np.nan], np.float32))[0] == 0x7E00
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    wid = O.fp16_widen(allh)
    refw = _fp16_widen(allh)
    nan = np.isnan(refw)
    assert np.array_equal(np.isnan(wid), nan)
    assert np.array_equal(wid[~nan].view(np.uint32), refw[~nan].view(np.uint32))
    assert np.array_equal(O.fp16_round(wid[~nan]), allh[~nan])  # exact round trip


def pin_mixed_f16_precision(O):
    """fp16 mixed mode: the master starts as the exact widening of the fp16
    parameters, the gathered output is the fp16 rounding of the master, and the
    master follows the fp64 trajectory within fp32 rounding."""
    rng = np.random.default_rng(22)
    n, N, T = 2048, 8, 5
    p_bits = _fp16_bits((0.02 * rng.standard_normal(n)).astype(np.float32))
    mst, m, v = O.init_states(MODE_MIXED_F16, p_bits)
    assert np.array_equal(mst, _fp16_widen(p_bits)) and not m.any() and not v.any()
    w64 = _fp16_widen(p_bits).astype(np.float64)
    _, m64, v64 = O.init_states(MODE_F64, w64)
    p = p_bits
    for t in range(1, T + 1):
        gb = [_fp16_bits((1e-3 * rng.standard_normal(n)).astype(np.float32)) for _ in range(N)]
        p, mst, m, v = O.zero_step(MODE_MIXED_F16, p, gb, mst, m, v, t, 1e-4, 0.9, 0.95, 1e-8)
        w64, _, m64, v64 = O.zero_step(MODE_F64, w64,
                                       [_fp16_widen(g).astype(np.float64) for g in gb],
                                       None, m64, v64, t, 1e-4, 0.9, 0.95, 1e-8)
        assert np.array_equal(p, _fp16_bits(mst))
        assert np.all(np.abs(mst - w64) <= 1e-6 * np.maximum(1, np.abs(w64)))
        assert np.allclose(m, m64, rtol=1e-5, atol=2e-6 * np.abs(m64).max())


# ---------------------------------------------------------------------------
# Memory
# ---------------------------------------------------------------------------
WIDTHS = {"mixed": (2, 2, 12), "f32": (4, 4, 8), "f64": (8, 8, 16)}


def pin_memory_byte_table(O):
    """openlearn L11.3, section '3. Worked example by hand': the byte table."""
    g = _golden("p1_worked_example.json")
    n, N, bw = g["n"], g["n_workers"], g["bytes_per_value"]
    table = g["byte_table"]
    for stage in (1, 2, 3):
        for r in (0, 3):
            got = O.memory_bytes(n, N, r, stage, bw, bw, 2 * bw, convention=1)
            exp = table[f"stage{stage}_rank{r}"]
            assert {k: got[k] for k in exp} == exp, (stage, r, got)
    got = O.memory_bytes(n, N, 0, 0, bw, bw, 2 * bw, convention=1)
    assert {k: got[k] for k in table["one_process"]} == table["one_process"]
    assert got["total"] == g["one_process_total"]
    assert O.memory_bytes(n, N, 0, 3, bw, bw, 2 * bw, convention=1)["total"] == g["stage3_rank0_total"]


def pin_memory_closed_forms(O):
    """The closed forms and their numeric instances on the pages."""
    cases = _golden("memory_closed_forms.json")["cases"]
    P, G, K = WIDTHS["mixed"]
    # 16 bytes per parameter, and the per-stage formulas, with N dividing n exactly
    for N in (1, 2, 4, 8, 64):
        n = 64 * 1000
        for stage, (lead, tail) in {1: (4, 12), 2: (2, 14), 3: (0, 16)}.items():
            got = O.memory_bytes(n, N, 0, stage, P, G, K)["total"]
            assert got * N == (lead * N + tail) * n, (N, stage, got)
        assert O.memory_bytes(n, N, 0, 0, P, G, K)["total"] == 16 * n
    assert O.memory_bytes(1000, 1, 0, 0, *WIDTHS["f32"])["total"] == 16 * 1000
    # 8B model on 8 GPUs: about 120 / 41 / 28 / 15 GiB
    c8 = cases[3]
    gib = [O.memory_bytes(c8["psi"], c8["n_gpus"], 0, s, P, G, K)["total"] / 2 ** 30
           for s in range(4)]
    assert [float(f"{x:.2g}") for x in gib] == c8["gib_rounded"], gib
    assert O.memory_bytes(c8["psi"], 64, 0, 3, P, G, K)["total"] / 2 ** 30 < c8["zero3_64_gpus_gib_below"]
    # 175B on 64 GPUs under ZeRO-3: 43.75 GB
    c = cases[4]
    assert O.memory_bytes(c["psi"], c["n_gpus"], 0, 3, P, G, K)["total"] == int(c["gb"] * 1e9)
    # 20B on 8 GPUs with 10 GB of activations: 330 / 120 / 85 / 50 GB
    c = cases[5]
    need = [O.memory_bytes(c["psi"], c["n_gpus"], 0, s, P, G, K)["total"] / 1e9 + c["activations_gb"]
            for s in range(4)]
    assert need == c["gb"], need
    assert [x < 80 for x in need] == c["fits_80gb"]
    # the decision rule: the smallest stage that fits is ZeRO-3 here
    assert O.min_stage(c["psi"], c["n_gpus"], P, G, K, int(c["activations_gb"] * 1e9),
                       int(80e9)) == c["fits_80gb"].index(True)
    assert O.min_stage(c["psi"], c["n_gpus"], P, G, K, int(c["activations_gb"] * 1e9),
                       int(331e9)) == 0  # 330 GB < 331 GB: plain data parallelism fits
    assert O.min_stage(c["psi"], c["n_gpus"], P, G, K, int(c["activations_gb"] * 1e9),
                       int(50e9)) == -1  # 50 GB is not below 50 GB: nothing fits
    # 320M parameters in fp32: 5.12 GB
    c = cases[6]
    assert O.memory_bytes(c["psi"], 1, 0, 0, *WIDTHS["f32"])["total"] == int(c["gb"] * 1e9)
    # Adam's share of the memory
    c = cases[7]
    d = O.memory_bytes(10 ** 6, 1, 0, 0, *WIDTHS["f32"])
    assert d["optimizer"] / d["total"] == c["fraction_f32"]
    d = O.memory_bytes(10 ** 6, 1, 0, 0, *WIDTHS["mixed"])
    lo, hi = c["fraction_mixed_range"]
    assert lo <= d["optimizer"] / d["total"] <= hi


# ---------------------------------------------------------------------------
# Materialised mean gradient and global-norm clipping
# ---------------------------------------------------------------------------
def pin_mean_grad_worked_example(O):
    """ZeRO-Sharded Adam Step, section 'The step': the reduce-scatter gives worker 0
    [0.3, 0.2, 0.4] and worker 1 [0.0, 2.0]; their squared norms sum to 4.29."""
    g = _golden("p2_worked_example.json")
    grads = [np.array(x, np.float64) for x in g["grads"]]
    mean, ss = O.mean_grad(MODE_F64, g["n"], g["n_workers"], grads)
    printed = np.concatenate([np.array(x) for x in g["shard_means"]])
    assert np.allclose(mean, printed, rtol=0, atol=1e-15), mean
    assert abs(ss - float(np.sum(printed ** 2))) <= 1e-14
    for r, part in enumerate(g["shard_means"]):
        chunks = [x[slice(*O.split_bounds(g["n"], g["n_workers"], r))] for x in grads]
        mr, sr = O.mean_grad(MODE_F64, g["n"], g["n_workers"], chunks, rank=r)
        assert np.allclose(mr, part, rtol=0, atol=1e-15)
        assert abs(sr - float(np.sum(np.array(part) ** 2))) <= 1e-14


def pin_mean_grad_sumsq_exact_sum(O):
    """The squared norm of fp32 mean gradients: every square is exact in double, so
    math.fsum (a correctly rounded sum) gives the exact sum rounded once; the
    oracle's plain double sum is within (n-1) * 2^-53 of it relatively."""
    import math
    rng = np.random.default_rng(21)
    for n, N in ((100_003, 8), (4099, 3), (1000, 64)):
        grads = [(1e-3 * rng.standard_normal(n)).astype(np.float32) for _ in range(N)]
        mean, ss = O.mean_grad(MODE_F32, n, N, grads)
        exact = math.fsum(float(x) * float(x) for x in mean.astype(np.float64))
        assert abs(ss - exact) <= (n - 1) * 2.0 ** -53 * exact, (ss, exact)
        # rank mode: each shard's partial, and their rank-order sum is the total
        total = 0.0
        for r in range(N):
            a, b = O.split_bounds(n, N, r)
            mr, sr = O.mean_grad(MODE_F32, n, N, [x[a:b] for x in grads], rank=r)
            assert np.array_equal(mr, mean[a:b])
            total = total + sr
        assert total == ss


def pin_step_from_mean_equals_step(O):
    """Materialising the reduce-scatter output does not change the arithmetic: the
    step from the mean gradient, unclipped or clipped with a threshold the norm does
    not reach, equals the fused step bit for bit, in every mode."""
    rng = np.random.default_rng(22)
    for mode in (MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16):
        n, N = 3001, 5
        w, grads = _case_for_mode(rng, mode, n, N)
        mst, m, v = O.init_states(mode, w)
        flags = (rng.random(n) < 0.5).astype(np.uint8)
        ref = O.zero_step(mode, w, grads, mst, m, v, 3, 1e-3, 0.9, 0.95, 1e-8, 0.1, decay=flags)
        mean, ss = O.mean_grad(mode, n, N, grads)
        for clip in (None, 10.0 * math.sqrt(ss) + 1.0):
            got = O.step_mean(mode, N, w, mean, mst, m, v, 3, 1e-3, 0.9, 0.95, 1e-8, 0.1,
                              decay=flags, clip_sumsq=None if clip is None else ss,
                              max_norm=clip or 0.0)
            for x, y in zip(got, ref):
                if x is not None:
                    assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (mode, clip)


def pin_clipping_vs_torch(O):
    """One worker: clipping by the global norm then Adam/AdamW equals
    torch.nn.utils.clip_grad_norm_ followed by torch.optim (fp64), with the
    threshold crossed on some steps and not on others."""
    import torch
    rng = np.random.default_rng(23)
    n, T = 257, 8
    for wd, adamw in ((0.0, False), (0.1, True)):
        w0 = rng.standard_normal(n)
        gseq = [rng.standard_normal(n) * (3.0 if t % 2 else 0.2) for t in range(T)]
        max_norm = 5.0
        p = torch.nn.Parameter(torch.tensor(w0))
        cls = torch.optim.AdamW if adamw else torch.optim.Adam
        opt = cls([p], lr=1e-2, betas=(0.9, 0.95), eps=1e-8, weight_decay=wd, foreach=False)
        _, m, v = O.init_states(MODE_F64, w0)
        w = w0
        clipped = 0
        for t, g in enumerate(gseq, 1):
            p.grad = torch.tensor(g)
            tn = float(torch.nn.utils.clip_grad_norm_([p], max_norm, foreach=False))
            opt.step()
            mean, ss = O.mean_grad(MODE_F64, n, 1, [g])
            assert abs(math.sqrt(ss) - tn) <= 1e-13 * tn
            clipped += tn > max_norm
            w, _, m, v = O.step_mean(MODE_F64, 1, w, mean, None, m, v, t, 1e-2, 0.9, 0.95, 1e-8,
                                     wd, clip_sumsq=ss, max_norm=max_norm)
            tw = p.detach().numpy()
            assert np.allclose(w, tw, rtol=1e-12, atol=1e-14), (t, np.max(np.abs(w - tw)))
        assert 0 < clipped < T


def pin_clipping_nonfinite_vs_torch(O):
    """A non-finite global norm, as torch.nn.utils.clip_grad_norm_ handles it
    (fp64, one worker): a NaN entry makes the norm NaN, and its clamp at 1 lets
    the NaN factor through, so every gradient entry becomes NaN; an infinite
    entry gives a zero factor, so the finite entries become 0 and the infinite
    one NaN. The oracle's clipped mean must match torch's clipped gradient
    entry for entry (NaN where torch has NaN), and so must one Adam step."""
    import torch
    n = 7
    w0 = np.linspace(-1.0, 1.0, n)
    for bad in (float("nan"), float("inf")):
        g = np.linspace(0.1, 0.7, n)
        g[3] = bad
        p = torch.nn.Parameter(torch.tensor(w0))
        p.grad = torch.tensor(g)
        torch.nn.utils.clip_grad_norm_([p], 1.0, foreach=False)
        tg = p.grad.numpy()
        mean, ss = O.mean_grad(MODE_F64, n, 1, [g])
        coef = O.clip_factor(ss, 1.0)
        ours = mean * coef
        assert np.array_equal(np.isnan(ours), np.isnan(tg)), (bad, ours, tg)
        fin = ~np.isnan(tg)
        assert np.array_equal(ours[fin], tg[fin]), (bad, ours, tg)
        opt = torch.optim.Adam([p], lr=1e-2, betas=(0.9, 0.95), eps=1e-8, foreach=False)
        opt.step()
        _, m, v = O.init_states(MODE_F64, w0)
        w, _, _, _ = O.step_mean(MODE_F64, 1, w0, mean, None, m, v, 1, 1e-2, 0.9, 0.95, 1e-8,
                                 clip_sumsq=ss, max_norm=1.0)
        tw = p.detach().numpy()
        assert np.array_equal(np.isnan(w), np.isnan(tw)), (bad, w, tw)
        assert np.allclose(w[~np.isnan(tw)], tw[~np.isnan(tw)], rtol=1e-12, atol=0.0)
    if np.isnan(O.clip_factor(float("nan"), 1.0)) is not np.True_:
        raise AssertionError("a NaN norm must give a NaN factor")


def pin_clipping_closed_form(O):
    """With clipping active at t = 1, m1 = (1-b1) * c * gbar with
    c = max_norm / (|gbar| + 1e-6), so |m1| / (1-b1) = max_norm |gbar| / (|gbar| + 1e-6)."""
    rng = np.random.default_rng(24)
    n, N = 5000, 4
    w, grads = _rand_case(rng, n, N)
    mean, ss = O.mean_grad(MODE_F64, n, N, grads)
    norm = math.sqrt(ss)
    for max_norm in (0.5, 0.01 * norm):
        _, m0, v0 = O.init_states(MODE_F64, w)
        _, _, m1, _ = O.step_mean(MODE_F64, N, w, mean, None, m0, v0, 1, 1e-3, 0.9, 0.999, 1e-8,
                                  clip_sumsq=ss, max_norm=max_norm)
        got = np.linalg.norm(m1) / 0.1
        assert abs(got - max_norm * norm / (norm + 1e-6)) <= 1e-12 * max_norm
    assert O.clip_factor(4.0, 100.0) == 1.0


# ---------------------------------------------------------------------------
# Momentum SGD
# ---------------------------------------------------------------------------
SGD_VARIANTS = [  # (momentum, dampening, nesterov, weight decay)
    (0.9, 0.0, False, 0.0),
    (0.9, 0.1, False, 0.01),
    (0.8, 0.0, True, 0.05),
    (0.0, 0.0, False, 0.1),
]


def pin_sgd_vs_torch(O):
    """One worker, fp64: the oracle's momentum SGD equals torch.optim.SGD."""
    import torch
    rng = np.random.default_rng(25)
    n, T, lr = 300, 6, 0.05
    for mom, damp, nest, wd in SGD_VARIANTS:
        w0 = rng.standard_normal(n)
        gseq = [rng.standard_normal(n) for _ in range(T)]
        p = torch.nn.Parameter(torch.tensor(w0))
        opt = torch.optim.SGD([p], lr=lr, momentum=mom, dampening=damp, nesterov=nest,
                              weight_decay=wd, foreach=False)
        w, buf = w0, np.zeros(n)
        for t, g in enumerate(gseq, 1):
            p.grad = torch.tensor(g)
            opt.step()
            w, _, buf = O.sgd_step(MODE_F64, w, [g], None, buf, t, lr, wd, mom, damp, nest)
            assert np.allclose(w, p.detach().numpy(), rtol=1e-12, atol=1e-14), (mom, damp, nest, t)
            if mom:
                tb = opt.state[p]["momentum_buffer"].numpy()
                assert np.allclose(buf, tb, rtol=1e-12, atol=1e-14)


def pin_sgd_constant_gradient(O):
    """Momentum mu, no dampening, the same mean gradient c every step:
    buf_t = c (1 - mu^t) / (1 - mu), w_t = w0 - lr c sum_{s<=t} (1 - mu^s) / (1 - mu)."""
    rng = np.random.default_rng(26)
    n, N, T, lr, mu = 400, 4, 12, 0.01, 0.9
    w0 = rng.standard_normal(n)
    c = rng.standard_normal(n)
    grads = [N * c] + [np.zeros(n)] * (N - 1)
    w, buf = w0, np.zeros(n)
    acc = 0.0
    for t in range(1, T + 1):
        w, _, buf = O.sgd_step(MODE_F64, w, grads, None, buf, t, lr, 0.0, mu)
        assert np.allclose(buf, c * (1 - mu ** t) / (1 - mu), rtol=1e-12, atol=1e-15)
        acc += (1 - mu ** t) / (1 - mu)
    assert np.allclose(w, w0 - lr * c * acc, rtol=1e-12, atol=1e-13)


def pin_sgd_sharded_equals_shard_free_and_rank_share(O):
    rng = np.random.default_rng(27)
    for mode in (MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16):
        n, N = 2051, 7
        w, _ = _case_for_mode(rng, mode, n, 1)
        mst, buf, _ = O.init_states(mode, w)
        flags = (rng.random(n) < 0.5).astype(np.uint8)
        ws, bs, ms_ = w, buf, mst
        for t in (1, 2, 3):
            _, grads = _case_for_mode(rng, mode, n, N)
            args = (t, 0.01, 0.05, 0.9, 0.1, False, flags)
            a_p, a_m, a_b = O.sgd_step(mode, ws, grads, ms_, bs, *args, form="sharded")
            f_p, f_m, f_b = O.sgd_step(mode, ws, grads, ms_, bs, *args, form="full")
            assert np.array_equal(a_p.view(np.uint8), f_p.view(np.uint8)) and np.array_equal(a_b, f_b)
            for r in (0, N // 2, N - 1):
                lo, hi = O.split_bounds(n, N, r)
                master_r = (ms_ if mode in MIXED_MODES else ws)[lo:hi].astype(bs.dtype)
                r_p, r_m, r_b = O.sgd_step(mode, ws, [g[lo:hi] for g in grads], master_r,
                                           bs[lo:hi], *args, form="rank", N=N, rank=r)
                assert np.array_equal(r_p[lo:hi].view(np.uint8), a_p[lo:hi].view(np.uint8))
                assert np.array_equal(r_p[:lo].view(np.uint8), ws[:lo].view(np.uint8))
                assert np.array_equal(r_p[hi:].view(np.uint8), ws[hi:].view(np.uint8))
                assert np.array_equal(r_b, a_b[lo:hi])
            ws, ms_, bs = a_p, a_m, a_b


ALL_PINS = [
    pin_p2_worked_example,
    pin_p1_worked_example,
    pin_p5_tensor_shards,
    pin_split_bounds_numpy,
    pin_first_step_closed_form,
    pin_constant_gradient_trajectory,
    pin_torch_adam_single_worker,
    pin_torch_adam_mean_of_workers,
    pin_decay_mask,
    pin_torch_adam_f32,
    pin_sharded_equals_shard_free,
    pin_rank_share_equals_shard,
    pin_bf16_rounding,
    pin_mixed_precision,
    pin_fp16_rounding,
    pin_mixed_f16_precision,
    pin_memory_byte_table,
    pin_memory_closed_forms,
    pin_mean_grad_worked_example,
    pin_mean_grad_sumsq_exact_sum,
    pin_step_from_mean_equals_step,
    pin_clipping_vs_torch,
    pin_clipping_closed_form,
    pin_clipping_nonfinite_vs_torch,
    pin_sgd_vs_torch,
    pin_sgd_constant_gradient,
    pin_sgd_sharded_equals_shard_free_and_rank_share,
]
