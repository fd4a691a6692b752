"""Seeded random configurations of the step against the oracle.

Each case draws a mode (fp64, fp32, bf16 or fp16 mixed precision), an optimizer (Adam/AdamW, or momentum SGD with or
without dampening and Nesterov), n from 1 to ~3e5, N up to 256 (N > n included),
full or rank mode, no decay / decay everywhere / a random per-element mask, a
call path (one zero_step; buckets of zero_step_range in a random order;
buckets of zero_step_range_dev with the step scalars in device memory; all
buckets in one zero_step_buckets call; the
materialised mean then zero_step_mean; or zero_step_clipped with a threshold
never reached, whose factor is exactly 1) and 1-3 steps, and compares every
element with the oracle's unclipped step at the parity bar of
oracle/compare.py. Inputs are drawn on the host with numpy and uploaded."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import zero_sharded_optimizer_amd as z  # noqa: E402
from oracle import MIXED_MODES, MODE_F32, MODE_F64, MODE_MIXED, MODE_MIXED_F16  # noqa: E402
from gpu_cases import compare_bits  # noqa: E402
from gpu_cases import host, say  # noqa: E402

_PDT = {MODE_F64: np.float64, MODE_F32: np.float32}
_SDT = {MODE_F64: torch.float64, MODE_F32: torch.float32, MODE_MIXED: torch.float32,
        MODE_MIXED_F16: torch.float32}


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _fp16_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _half_bits(mode, x):
    return _bf16_bits(x) if mode == MODE_MIXED else _fp16_bits(x)


def _host_values(rng, mode, size, scale):
    x = scale * rng.standard_normal(size)
    return _half_bits(mode, x) if mode in MIXED_MODES else x.astype(_PDT[mode])


def _device(x, mode):
    if mode in MIXED_MODES:
        dt = torch.bfloat16 if mode == MODE_MIXED else torch.float16
        return torch.from_numpy(x.view(np.int16).copy()).view(dt).cuda()
    return torch.from_numpy(x.copy()).cuda()


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    c = dict(seed=seed)
    c["mode"] = int(rng.choice([MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16]))
    c["sgd"] = bool(rng.random() < 0.35)
    c["n"] = int(np.exp(rng.uniform(0.0, np.log(300_000))))
    c["N"] = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 16, 33, 64, 100, 256]))
    c["rank"] = -1 if rng.random() < 0.6 else int(rng.integers(0, c["N"]))
    c["decay"] = str(rng.choice(["none", "all", "mask"]))
    c["wd"] = 0.0 if c["decay"] == "none" else float(rng.choice([0.01, 0.1]))
    c["path"] = str(rng.choice(["step", "range", "range_dev", "split", "clip1", "native"]))
    if c["path"] == "clip1" and c["rank"] >= 0:
        c["path"] = "split"  # a clipped step needs every shard: full mode only
    c["steps"] = int(rng.integers(1, 4))
    mom = float(rng.choice([0.0, 0.9]))
    damp = float(rng.choice([0.0, 0.1])) if mom else 0.0
    c["sgd_args"] = (mom, damp, bool(mom and not damp and rng.random() < 0.5))
    return c, rng


def _buckets(rng, L):
    """Random bucket edges over [0, L) with every begin a multiple of 8, in a
    random order."""
    edges = [0]
    while edges[-1] < L:
        edges.append(min(L, edges[-1] + 8 * int(rng.integers(1, max(2, L // 8 // 3 + 2)))))
    pairs = list(zip(edges[:-1], edges[1:]))
    rng.shuffle(pairs)
    return pairs


@pytest.mark.parametrize("seed", range(400))
def test_random_configuration_matches_the_oracle(oracle, seed):
    c, rng = _draw(seed)
    mode, n, N, rank = c["mode"], c["n"], c["N"], c["rank"]
    say(f"[case] fuzz {c}")
    a, b = oracle.split_bounds(n, N, rank) if rank >= 0 else (0, n)
    L = b - a
    lr = 1e-2 if c["sgd"] else 1e-3
    mom, damp, nest = c["sgd_args"]
    flags = rng.random(n) < 0.5 if c["decay"] == "mask" else None
    hp = z.HParams(n=n, n_workers=N, mode=mode, lr=lr, beta1=0.9, beta2=0.99, eps=1e-8,
                   weight_decay=c["wd"], rank=rank,
                   wd_mask=z.wd_mask_from_flags(flags) if flags is not None else None,
                   optimizer=z.ZERO_OPT_SGD if c["sgd"] else z.ZERO_OPT_ADAM,
                   momentum=mom, dampening=damp, nesterov=nest)
    dec = None if flags is None else flags.astype(np.uint8)
    sdt = _SDT[mode]
    npsdt = np.float64 if mode == MODE_F64 else np.float32
    p_h = _host_values(rng, mode, n, 0.5)
    need_master = mode in MIXED_MODES or rank >= 0
    if rank >= 0:  # the rank's master, and its slot as the rounding of it
        mst_h = (0.5 * rng.standard_normal(L)).astype(npsdt)
        p_h[a:b] = _half_bits(mode, mst_h) if mode in MIXED_MODES else mst_h.astype(_PDT[mode])
    param = _device(p_h, mode)
    st = z.States(torch.empty(L, dtype=sdt, device="cuda") if need_master else None,
                  torch.empty(L, dtype=sdt, device="cuda"),
                  None if c["sgd"] else torch.empty(L, dtype=sdt, device="cuda"))
    if L:
        z.zero_init_states(hp, param, st)
    if rank >= 0:
        st.master.copy_(torch.from_numpy(mst_h))
        o_mst, o_m, o_v = mst_h.copy(), np.zeros(L, npsdt), np.zeros(L, npsdt)
    else:
        o_mst, o_m, o_v = oracle.init_states(mode, p_h)
    o_p = p_h.copy()
    scal = torch.empty(z.STEP_SCALARS_BYTES, dtype=torch.uint8, device="cuda")
    for t in range(1, c["steps"] + 1):
        g_h = [_host_values(rng, mode, L if rank >= 0 else n, 1e-2) for _ in range(N)]
        grads = [_device(g, mode) for g in g_h]
        if c["path"] == "step":
            z.zero_step(hp, param, grads, st, t)
        elif c["path"] == "split":  # materialised mean, then the step from it
            mean = torch.empty(L, dtype=sdt, device="cuda")
            z.zero_mean_grad(hp, grads, mean)
            z.zero_step_mean(hp, param, mean, st, t)
        elif c["path"] == "native":  # every bucket in one zero_step_buckets call
            z.zero_step_buckets(hp, param, grads, st, t, _buckets(rng, L))
        elif c["path"] == "clip1":  # clipped, threshold never reached: factor exactly 1
            ws = torch.empty(z.zero_step_clipped_workspace_bytes(hp), dtype=torch.uint8,
                             device="cuda")
            z.zero_step_clipped(hp, param, grads, st, t, 1e30, ws)
        else:
            if c["path"] == "range_dev":
                scal.copy_(torch.from_numpy(z.zero_step_scalars(hp, t)))
            for lo, hi in _buckets(rng, L):
                if c["path"] == "range":
                    z.zero_step_range(hp, param, grads, st, t, lo, hi)
                else:
                    z.zero_step_range_dev(hp, param, grads, st, scal, lo, hi)
        if c["sgd"]:
            o_p, o_mst, o_m = oracle.sgd_step(mode, o_p, g_h, o_mst, o_m, t, lr, c["wd"], mom,
                                              damp, nest, dec, form="rank" if rank >= 0 else
                                              "sharded", N=N, rank=rank)
        elif rank >= 0:
            o_p, o_mst, o_m, o_v = oracle.rank_step(mode, N, rank, o_p, g_h, o_mst, o_m, o_v, t,
                                                    lr, 0.9, 0.99, 1e-8, c["wd"], dec)
        else:
            o_p, o_mst, o_m, o_v = oracle.zero_step(mode, o_p, g_h, o_mst, o_m, o_v, t, lr, 0.9,
                                                    0.99, 1e-8, c["wd"], dec)
    torch.cuda.synchronize()
    pk = {MODE_F64: "exact", MODE_F32: "f32", MODE_MIXED: "bf16", MODE_MIXED_F16: "fp16"}[mode]
    sk = "exact" if mode == MODE_F64 else "f32"
    compare_bits("param", host(param), o_p, pk)
    if not c["sgd"] or mom:
        compare_bits("m", host(st.m), o_m, sk)
    if not c["sgd"]:
        compare_bits("v", host(st.v), o_v, sk)
    if need_master:
        compare_bits("master", host(st.master), o_mst, sk)
