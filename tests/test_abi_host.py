"""The C-ABI library on the host, no GPU: it loads, exports every function
include/zero_adam.h declares, and its host logic (shard bounds, memory model,
argument validation) is right. No call here reaches a kernel launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import zero_sharded_optimizer_amd as z
from zero_sharded_optimizer_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 32  # fake, 16-byte aligned "device" addresses: never dereferenced here


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(zero_\w+)\s*\(", txt, flags=re.M)
    return names


def test_library_exports_every_declared_function():
    lib = _abi.load()
    names = declared_functions()
    assert set(names) >= set(_abi.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_header_is_plain_c():
    """Plain C declarations: no torch or C++ types outside the comments."""
    txt = open(os.path.join(ROOT, "include", "zero_adam.h")).read()
    code = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    assert 'extern "C"' in code
    for word in ("torch", "at::", "c10", "std::", "Tensor", "hipStream_t"):
        assert word not in code, word


# -- shard bounds -------------------------------------------------------------
def test_shard_bounds_match_numpy_array_split():
    for n in list(range(0, 60)) + [1_048_579, 124_439_808, 8_000_000_000]:
        for N in (1, 2, 3, 4, 5, 7, 8, 64, 70):
            if n > 10 ** 7:
                sizes = [n // N + (1 if r < n % N else 0) for r in range(N)]
            else:
                sizes = [len(p) for p in np.array_split(np.arange(n), N)]
            start = 0
            for r in range(N):
                assert z.zero_shard_bounds(n, N, r) == (start, start + sizes[r])
                start += sizes[r]


def test_shard_bounds_match_oracle(oracle):
    rng = np.random.default_rng(1)
    for _ in range(2000):
        n = int(rng.integers(0, 10 ** 12))
        N = int(rng.integers(1, 300))
        r = int(rng.integers(0, N))
        assert z.zero_shard_bounds(n, N, r) == oracle.split_bounds(n, N, r)


@pytest.mark.parametrize("args", [(-1, 2, 0), (10, 0, 0), (10, 2, 2), (10, 2, -1)])
def test_shard_bounds_rejects(args):
    with pytest.raises(z.ZeroError) as e:
        z.zero_shard_bounds(*args)
    assert e.value.status == z.ZERO_EINVAL and e.value.message


# -- memory model -------------------------------------------------------------
WIDTH = {z.ZERO_MODE_MIXED_BF16: (2, 2, 12), z.ZERO_MODE_MIXED_F16: (2, 2, 12),
         z.ZERO_MODE_F32: (4, 4, 8), z.ZERO_MODE_F64: (8, 8, 16)}


def test_memory_bytes_agrees_with_oracle(oracle):
    rng = np.random.default_rng(2)
    for _ in range(3000):
        n = int(rng.integers(1, 10 ** 11))
        N = int(rng.integers(1, 100))
        r = int(rng.integers(0, N))
        stage = int(rng.integers(0, 4))
        mode = int(rng.integers(0, 4))
        P, G, K = WIDTH[mode]
        got = z.zero_memory_bytes(n, N, r, stage, mode, 0)
        assert got == oracle.memory_bytes(n, N, r, stage, P, G, K, 0)
        if mode not in (z.ZERO_MODE_MIXED_BF16, z.ZERO_MODE_MIXED_F16):
            got = z.zero_memory_bytes(n, N, r, stage, mode, 1)
            assert got == oracle.memory_bytes(n, N, r, stage, P, G, K, 1)


def test_memory_bytes_byte_table():
    """openlearn L11.3, section '3. Worked example by hand': the byte table."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "p1_worked_example.json")))
    for key, exp in g["byte_table"].items():
        if key == "one_process":
            got = z.zero_memory_bytes(10, 4, 0, 0, z.ZERO_MODE_F64, 1)
        else:
            stage, rank = int(key[5]), int(key[-1])
            got = z.zero_memory_bytes(10, 4, rank, stage, z.ZERO_MODE_F64, 1)
        assert {k: got[k] for k in exp} == exp, key


def test_memory_bytes_closed_forms():
    """Data Parallelism & ZeRO, section 'ZeRO, stage by stage': 16, 4 + 12/N,
    2 + 14/N, 16/N bytes per parameter; an 8B model on 8 GPUs at 120/41/28/15 GiB."""
    n = 8_000_000_000
    gib = [z.zero_memory_bytes(n, 8, 0, s, z.ZERO_MODE_MIXED_BF16)["total"] / 2 ** 30 for s in range(4)]
    assert [float(f"{x:.2g}") for x in gib] == [120, 41, 28, 15]
    for N in (2, 8, 64):
        m = 64_000
        for s, (lead, tail) in {1: (4, 12), 2: (2, 14), 3: (0, 16)}.items():
            assert z.zero_memory_bytes(m, N, N - 1, s, z.ZERO_MODE_MIXED_BF16)["total"] * N == (lead * N + tail) * m
    assert z.zero_memory_bytes(320_000_000, 1, 0, 0, z.ZERO_MODE_F32)["total"] == 5_120_000_000


@pytest.mark.parametrize("args,status", [
    ((0, 4, 0, 1, 0, 0), z.ZERO_EINVAL),      # no parameters
    ((10, 0, 0, 1, 0, 0), z.ZERO_EINVAL),
    ((10, 4, 4, 1, 0, 0), z.ZERO_EINVAL),
    ((10, 4, 0, 4, 0, 0), z.ZERO_EINVAL),     # stage 4
    ((10, 4, 0, -1, 0, 0), z.ZERO_EINVAL),
    ((10, 4, 0, 1, 4, 0), z.ZERO_EINVAL),     # unknown mode
    ((10, 4, 0, 1, 0, 2), z.ZERO_EINVAL),     # unknown convention
    ((10, 4, 0, 1, 2, 1), z.ZERO_EUNSUPPORTED),
    ((10, 4, 0, 1, 3, 1), z.ZERO_EUNSUPPORTED),
])
def test_memory_bytes_rejects(args, status):
    with pytest.raises(z.ZeroError) as e:
        z.zero_memory_bytes(*args)
    assert e.value.status == status


# -- step / init validation (rejected before any HIP call) ---------------------
def _hp(**kw):
    d = dict(n=1000, n_workers=4, rank=-1, mode=z.ZERO_MODE_F32, optimizer=0, lr=1e-3, beta1=0.9,
             beta2=0.999, eps=1e-8, weight_decay=0.0, wd_mask=None, momentum=0.0, dampening=0.0,
             nesterov=0, reserved=0)
    d.update(kw)
    return _abi.zero_hparams(**d)


def _call_step(hp, param=A, grads=None, master=None, m=A + (1 << 24), v=A + (2 << 24), t=1):
    lib = _abi.load()
    if grads is None:
        grads = [A + ((3 + k) << 24) for k in range(hp.n_workers)]
    arr = (C.c_void_p * max(1, len(grads)))(*grads)
    st = _abi.zero_states(master=master, m=m, v=v)
    rc = lib.zero_step(C.byref(hp), param, arr, C.byref(st), t, None)
    return rc, lib.zero_last_error().decode()


BAD_STEPS = {
    "no parameters": (dict(n=0), {}),
    "zero workers": (dict(n_workers=0), {}),
    "too many workers": (dict(n_workers=257), {}),
    "rank too large": (dict(rank=4), {}),
    "rank below -1": (dict(rank=-2), {}),
    "unknown mode": (dict(mode=7), {}),
    "reserved": (dict(reserved=1), {}),
    "t = 0": ({}, dict(t=0)),
    "beta1 = 1": (dict(beta1=1.0), {}),
    "beta2 < 0": (dict(beta2=-0.1), {}),
    "eps = 0": (dict(eps=0.0), {}),
    "lr nan": (dict(lr=float("nan")), {}),
    "lr inf": (dict(lr=float("inf")), {}),
    "wd < 0": (dict(weight_decay=-0.1), {}),
    "wd nan": (dict(weight_decay=float("nan")), {}),
    "mask misaligned": (dict(weight_decay=0.1, wd_mask=A + 2), {}),
    "null param": ({}, dict(param=None)),
    "misaligned param": ({}, dict(param=A + 4)),
    "null m": ({}, dict(m=None)),
    "misaligned v": ({}, dict(v=A + (2 << 24) + 8)),
    "master in full fp32": ({}, dict(master=A + (9 << 24))),
    "master missing in mixed": (dict(mode=z.ZERO_MODE_MIXED_BF16), {}),
    "master missing in rank mode": (dict(rank=1), {}),
    "misaligned master": (dict(mode=z.ZERO_MODE_MIXED_BF16), dict(master=A + (9 << 24) + 4)),
    "null grad": ({}, dict(grads=[A + (3 << 24), None, A + (5 << 24), A + (6 << 24)])),
    "misaligned grad": ({}, dict(grads=[A + (3 << 24), A + (4 << 24) + 4, A + (5 << 24), A + (6 << 24)])),
    "m overlaps v": ({}, dict(v=A + (1 << 24) + 16)),
    "param overlaps m": ({}, dict(m=A + 16)),
    "grad overlaps m": ({}, dict(grads=[A + (1 << 24), A + (4 << 24), A + (5 << 24), A + (6 << 24)])),
    "mask overlaps v": (dict(weight_decay=0.1, wd_mask=A + (2 << 24)), {}),
    "unknown optimizer": (dict(optimizer=2), {}),
    "sgd momentum < 0": (dict(optimizer=1, momentum=-0.5), {}),
    "sgd momentum nan": (dict(optimizer=1, momentum=float("nan")), {}),
    "sgd dampening > 1": (dict(optimizer=1, momentum=0.9, dampening=1.5), {}),
    "sgd nesterov with dampening": (dict(optimizer=1, momentum=0.9, dampening=0.1, nesterov=1), {}),
    "sgd nesterov without momentum": (dict(optimizer=1, nesterov=1), {}),
    "sgd nesterov = 2": (dict(optimizer=1, momentum=0.9, nesterov=2), {}),
    "sgd null m": (dict(optimizer=1, momentum=0.9), dict(m=None)),
}


@pytest.mark.parametrize("case", sorted(BAD_STEPS))
def test_step_rejects(case):
    hpkw, callkw = BAD_STEPS[case]
    rc, msg = _call_step(_hp(**hpkw), **callkw)
    assert rc == z.ZERO_EINVAL, (case, rc, msg)
    assert msg, case


def test_step_null_hparams_and_states():
    lib = _abi.load()
    arr = (C.c_void_p * 1)(A)
    assert lib.zero_step(None, A, arr, None, 1, None) == z.ZERO_EINVAL
    hp = _hp(n_workers=1)
    assert lib.zero_step(C.byref(hp), A, arr, None, 1, None) == z.ZERO_EINVAL
    assert lib.zero_step(C.byref(hp), A, None, C.byref(_abi.zero_states(None, A, A + 4096)), 1,
                         None) == z.ZERO_EINVAL


def test_grads_may_alias_each_other_but_checks_still_run():
    # identical gradient buffers for every worker are read-only and allowed; the call
    # is still rejected here, for t = 0, so nothing is launched
    hp = _hp()
    rc, msg = _call_step(hp, grads=[A + (3 << 24)] * 4, t=0)
    assert rc == z.ZERO_EINVAL and "t must be" in msg


def test_empty_rank_shard_is_a_no_op():
    """N > n gives trailing empty shards (numpy semantics); a rank-mode call for
    an empty shard is valid and enqueues nothing."""
    hp = _hp(n=3, n_workers=5, rank=4)
    rc, msg = _call_step(hp, master=A + (9 << 24))
    assert rc == z.ZERO_OK, msg
    lib = _abi.load()
    st = _abi.zero_states(master=A + (9 << 24), m=A + (1 << 24), v=A + (2 << 24))
    assert lib.zero_init_states(C.byref(hp), A, C.byref(st), None) == z.ZERO_OK


@pytest.mark.parametrize("case", ["no parameters", "master in full fp32", "m overlaps v",
                                  "master missing in mixed", "unknown mode"])
def test_init_rejects(case):
    hpkw, callkw = BAD_STEPS[case]
    lib = _abi.load()
    hp = _hp(**hpkw)
    st = _abi.zero_states(master=callkw.get("master"), m=callkw.get("m", A + (1 << 24)),
                          v=callkw.get("v", A + (2 << 24)))
    assert lib.zero_init_states(C.byref(hp), A, C.byref(st), None) == z.ZERO_EINVAL
    assert lib.zero_last_error()


# -- binding ------------------------------------------------------------------
def test_binding_rejects_host_tensors():
    import torch
    hp = z.HParams(n=8, n_workers=1, mode=z.ZERO_MODE_F32, lr=1e-3, beta1=0.9, beta2=0.999,
                   eps=1e-8)
    x = torch.zeros(8)
    st = z.States(None, torch.zeros(8), torch.zeros(8))
    with pytest.raises(ValueError, match="GPU tensor"):
        z.zero_step(hp, x, [torch.zeros(8)], st, 1, stream=0)


def test_wd_mask_packing():
    flags = np.zeros(70, bool)
    flags[[0, 5, 31, 32, 63, 69]] = True
    w = z.wd_mask_from_flags(flags, device="cpu").numpy().view(np.uint32)
    assert w.size == 3
    bits = [(int(w[i // 32]) >> (i % 32)) & 1 for i in range(70)]
    assert bits == flags.astype(int).tolist()


# -- mean gradient and clipping entry points (host validation) -----------------
def test_workspace_sizes_follow_the_launch_geometry():
    lib = _abi.load()
    out = C.c_size_t()
    hp = _hp(n=1_000_000, n_workers=8, mode=z.ZERO_MODE_F32)
    assert lib.zero_mean_grad_workspace_bytes(C.byref(hp), C.byref(out)) == z.ZERO_OK
    mean_ws = out.value
    assert mean_ws % 8 == 0 and mean_ws >= 8
    assert lib.zero_step_clipped_workspace_bytes(C.byref(hp), C.byref(out)) == z.ZERO_OK
    assert out.value >= 4 * 1_000_000 + mean_ws + 8
    hp0 = _hp(n=3, n_workers=5, rank=4)  # empty shard: one partial
    assert lib.zero_mean_grad_workspace_bytes(C.byref(hp0), C.byref(out)) == z.ZERO_OK
    assert out.value == 8


def test_clipped_step_rejects_rank_mode_and_bad_max_norm():
    lib = _abi.load()
    st = _abi.zero_states(master=A + (9 << 24), m=A + (1 << 24), v=A + (2 << 24))
    arr = (C.c_void_p * 4)(*[A + ((3 + k) << 24) for k in range(4)])
    hp = _hp(rank=1)
    rc = lib.zero_step_clipped(C.byref(hp), A, arr, C.byref(st), 1, 1.0, None, A + (20 << 24),
                               1 << 24, None)
    assert rc == z.ZERO_EUNSUPPORTED
    st = _abi.zero_states(master=None, m=A + (1 << 24), v=A + (2 << 24))
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        rc = lib.zero_step_clipped(C.byref(_hp()), A, arr, C.byref(st), 1, bad, None,
                                   A + (20 << 24), 1 << 24, None)
        assert rc == z.ZERO_EINVAL, bad
    # workspace too small, misaligned, overlapping m
    for ws, nb in ((A + (20 << 24), 16), (A + (20 << 24) + 4, 1 << 24), (A + (1 << 24), 1 << 24)):
        rc = lib.zero_step_clipped(C.byref(_hp()), A, arr, C.byref(st), 1, 1.0, None, ws, nb, None)
        assert rc == z.ZERO_EINVAL, (ws, nb)


def test_step_mean_and_mean_grad_reject():
    lib = _abi.load()
    st = _abi.zero_states(master=None, m=A + (1 << 24), v=A + (2 << 24))
    hp = _hp()
    # clipping with a bad max_norm; mean overlapping m
    assert lib.zero_step_mean(C.byref(hp), A, A + (5 << 24), C.byref(st), 1, A + (7 << 24), 0.0,
                              None) == z.ZERO_EINVAL
    assert lib.zero_step_mean(C.byref(hp), A, A + (1 << 24), C.byref(st), 1, None, 0.0,
                              None) == z.ZERO_EINVAL
    assert lib.zero_step_mean(C.byref(hp), A, A + (5 << 24) + 8, C.byref(st), 1, None, 0.0,
                              None) == z.ZERO_EINVAL
    arr = (C.c_void_p * 4)(*[A + ((3 + k) << 24) for k in range(4)])
    # mean_out misaligned / overlapping a gradient; workspace missing for a norm
    assert lib.zero_mean_grad(C.byref(hp), arr, A + 4, None, None, 0, None) == z.ZERO_EINVAL
    assert lib.zero_mean_grad(C.byref(hp), arr, A + (3 << 24), None, None, 0, None) == z.ZERO_EINVAL
    assert lib.zero_mean_grad(C.byref(hp), arr, A, A + (9 << 24), None, 0, None) == z.ZERO_EINVAL
    assert lib.zero_mean_grad(C.byref(_hp(n=0)), arr, A, None, None, 0, None) == z.ZERO_EINVAL


def test_step_range_rejects_bad_ranges():
    lib = _abi.load()
    st = _abi.zero_states(master=None, m=A + (1 << 24), v=A + (2 << 24))
    arr = (C.c_void_p * 4)(*[A + ((3 + k) << 24) for k in range(4)])
    hp = _hp()
    for begin, end in ((-8, 10), (16, 8), (0, 1001), (4, 100)):
        rc = lib.zero_step_range(C.byref(hp), A, arr, C.byref(st), 1, begin, end, None)
        assert rc == z.ZERO_EINVAL, (begin, end)
    # an empty range is valid and launches nothing
    assert lib.zero_step_range(C.byref(hp), A, arr, C.byref(st), 1, 8, 8, None) == z.ZERO_OK


def test_sgd_ignores_adam_fields_and_allows_null_v():
    """SGD ignores beta1/beta2/eps (here invalid for Adam) and may leave v NULL;
    the call is rejected only for t = 0 here, so nothing is launched."""
    hp = _hp(optimizer=1, momentum=0.9, beta1=5.0, beta2=-1.0, eps=0.0)
    rc, msg = _call_step(hp, v=None, t=0)
    assert rc == z.ZERO_EINVAL and "t must be" in msg


def test_step_scalars_fill_matches_the_step_formula():
    """zero_step_scalars_fill forms 1 - beta^t in double exactly as the step
    does (C pow, as Python's float ** is), and rejects what zero_step rejects."""
    hp = _hp()
    for t in (1, 2, 3, 10, 1000, 10 ** 6):
        b = z.zero_step_scalars(z.HParams(n=1000, n_workers=4, mode=1, lr=1e-3, beta1=0.9,
                                          beta2=0.999, eps=1e-8), t)
        bias1, bias2 = b[:16].view(np.float64)
        assert bias1 == 1.0 - 0.9 ** t and bias2 == 1.0 - 0.999 ** t
        assert int(b[16:].view(np.int64)[0]) == t
    lib = _abi.load()
    out = _abi.zero_step_scalars()
    assert lib.zero_step_scalars_fill(C.byref(hp), 0, C.byref(out)) == z.ZERO_EINVAL
    assert lib.zero_step_scalars_fill(C.byref(hp), 1, None) == z.ZERO_EINVAL
    assert lib.zero_step_scalars_fill(C.byref(_hp(beta1=1.0)), 1, C.byref(out)) == z.ZERO_EINVAL
    assert lib.zero_step_scalars_fill(None, 1, C.byref(out)) == z.ZERO_EINVAL
    assert C.sizeof(_abi.zero_step_scalars) == 24 == z.STEP_SCALARS_BYTES


def test_step_range_dev_rejects_before_any_launch():
    lib = _abi.load()
    st = _abi.zero_states(master=None, m=A + (1 << 24), v=A + (2 << 24))
    arr = (C.c_void_p * 4)(*[A + ((3 + k) << 24) for k in range(4)])
    hp = _hp()
    ok_scal = A + (40 << 24)
    for scal, begin, end in ((None, 0, 8), (ok_scal + 4, 0, 8),  # NULL, misaligned scalars
                             (A + (1 << 24) + 8, 0, 8),           # scalars inside m
                             (ok_scal, -8, 10), (ok_scal, 4, 100)):  # bad ranges
        rc = lib.zero_step_range_dev(C.byref(hp), A, arr, C.byref(st), scal, begin, end, None)
        assert rc == z.ZERO_EINVAL, (scal, begin, end)
    # an empty range is valid and launches nothing
    assert lib.zero_step_range_dev(C.byref(hp), A, arr, C.byref(st), ok_scal, 8, 8,
                                   None) == z.ZERO_OK


def test_input_recipe_shard_matches_numpy_array_split():
    """The input generator's rank chunks are numpy's array_split sections."""
    from dataclasses import replace
    from zero_sharded_optimizer_amd import synth
    base = synth.WORKLOADS["mixed-rank0-of-8B-n8"]
    for n in (1, 5, 17, 100, 1001):
        for N in (1, 3, 8, 64):
            sizes = [s.size for s in np.array_split(np.arange(n), N)]
            starts = np.cumsum([0] + sizes[:-1])
            for r in range(N):
                a, b = replace(base, n=n, n_workers=N, rank=r).shard
                assert (a, b) == (starts[r], starts[r] + sizes[r])


def test_min_stage_agrees_with_the_oracle_and_the_page(oracle):
    """The smallest ZeRO stage that fits: the page's 20B example (8 GPUs, 10 GB of
    activations, 80 GB each) needs ZeRO-3; random cases agree with the oracle."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "memory_closed_forms.json")))
    c = g["cases"][5]
    act = int(c["activations_gb"] * 1e9)
    assert z.zero_min_stage(c["psi"], c["n_gpus"], z.ZERO_MODE_MIXED_BF16, act, int(80e9)) == 3
    assert z.zero_min_stage(c["psi"], c["n_gpus"], z.ZERO_MODE_MIXED_F16, act, int(120e9)) == 2
    rng = np.random.default_rng(5)
    for _ in range(2000):
        n = int(rng.integers(1, 10 ** 12))
        N = int(rng.integers(1, 129))
        mode = int(rng.integers(0, 4))
        act = int(rng.integers(0, 10 ** 11))
        avail = int(rng.integers(0, 4 * 10 ** 12))
        P, G, K = WIDTH[mode]
        assert z.zero_min_stage(n, N, mode, act, avail) == oracle.min_stage(n, N, P, G, K, act, avail)
    for bad in ((0, 8, 1, 0, 10), (10, 0, 1, 0, 10), (10, 8, 9, 0, 10), (10, 8, 1, -1, 10)):
        with pytest.raises(z.ZeroError):
            z.zero_min_stage(*bad)


def test_n_above_two_to_the_56_is_rejected():
    """Every byte count formed from n stays inside int64: n > 2^56 is rejected by
    the step, the memory model and the stage choice."""
    rc, msg = _call_step(_hp(n=(1 << 56) + 1))
    assert rc == z.ZERO_EINVAL and "2^56" in msg
    with pytest.raises(z.ZeroError):
        z.zero_memory_bytes((1 << 56) + 1, 4, 0, 1, z.ZERO_MODE_F64)
    with pytest.raises(z.ZeroError):
        z.zero_min_stage((1 << 56) + 1, 4, z.ZERO_MODE_F64, 0, 1 << 62)
    d = z.zero_memory_bytes(1 << 56, 1, 0, 0, z.ZERO_MODE_F64)
    assert d["total"] == 32 << 56


def test_min_stage_does_not_overflow_with_huge_activations():
    """activation_bytes near INT64_MAX: no stage fits (no wrap-around)."""
    big = (1 << 63) - 1
    assert z.zero_min_stage(1000, 4, z.ZERO_MODE_F32, big, big) == -1
    assert z.zero_min_stage(1000, 4, z.ZERO_MODE_F32, big - 100, big) == -1
    assert z.zero_min_stage(1000, 4, z.ZERO_MODE_F32, 0, big) == 0


def test_step_mean_rejects_a_clip_norm_inside_an_output():
    """The clipped step reads the squared norm while it writes its outputs: a
    norm inside m (or the parameter) is rejected before any launch."""
    lib = _abi.load()
    st = _abi.zero_states(master=None, m=A + (1 << 24), v=A + (2 << 24))
    hp = _hp()
    mean = A + (5 << 24)
    for norm in (A + (1 << 24) + 64, A + 8, A + (2 << 24)):
        rc = lib.zero_step_mean(C.byref(hp), A, mean, C.byref(st), 1, norm, 1.0, None)
        assert rc == z.ZERO_EINVAL and "clip_sumsq overlaps" in lib.zero_last_error().decode()


def test_binding_rejects_tensors_on_several_devices():
    """The binding checks that one call's tensors share a device, and that a
    torch stream given for the call is on that device (fake tensors: only the
    device attribute is read)."""
    class Fake:
        def __init__(self, dev):
            self.device = dev

        def data_ptr(self):
            return A

    class FakeStream:
        def __init__(self, dev):
            self.device = dev

    z._same_device(None, Fake("cuda:0"), [Fake("cuda:0"), None, A],
                   z.States(None, Fake("cuda:0"), None))
    with pytest.raises(ValueError, match="one device"):
        z._same_device(None, Fake("cuda:0"), [Fake("cuda:1")])
    with pytest.raises(ValueError, match="one device"):
        z._same_device(None, Fake("cuda:0"), z.States(Fake("cuda:1"), Fake("cuda:0"), None))
    with pytest.raises(ValueError, match="stream is on"):
        z._same_device(FakeStream("cuda:1"), Fake("cuda:0"))
    z._same_device(FakeStream("cuda:0"), Fake("cuda:0"))
    z._same_device(FakeStream("cuda:3"))  # no tensors: nothing to compare


def test_one_hip_runtime_when_the_library_loads_first():
    """A host-only call that loads libzero.so before the program has touched
    torch still leaves one HIP runtime in the process: torch's (the binding
    loads torch first). Checked in a fresh interpreter, without a GPU."""
    import subprocess
    import sys
    code = ("import zero_sharded_optimizer_amd as z\n"
            "z.zero_memory_bytes(10, 2, 0, 1, z.ZERO_MODE_F32)\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "print('\\n'.join(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    paths = [p for p in out.stdout.splitlines() if p.strip()]
    import torch
    torch_dir = os.path.realpath(os.path.dirname(torch.__file__))
    assert len(paths) == 1, paths
    assert os.path.realpath(paths[0]).startswith(torch_dir), paths


def test_every_call_raises_without_the_library():
    """No CPU fallback: with libzero.so absent, a host-only call and a step both
    raise, naming the missing file (fresh interpreter, library path redirected)."""
    import subprocess
    import sys
    code = ("import zero_sharded_optimizer_amd as z\n"
            "from zero_sharded_optimizer_amd import _abi\n"
            "_abi.LIB_PATH = '/nonexistent/libzero.so'\n"
            "for call in (lambda: z.zero_shard_bounds(10, 2, 0),\n"
            "             lambda: z.zero_memory_bytes(10, 2, 0, 1, 1),\n"
            "             lambda: z.zero_step(z.HParams(n=8, n_workers=1, mode=1, lr=1e-3,\n"
            "                                           beta1=0.9, beta2=0.999, eps=1e-8),\n"
            "                                 1 << 32, [2 << 32], z.States(None, 3 << 32, 4 << 32),\n"
            "                                 1, stream=0)):\n"
            "    try:\n"
            "        call()\n"
            "    except RuntimeError as e:\n"
            "        assert 'libzero.so is missing' in str(e), e\n"
            "    else:\n"
            "        raise SystemExit('a call ran without the library')\n"
            "print('all raised')\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "all raised" in out.stdout


def test_step_with_mean_rejects_before_any_launch():
    """zero_step_with_mean validates everything zero_step does, plus its mean
    buffer: NULL, misaligned, or overlapping an output, a gradient or the mask."""
    lib = _abi.load()
    st = _abi.zero_states(master=None, m=A + (1 << 24), v=A + (2 << 24))
    arr = (C.c_void_p * 4)(*[A + ((3 + k) << 24) for k in range(4)])
    hp = _hp()
    for mean in (None, A + (9 << 24) + 4, A + 16, A + (1 << 24) + 64, A + (2 << 24),
                 A + (4 << 24) + 16):
        assert lib.zero_step_with_mean(C.byref(hp), A, arr, C.byref(st), 1, mean,
                                       None) == z.ZERO_EINVAL, mean
        assert lib.zero_last_error()
    hpm = _hp(weight_decay=0.1, wd_mask=A + (9 << 24))
    assert lib.zero_step_with_mean(C.byref(hpm), A, arr, C.byref(st), 1, A + (9 << 24),
                                   None) == z.ZERO_EINVAL
    # the checks of zero_step come first: t = 0 is rejected with a valid mean buffer
    assert lib.zero_step_with_mean(C.byref(hp), A, arr, C.byref(st), 0, A + (9 << 24),
                                   None) == z.ZERO_EINVAL
    assert "t must be" in lib.zero_last_error().decode()
    # an empty rank shard is valid with no mean buffer and launches nothing
    hpe = _hp(n=3, n_workers=5, rank=4)
    ste = _abi.zero_states(master=A + (9 << 24), m=A + (1 << 24), v=A + (2 << 24))
    arr5 = (C.c_void_p * 5)(*[A + ((3 + k) << 24) for k in range(5)])
    assert lib.zero_step_with_mean(C.byref(hpe), A, arr5, C.byref(ste), 1, None,
                                   None) == z.ZERO_OK


def test_noalloc_mean_grad_rejects_ranges_beyond_its_scratch():
    """zero_mean_grad_noalloc's scratch holds 2^21 partial sums: 2^33 elements
    in fp32 (2^30 + 1 in fp64, whose one leftover element block 0 takes). One
    element more is rejected on the host, with a
    message naming the limit, before any device call; without a squared norm
    the scratch is not used and the limit does not apply (rejected here for
    another reason, a misaligned mean, so nothing runs)."""
    lib = _abi.load()
    for mode, limit in ((z.ZERO_MODE_F32, 1 << 33), (z.ZERO_MODE_F64, (1 << 30) + 1),
                        (z.ZERO_MODE_MIXED_BF16, 1 << 33)):
        hp = _hp(n=limit + 1, n_workers=1, mode=mode)
        arr = (C.c_void_p * 1)(1 << 45)
        rc = lib.zero_mean_grad_noalloc(C.byref(hp), arr, 1 << 46, 1 << 47, None)
        assert rc == z.ZERO_EINVAL
        msg = lib.zero_last_error().decode()
        assert "scratch" in msg and str(1 << 21) in msg, msg
        rc = lib.zero_mean_grad_noalloc(C.byref(hp), arr, (1 << 46) + 4, None, None)
        assert rc == z.ZERO_EINVAL and "mean_out" in lib.zero_last_error().decode()
