"""Special values through the fused step: NaN and infinities propagate under IEEE
rules with no special casing, sums that overflow become infinities, subnormal
gradients are kept (no flush to zero), signed zeros survive, and a NaN master
is written back to bf16 as 0x7FC0. The device must agree with the oracle
element by element (NaN on both sides counts as equal)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import zero_sharded_optimizer_amd as z  # noqa: E402
from oracle import MODE_F32, MODE_F64, MODE_MIXED, MODE_MIXED_F16  # noqa: E402
from gpu_cases import compare_bits  # noqa: E402
from gpu_cases import host, say  # noqa: E402


def _specials(dtype):
    fi = np.finfo(dtype)
    return np.array([np.nan, np.inf, -np.inf, fi.max, -fi.max, fi.tiny, -fi.tiny,
                     fi.tiny * fi.eps, -fi.tiny * fi.eps, 0.0, -0.0, 1e-30, 3.0], dtype=dtype)


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _fp16_bits(x):
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("mode", [MODE_F64, MODE_F32, MODE_MIXED, MODE_MIXED_F16])
def test_special_values_match_the_oracle(oracle, mode):
    say(f"[case] special values mode={mode}")
    rng = np.random.default_rng(31)
    n, N = 4099, 4
    fdt = np.float64 if mode == MODE_F64 else np.float32
    sp = _specials(np.float16 if mode == MODE_MIXED_F16 else fdt).astype(fdt)
    grads = [(1e-3 * rng.standard_normal(n)).astype(fdt) for _ in range(N)]
    # plant special values in different workers at different places
    for k in range(N):
        pos = rng.choice(n, 3 * sp.size, replace=False)
        grads[k][pos] = np.tile(sp, 3)[: pos.size]
    w0 = rng.standard_normal(n).astype(fdt)
    w0[:sp.size] = sp  # special parameters too
    if mode in (MODE_MIXED, MODE_MIXED_F16):
        bits = _bf16_bits if mode == MODE_MIXED else _fp16_bits
        p_h = bits(w0)
        g_h = [bits(g) for g in grads]
        tdt = torch.bfloat16 if mode == MODE_MIXED else torch.float16
        p_d = torch.from_numpy(p_h.view(np.int16).copy()).view(tdt).cuda()
        g_d = [torch.from_numpy(g.view(np.int16).copy()).view(tdt).cuda() for g in g_h]
    else:
        p_h, g_h = w0, grads
        p_d = torch.from_numpy(w0.copy()).cuda()
        g_d = [torch.from_numpy(g.copy()).cuda() for g in grads]
    sdt = torch.float64 if mode == MODE_F64 else torch.float32
    mixed = mode in (MODE_MIXED, MODE_MIXED_F16)
    st = z.States(torch.empty(n, dtype=sdt, device="cuda") if mixed else None,
                  torch.empty(n, dtype=sdt, device="cuda"), torch.empty(n, dtype=sdt, device="cuda"))
    hp = z.HParams(n=n, n_workers=N, mode=mode, lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8,
                   weight_decay=0.1)
    z.zero_init_states(hp, p_d, st)
    mst, m, v = oracle.init_states(mode, p_h)
    for t in (1, 2):
        z.zero_step(hp, p_d, g_d, st, t)
        p_h, mst, m, v = oracle.zero_step(mode, p_h, g_h, mst, m, v, t, 1e-2, 0.9, 0.999, 1e-8,
                                          0.1)
    torch.cuda.synchronize()
    kind = "exact" if mode == MODE_F64 else "f32"
    got_p = host(p_d)
    if mixed:
        compare_bits("param", got_p, p_h, "bf16" if mode == MODE_MIXED else "fp16")
        nan_out = got_p[np.isnan(mst)]
        assert nan_out.size > 0 and np.all(nan_out == (0x7FC0 if mode == MODE_MIXED else 0x7E00))
        compare_bits("master", host(st.master), mst, kind)
    else:
        compare_bits("param", got_p, p_h, kind)
    compare_bits("m", host(st.m), m, kind)
    compare_bits("v", host(st.v), v, kind)
    # the special values did reach the state
    assert np.isnan(m).any() and np.isinf(m).any()


def test_subnormal_gradients_are_not_flushed(oracle):
    """fp32 gradients in the subnormal range: the mean and the first moment keep
    them (a flush to zero would leave m exactly 0)."""
    say("[case] subnormal gradients")
    n, N = 1024, 2
    tiny = np.finfo(np.float32).tiny
    g = np.full(n, 8 * tiny * np.finfo(np.float32).eps, dtype=np.float32)  # subnormal
    w = np.ones(n, np.float32)
    hp = z.HParams(n=n, n_workers=N, mode=MODE_F32, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    p_d = torch.from_numpy(w.copy()).cuda()
    st = z.States(None, torch.empty(n, device="cuda"), torch.empty(n, device="cuda"))
    z.zero_init_states(hp, p_d, st)
    z.zero_step(hp, p_d, [torch.from_numpy(g).cuda()] * N, st, 1)
    torch.cuda.synchronize()
    ref = oracle.zero_step(MODE_F32, w, [g, g], None, np.zeros(n, np.float32),
                           np.zeros(n, np.float32), 1, 1e-3, 0.9, 0.999, 1e-8)
    m = host(st.m)
    assert np.all(m > 0) and np.array_equal(m, ref[2])
    assert np.array_equal(host(p_d), ref[0])


@pytest.mark.parametrize("case", ["overflow", "underflow"])
def test_fp16_gathered_copy_overflows_and_underflows(oracle, case):
    """fp16 mixed precision: masters pushed past 65504 give an fp16 infinity in the
    gathered copy while the fp32 master stays finite; masters moved by tiny
    steps near 3e-6 give fp16 subnormals; both as the oracle rounds them."""
    say(f"[case] fp16 {case} of the gathered copy")
    rng = np.random.default_rng(32)
    n, N = 8192, 2
    mag, lr = (65500.0, 16.0) if case == "overflow" else (3e-6, 1e-6)
    w0 = (mag * np.where(rng.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    p_h = _fp16_bits(w0)
    push = -np.sign(w0) if case == "overflow" else np.where(rng.random(n) < 0.5, -1.0, 1.0)
    g_h = [_fp16_bits((push * 1e-2 * rng.random(n)).astype(np.float32)) for _ in range(N)]
    p_d = torch.from_numpy(p_h.view(np.int16).copy()).view(torch.float16).cuda()
    g_d = [torch.from_numpy(g.view(np.int16).copy()).view(torch.float16).cuda() for g in g_h]
    st = z.States(torch.empty(n, device="cuda"), torch.empty(n, device="cuda"),
                  torch.empty(n, device="cuda"))
    hp = z.HParams(n=n, n_workers=N, mode=MODE_MIXED_F16, lr=lr, beta1=0.9, beta2=0.999, eps=1e-8)
    z.zero_init_states(hp, p_d, st)
    mst, m, v = oracle.init_states(MODE_MIXED_F16, p_h)
    for t in (1, 2):
        z.zero_step(hp, p_d, g_d, st, t)
        p_h, mst, m, v = oracle.zero_step(MODE_MIXED_F16, p_h, g_h, mst, m, v, t, lr, 0.9, 0.999,
                                          1e-8)
    torch.cuda.synchronize()
    got = host(p_d)
    compare_bits("param", got, p_h, "fp16")
    compare_bits("master", host(st.master), mst, "f32")
    assert np.all(np.isfinite(mst))
    if case == "overflow":
        assert np.all((p_h & 0x7FFF) == 0x7C00)  # every gathered value is an infinity
    else:
        sub = ((p_h & 0x7C00) == 0) & ((p_h & 0x3FF) != 0)
        assert sub.mean() > 0.9  # fp16 subnormals
    assert np.array_equal(got, p_h)
