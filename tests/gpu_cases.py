"""Drivers shared by the GPU parity tests: run the fused step through the C ABI
and the CPU oracle on the same seeded inputs, and compare with the parity bar
of oracle/compare.py.

The stated bar (fp64 bit-exact; fp32 within 1e-6 * max(1, |ref|); bf16/fp16
within 1 ulp) is the contract's floor. The fused step, its sub-ranges and
buckets, momentum SGD and the mean are computed in the oracle's operation
order with one IEEE rounding per operation and no fused multiply-add, so every
element must also be bit-identical: compare_bits and check_all assert that on
top of the bar (for fp32 m and v the relative bar alone would be loose, since
v ~ 1e-8 sits far below its absolute floor of 1e-6)."""
import numpy as np

import zero_sharded_optimizer_amd as z
from zero_sharded_optimizer_amd import synth
from oracle import MIXED_MODES, MODE_F64, MODE_MIXED
from oracle.compare import compare


def say(msg):
    print(msg, flush=True)


def host(x):
    import torch
    if x.dtype in (torch.bfloat16, torch.float16):
        return x.view(torch.int16).cpu().numpy().view(np.uint16).copy()
    return x.cpu().numpy().copy()


def compare_bits(name, got, ref, kind):
    """compare() at the stated bar, then bit-identity of every element (NaN
    matching NaN); returns the stats."""
    st = compare(name, got, ref, kind)
    assert st["bitexact"] == st["n"] and st["max_ulp"] == 0, (
        f"{name}: {st['n'] - st['bitexact']} of {st['n']} elements not bit-identical "
        f"(max {st['max_ulp']} ulp)")
    return st


def device_bytes(wl):
    """Device memory a sampled full-size run of wl holds at its peak: the N
    gradients, the gathered parameters, master/m/v, and one fp32 draw buffer of
    the generators."""
    import torch
    G = torch.empty(0, dtype=synth.param_dtype(wl)).element_size()
    S = torch.empty(0, dtype=synth.state_dtype(wl)).element_size()
    L = wl.length
    return wl.n_workers * L * G + wl.n * G + 3 * L * S + 4 * L


def need_free(nbytes):
    """Skip (with the reason) when the device has less than nbytes free plus a
    tenth: such a case would fail on memory, and under -x stop every later test."""
    import pytest
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 1.1 * nbytes:
        pytest.skip(f"needs {nbytes / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")


def kinds(wl):
    """(param kind, state kind) of the parity bar for a workload's mode."""
    if wl.mode == MODE_F64:
        return "exact", "exact"
    if wl.mode in MIXED_MODES:
        return ("bf16" if wl.mode == MODE_MIXED else "fp16"), "f32"
    return "f32", "f32"


def hparams(wl, mask=None):
    return z.HParams(n=wl.n, n_workers=wl.n_workers, mode=wl.mode, lr=wl.lr, beta1=wl.beta1,
                     beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay, rank=wl.rank,
                     wd_mask=mask)


def setup(wl):
    """Device buffers for a workload, initialised as the step expects."""
    return setup_with_master(wl)[:4]


def setup_with_master(wl):
    """setup(), plus the rank-mode master chunk as drawn (None in full mode)."""
    import torch
    param, master0 = synth.make_params(wl, "cuda")
    a, b = wl.shard
    L = b - a
    sdt = synth.state_dtype(wl)
    flags = synth.decay_flags(wl)
    mask = z.wd_mask_from_flags(flags) if flags is not None else None
    need_master = wl.mode in MIXED_MODES or wl.rank >= 0
    st = z.States(master=torch.empty(L, dtype=sdt, device="cuda") if need_master else None,
                  m=torch.empty(L, dtype=sdt, device="cuda"),
                  v=torch.empty(L, dtype=sdt, device="cuda"))
    hp = hparams(wl, mask)
    z.zero_init_states(hp, param, st)
    if master0 is not None:
        # rank mode: the rank's master is drawn directly; its gathered slot holds
        # the rounding of that master, as after an earlier step
        st.master.copy_(master0)
        param[a:b].copy_(master0.to(param.dtype))
    return hp, param, st, flags, master0


def check_all(tag, wl, param_d, st, ref):
    """ref = (param, master, m, v) from the oracle; every element within the bar
    and bit-identical. Returns the stats list."""
    pk, sk = kinds(wl)
    p_ref, mst_ref, m_ref, v_ref = ref
    out = [compare_bits(f"{tag} param", param_d, p_ref, pk),
           compare_bits(f"{tag} m", host(st.m) if not isinstance(st.m, np.ndarray) else st.m,
                        m_ref, sk),
           compare_bits(f"{tag} v", host(st.v) if not isinstance(st.v, np.ndarray) else st.v,
                        v_ref, sk)]
    if mst_ref is not None:
        mst = st.master if isinstance(st.master, np.ndarray) else host(st.master)
        out.append(compare_bits(f"{tag} master", mst, mst_ref, sk))
    return out


def oracle_start(O, wl, p_h, master0_h):
    """The oracle's own initial state for the elements in p_h (the gathered
    parameters of the call's elements): init_states of those parameters in full
    mode; in rank mode zero moments beside the drawn master chunk. Nothing here
    comes from the device."""
    if wl.rank < 0:
        return O.init_states(wl.mode, p_h)
    _, m0, v0 = O.init_states(wl.mode, p_h)
    return master0_h, m0, v0


def check_initial(tag, st_h, ref):
    """The device's initialised (master, m, v) against the oracle's, bit for bit."""
    for name, got, want in zip(("master", "m", "v"), st_h, ref):
        if want is None:
            assert got is None, f"{tag}: the device holds a {name} the oracle does not"
            continue
        compare_bits(f"{tag} initial {name}", got, want, "exact")


def run_full(O, wl, steps, compare_every=1):
    """Every element compared, every `compare_every` steps and at the end."""
    import torch
    say(f"[case] full compare {wl.name}: mode={wl.mode} n={wl.n} N={wl.n_workers} "
        f"rank={wl.rank} steps={steps}")
    hp, param, st, flags, master0 = setup_with_master(wl)
    dec = None if flags is None else flags.astype(np.uint8)
    a, b = wl.shard
    p_h = host(param)
    mst_h, m_h, v_h = oracle_start(O, wl, p_h if wl.rank < 0 else p_h[a:b],
                                   None if master0 is None else host(master0))
    torch.cuda.synchronize()
    check_initial(wl.name, (host(st.master) if st.master is not None else None, host(st.m),
                            host(st.v)), (mst_h, m_h, v_h))
    stats = []
    for t in range(1, steps + 1):
        grads = synth.make_grads(wl, t, "cuda")
        g_h = [host(g) for g in grads]
        z.zero_step(hp, param, grads, st, t)
        if wl.rank < 0:
            p_h, mst_h, m_h, v_h = O.zero_step(wl.mode, p_h, g_h, mst_h, m_h, v_h, t, wl.lr,
                                               wl.beta1, wl.beta2, wl.eps, wl.weight_decay, dec)
        else:
            p_h, mst_h, m_h, v_h = O.rank_step(wl.mode, wl.n_workers, wl.rank, p_h, g_h, mst_h,
                                               m_h, v_h, t, wl.lr, wl.beta1, wl.beta2, wl.eps,
                                               wl.weight_decay, dec)
        if t % compare_every == 0 or t == steps:
            torch.cuda.synchronize()
            stats = check_all(f"{wl.name} t={t}", wl, host(param), st,
                              (p_h, mst_h if st.master is not None else None, m_h, v_h))
            # gradients are read-only
            for k in (0, wl.n_workers - 1):
                assert np.array_equal(host(grads[k]).view(np.uint8), g_h[k].view(np.uint8))
    say(f"[done] {wl.name}: " + "; ".join(
        f"{s['name'].split()[-1]} bitexact {s['bitexact']}/{s['n']} max_ulp {s['max_ulp']}"
        for s in stats))
    return stats


def run_sampled(O, wl, steps, count, compare_steps=None):
    """Full-size workload, compared on a sampled index set (exact per element,
    because the step is elementwise)."""
    import torch
    say(f"[case] sampled compare {wl.name}: mode={wl.mode} n={wl.n} N={wl.n_workers} "
        f"rank={wl.rank} steps={steps}")
    need_free(device_bytes(wl))
    hp, param, st, flags, master0 = setup_with_master(wl)
    a, b = wl.shard
    idx = synth.sample_indices(wl, count)
    idx_d = torch.from_numpy(idx).to("cuda")
    gidx_d = idx_d + a
    dec = None if flags is None else flags[idx + a].astype(np.uint8)
    if wl.decay == "all":
        dec = None
    p_h = host(param[gidx_d])
    mst_h, m_h, v_h = oracle_start(O, wl, p_h,
                                   None if master0 is None else host(master0[idx_d]))
    del master0
    torch.cuda.synchronize()
    check_initial(wl.name, (host(st.master[idx_d]) if st.master is not None else None,
                            host(st.m[idx_d]), host(st.v[idx_d])), (mst_h, m_h, v_h))
    outside = None
    if wl.rank >= 0:
        rng = np.random.default_rng(3)
        pool = np.concatenate([np.arange(0, a), np.arange(b, wl.n)]) if wl.n < 10 ** 7 else None
        if pool is not None and pool.size:
            outside = rng.choice(pool, min(4096, pool.size), replace=False)
        elif pool is None:
            cand = rng.integers(0, wl.n, 8192)
            outside = cand[(cand < a) | (cand >= b)][:4096]
        outside_d = torch.from_numpy(np.asarray(outside, np.int64)).to("cuda")
        outside_before = host(param[outside_d])
    steps_to_compare = set(compare_steps or range(1, steps + 1)) | {steps}
    stats = []
    for t in range(1, steps + 1):
        grads = synth.make_grads(wl, t, "cuda")
        z.zero_step(hp, param, grads, st, t)
        g_h = [host(g[idx_d]) for g in grads]
        del grads
        p_h, mst_h, m_h, v_h = O.full_step(wl.mode, p_h, g_h, mst_h, m_h, v_h, t, wl.lr, wl.beta1,
                                           wl.beta2, wl.eps, wl.weight_decay, dec)
        if t in steps_to_compare:
            torch.cuda.synchronize()
            dev = z.States(master=host(st.master[idx_d]) if st.master is not None else None,
                           m=host(st.m[idx_d]), v=host(st.v[idx_d]))
            stats = check_all(f"{wl.name} t={t}", wl, host(param[gidx_d]), dev,
                              (p_h, mst_h, m_h, v_h))
            say(f"  t={t}: {len(idx)} sampled elements within the bar")
    if outside is not None:
        assert np.array_equal(host(param[outside_d]).view(np.uint8), outside_before.view(np.uint8))
    say(f"[done] {wl.name}: " + "; ".join(
        f"{s['name'].split()[-1]} bitexact {s['bitexact']}/{s['n']} max_ulp {s['max_ulp']}"
        for s in stats))
    del param, st
    torch.cuda.empty_cache()
    return stats
