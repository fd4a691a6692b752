"""Benchmark of the fused ZeRO-sharded Adam step on one MI355X.

A step is one call of zero_step over one batch of resident synthetic inputs:
the reduce-scatter mean over N logical workers' gradients, Adam/AdamW on every
shard, and the all-gather write-back, in one kernel launch. Inputs are
generated on the device before the timed region; the timed region covers K
steps (t = W+1 .. W+K) bracketed by device synchronisation.

Prints one JSON line: throughput in parameters updated per second over the
whole timed region, the HBM roofline of the step kernel (algorithmic bytes per
launch over the mean launch duration, measured with HIP events on the stream
the kernel runs on), and the CPU oracle timed on a bounded sample of the same
workload on this host.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("params updated/sec + achieved HBM GB/s (% of peak), fused ZeRO Adam step, 1 GPU")
# one rank's real-shaped share of an 8B-model step: a 10^9-element shard, 8 bf16
# gradient chunks, fp32 master/m/v, AdamW 0.1, bf16 write-back into the slot
DEFAULT_WORKLOAD = "mixed-rank0-of-8B-n8"
CPU_SAMPLE = 1 << 26  # elements of the workload the CPU oracle steps
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
KERNEL_SRC = os.path.join(ROOT, "zero_sharded_optimizer_amd", "csrc", "zero_kernels.hip")


def bytes_per_param(wl):
    """Algorithmic HBM bytes per updated parameter: every worker's gradient read
    once; master (or in-place parameter), m and v read once and written once; the
    gathered parameter written once when it is a separate buffer (bf16 or fp16
    in the mixed modes, the rank's slot in rank mode); one decay-mask bit when a mask is used."""
    from zero_sharded_optimizer_amd import synth
    g = {0: 8, 1: 4, 2: 2, 3: 2}[wl.mode]
    s = 8 if wl.mode == 0 else 4
    p = g
    b = wl.n_workers * g + 6 * s
    if wl.mode in (2, 3) or wl.rank >= 0:
        b += p
    if synth.decay_flags(wl) is not None:
        b += 1 / 8
    return b


def bytes_per_param_clipped(wl):
    """The clipped step moves the fused step's bytes plus the materialised mean
    gradient, written once by the reduce-scatter kernel and read once by the step
    kernel (2 * sizeof(S)); the per-block partial sums are negligible."""
    s = 8 if wl.mode == 0 else 4
    return bytes_per_param(wl) + 2 * s


def bytes_per_param_with_mean(wl):
    """The step that also stores the averaged gradient (zero_step_with_mean):
    the fused step's bytes plus one value of the state type written."""
    return bytes_per_param(wl) + (8 if wl.mode == 0 else 4)


def kernel_hash():
    """Hash of the kernel source's code: comments and whitespace removed, so a
    comment-only edit does not mark the measured traffic as stale."""
    import re
    with open(KERNEL_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = re.sub(r"\s+", "", src)
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def load_traffic(workload, algo_bytes):
    """HBM bytes per launch measured by rocprofv3 counters (two --pmc runs,
    summarised in profiles/traffic_<workload>.json), if that summary was taken
    from the current kernel source; else None. Returns (bytes, source): the
    counters are not collected in the timed run itself."""
    rel = os.path.join("profiles", f"traffic_{workload}.json")
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_src_sha256_16") != kernel_hash() or not d.get("command"):
        return None, None
    return d.get("bytes_per_launch"), (f"{rel}: rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs "
                                       f"on kernel source {d['kernel_src_sha256_16']}")


STEP_KERNEL = "zero_step_kernel"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 4 << 30  # the copy ceiling's buffer: 4 GiB read + 4 GiB written per copy


def _pmc_rows(d):
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def pmc_summary(workload, fetch_dir, write_dir, cmd, variant=None):
    """HBM bytes per step launch from two rocprofv3 --pmc passes (FETCH_SIZE,
    WRITE_SIZE; KiB per dispatch). Each counter is scaled by what it reads for
    the plain 4 GiB device copy run in the same process (known bytes / counter).
    Writes profiles/traffic_<workload>.json and .md."""
    import statistics
    if not cmd.strip():
        raise SystemExit("--pmc-summary needs --cmd: the exact rocprofv3 commands of both runs")
    from zero_sharded_optimizer_amd import synth
    wl = synth.WORKLOADS[workload]
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(d) if r["Counter_Name"] == name]
        step = [float(r["Counter_Value"]) for r in rows if STEP_KERNEL in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL in r["Kernel_Name"]]
        big = max(copy)
        copy = [c for c in copy if c > 0.9 * big]  # the 4 GiB copies
        factor = COPY_BYTES / (statistics.median(copy) * 1024)
        res[name] = {"step_kib_mean": statistics.mean(step), "step_dispatches": len(step),
                     "copy_kib_median": statistics.median(copy), "copy_dispatches": len(copy),
                     "factor": factor,
                     "step_bytes": statistics.mean(step) * 1024 * factor}
    bpp = bytes_per_param_with_mean(wl) if variant == "mean" else bytes_per_param(wl)
    algo = bpp * wl.length
    total = res["FETCH_SIZE"]["step_bytes"] + res["WRITE_SIZE"]["step_bytes"]
    out = {"workload": workload, "kernel": STEP_KERNEL, "kernel_src_sha256_16": kernel_hash(),
           "bytes_per_launch": total, "algorithmic_bytes_per_launch": algo,
           "traffic_over_algorithmic": total / algo, "counters": res, "command": cmd,
           **({"variant": variant} if variant else {})}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    label = workload if not variant else f"{workload}_{variant}"
    base = os.path.join(ROOT, "profiles", f"traffic_{label}")
    with open(base + ".json", "w") as f:
        json.dump(out, f, indent=2)
    with open(base + ".md", "w") as f:
        f.write(f"# HBM traffic of {STEP_KERNEL}, workload {label}\n\n")
        f.write(f"Commands (run from the repository root on one MI355X):\n\n```\n{cmd}\n```\n\n")
        f.write("| counter | step kernel, KiB/dispatch | dispatches | 4 GiB copy, KiB | factor | bytes/launch |\n|---|---|---|---|---|---|\n")
        for k, v in res.items():
            f.write(f"| {k} | {v['step_kib_mean']:.1f} | {v['step_dispatches']} | {v['copy_kib_median']:.1f} | "
                    f"{v['factor']:.4f} | {v['step_bytes']:.4e} |\n")
        f.write(f"\nTraffic {total:.4e} B per launch against {algo:.4e} algorithmic bytes "
                f"({bpp} B/param x {wl.length} params): ratio "
                f"{total / algo:.4f}.\n")
    return out


def kt_summary(workload, kt_dir, cmd, variant=None, bench_json=None):
    """Per-kernel durations from rocprofv3 --kernel-trace --stats, as
    profiles/kernel_trace_<workload>[_<variant>].md (variant: e.g. "clip" for a
    --clip run). bench_json: the JSON line bench.py printed in the profiled
    run, whose HIP-event kernel time is set beside rocprofv3's average."""
    import csv
    import glob
    if not cmd.strip():
        raise SystemExit("--kt-summary needs --cmd: the exact rocprofv3 command of the run")
    f = glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    label = workload if not variant else f"{workload}_{variant}"
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{label}.md")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write(f"# rocprofv3 kernel statistics, workload {label}\n\n")
        fh.write(f"Command (run from the repository root on one MI355X):\n\n```\n{cmd}\n```\n\n")
        fh.write("Template arguments of `zero_step_kernel`: mode, fixed worker count (0: any "
                 "N), gradient-pointer capacity, threads per block, groups per thread, "
                 "optimizer (0 Adam, 1 SGD), load issue (0: state loads after the fold, 1: with "
                 "the gradient loads, 2: one stream in flight per wave), groups 64 apart "
                 "(wave-contiguous), averaged gradient stored.\n\n")
        fh.write("| kernel | calls | average ns | min ns | max ns | % of GPU time |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"].replace("(anonymous namespace)::", "")
            if name.startswith("void "):
                name = name[5:]
            cut = name.find(">(")
            name = name[:cut + 1] if cut >= 0 else name.split("(")[0]
            name = name[:110]
            fh.write(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['Percentage']):.2f} |\n")
        if bench_json:
            with open(bench_json) as jf:
                d = json.loads([ln for ln in jf.read().splitlines() if ln.startswith("{")][-1])
            step = [r for r in rows if r["Name"].find(STEP_KERNEL + "<") >= 0]
            calls = max(step, key=lambda r: int(r["Calls"]))
            avg_ms = float(calls["AverageNs"]) / 1e6
            fh.write(f"\nThe same run's bench.py line: step kernel {d['kernel_ms_mean']:.4f} ms "
                     f"(HIP events on the launch stream, mean of {d['steps']} launches), "
                     f"rocprofv3 average {avg_ms:.4f} ms over {calls['Calls']} launches "
                     f"(ratio {avg_ms / d['kernel_ms_mean']:.3f}); roofline achieved "
                     f"{d['roofline']['achieved']:.0f} GB/s, frac {d['roofline']['frac']:.4f}.\n")
    return path


def cpu_baseline(wl, target_s=12.0, sample_n=CPU_SAMPLE):
    """The CPU oracle (single-threaded, as it stands) on the first sample_n
    elements of the same workload, stepped until about target_s seconds. A
    rank-mode workload is sampled as a full-mode call over the same N, dtypes
    and hyperparameters: per element the arithmetic is the same, and the
    oracle's rank share would take the whole gathered vector."""
    import numpy as np
    import torch
    from oracle import Oracle
    from zero_sharded_optimizer_amd import synth
    O = Oracle()
    # the first sample_n elements, as a full-mode call over all N workers; the
    # decay flags (if any) are those of the workload's first sample_n elements
    small = synth.scaled(wl, min(sample_n, wl.length), rank=-1, shapes=(),
                         decay="all" if wl.decay == "all" else "none")
    n = small.n
    assert n > 0

    def host(x):
        if x.dtype in (torch.bfloat16, torch.float16):
            return x.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        return x.cpu().numpy().copy()

    param = host(synth.make_params(small, "cuda")[0])
    grads = [host(g) for g in synth.make_grads(small, 1, "cuda")]
    mst, m, v = O.init_states(small.mode, param)
    dec = None
    if wl.decay == "2d":
        dec = synth.decay_flags(wl)[:n].astype(np.uint8)
    steps, t0 = 0, time.perf_counter()
    while True:
        param, mst, m, v = O.zero_step(small.mode, param, grads, mst, m, v, steps + 1, small.lr,
                                       small.beta1, small.beta2, small.eps, small.weight_decay,
                                       dec)
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    return {"value": n * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} elements (2^{n.bit_length() - 1}) of the workload"
                      f"{' as a full-mode call' if wl.rank >= 0 else ''}, {wl.n_workers} "
                      f"workers, same dtypes and hyperparameters, {steps} steps, "
                      f"single-threaded C++ oracle, {el:.1f} s"}


def cpu_threads():
    """Host threads to use: the CPUs this process may run on, at most 16 (one
    GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n, int(os.environ.get("OMP_NUM_THREADS", n))))


def cpu_baseline_threads(wl, target_s=8.0, sample_n=CPU_SAMPLE):
    """The same oracle, unchanged, on the same sample split into one slice per
    host thread (the step is elementwise, so the slices are independent; the
    oracle's C code runs without Python's lock). Elements stepped per second
    over all threads."""
    import threading
    import numpy as np
    import torch
    from oracle import Oracle
    from zero_sharded_optimizer_amd import synth
    O = Oracle()
    small = synth.scaled(wl, min(sample_n, wl.length), rank=-1, shapes=(),
                         decay="all" if wl.decay == "all" else "none")
    n = small.n

    def host(x):
        if x.dtype in (torch.bfloat16, torch.float16):
            return x.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        return x.cpu().numpy().copy()

    param = host(synth.make_params(small, "cuda")[0])
    grads = [host(g) for g in synth.make_grads(small, 1, "cuda")]
    dec = synth.decay_flags(wl)[:n].astype(np.uint8) if wl.decay == "2d" else None
    T = min(cpu_threads(), n)
    edges = [n * i // T for i in range(T + 1)]
    done = [0] * T
    start = threading.Barrier(T + 1)

    def work(i):
        lo, hi = edges[i], edges[i + 1]
        p = param[lo:hi].copy()
        g = [x[lo:hi].copy() for x in grads]
        d = None if dec is None else dec[lo:hi].copy()
        mst, m, v = O.init_states(small.mode, p)
        start.wait()
        t0 = time.perf_counter()
        steps = 0
        while time.perf_counter() - t0 < target_s:
            p, mst, m, v = O.zero_step(small.mode, p, g, mst, m, v, steps + 1, small.lr,
                                       small.beta1, small.beta2, small.eps,
                                       small.weight_decay, d)
            steps += 1
        done[i] = steps * (hi - lo)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(T)]
    for th in threads:
        th.start()
    start.wait()
    t0 = time.perf_counter()
    for th in threads:
        th.join()
    el = time.perf_counter() - t0
    return {"value": sum(done) / el, "unit": "params/s", "cores": T, "kind": "oracle",
            "sample": f"first {n} elements of the workload in {T} slices, one per host "
                      f"thread, {wl.n_workers} workers, unchanged C++ oracle, {el:.1f} s"}


def copy_ceiling(nbytes=4 << 30, reps=10):
    """A plain device copy of nbytes: read + write bytes over the time, GB/s."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


CEIL_SHAPES = ("512x2", "512x2 wave-contiguous", "256x4 wave-contiguous", "256x1",
               "128x8 wave-contiguous", "64x2 one stream in flight",
               "64x2 one stream in flight, 16 blocks per CU")


def _zceil():
    """The streaming-ceiling library (built next to libzero.so)."""
    import ctypes
    path = os.path.join(ROOT, "zero_sharded_optimizer_amd", "libzceil.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    import torch  # noqa: F401  (torch's HIP runtime first, as for libzero.so)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.zceil_streams.restype = ctypes.c_int
    lib.zceil_streams.argtypes = [P(ctypes.c_void_p), P(ctypes.c_int32), ctypes.c_int32,
                                  P(ctypes.c_void_p), P(ctypes.c_int32), ctypes.c_int32,
                                  ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    return lib


def _time_streams(lib, in_w, out_w, ngroups, reps=10):
    """Best GB/s of zceil_streams over its launch shapes, on one set of fresh
    buffers: len(in_w) streams read and len(out_w) written, ngroups groups of
    in_w[i] / out_w[o] bytes each; per shape the mean over reps launches (HIP
    events on the launch stream). Returns (GB/s, shape name)."""
    import ctypes
    import torch
    ins = [torch.empty(ngroups * w, dtype=torch.uint8, device="cuda") for w in in_w]
    outs = [torch.empty(ngroups * w, dtype=torch.uint8, device="cuda") for w in out_w]
    pin = (ctypes.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
    pout = (ctypes.c_void_p * len(outs))(*[t.data_ptr() for t in outs])
    win = (ctypes.c_int32 * len(in_w))(*in_w)
    wout = (ctypes.c_int32 * len(out_w))(*out_w)
    stream = torch.cuda.current_stream()
    nbytes = ngroups * (sum(in_w) + sum(out_w))
    best = (0.0, None)
    for shape, name in enumerate(CEIL_SHAPES):
        def go():
            rc = lib.zceil_streams(pin, win, len(in_w), pout, wout, len(out_w), ngroups, shape,
                                   ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"zceil_streams returned {rc}")

        go()
        go()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record(stream)
        for _ in range(reps):
            go()
        e.record(stream)
        torch.cuda.synchronize()
        gbps = nbytes / (s.elapsed_time(e) / reps * 1e-3) / 1e9
        best = max(best, (gbps, name))
    del ins, outs
    torch.cuda.empty_cache()
    return best


def stream_ceilings(wl):
    """What the memory system delivers, measured in the same run with kernels
    that move bytes and do no arithmetic (zceil_streams; best of the launch
    shapes the step uses): a copy of 4 GiB; the workload's N gradient streams
    read and one 16-byte stream written; and the step's own stream mix at the
    workload's size (N gradient streams and 3 state streams read, 3 state
    streams and, in mixed precision, the bf16 copy written; the decay bitmask,
    0.125 B per parameter, is left out)."""
    lib = _zceil()
    a, b = wl.shard
    vec = 2 if wl.mode == 0 else 4
    ngroups = (b - a) // vec
    gw = 8 if wl.mode in (2, 3) else 16  # bytes of one group of one gradient stream
    N = wl.n_workers
    out = {}
    out["copy_GBps"], out["copy_shape"] = _time_streams(lib, [16], [16], (4 << 30) // 16)
    out["read_n_write_1_GBps"], out["read_n_write_1_shape"] = _time_streams(
        lib, [gw] * N, [16], ngroups)
    writes = [16, 16, 16] + ([8] if wl.mode in (2, 3) else [])
    out["step_streams"] = (f"{N} x {gw} B + 3 x 16 B read, {len(writes)} streams "
                           f"({'+'.join(str(w) for w in writes)} B) written per group")
    out["step_streams_GBps"], out["step_streams_shape"] = _time_streams(
        lib, [gw] * N + [16] * 3, writes, ngroups)
    return out


def bucket_edges(length, bucket_mib, gbytes):
    """(begin, end) buckets of about bucket_mib MiB of one worker's gradient,
    last bucket first (the order a backward pass finishes them); every begin a
    multiple of 8 elements."""
    size = max(8, int(bucket_mib * (1 << 20)) // gbytes // 8 * 8)
    edges = list(range(0, length, size)) + [length]
    return list(reversed(list(zip(edges[:-1], edges[1:]))))


def run_overlap(args, wl, hp, param, st, grads):
    """The bucketed step overlapped with the production of its gradients.

    A producer stream stands in for backward: for each bucket, last first, it
    runs one bf16 GEMM of gemm x gemm x gemm (compute, as backward's matrix
    products are), then writes that bucket of every worker's gradient (one
    strided device copy from a source of the same values: the gradients are
    the rows of one N x L tensor) and records an event. As a backward hook
    would, the host enqueues each bucket's step (zero_step_buckets with that one
    bucket and its event) right after the bucket's producer work, on the step
    stream, which waits on the device. Timed against the same producer work
    followed by the one-shot zero_step (serialised), and against each alone.
    Every step first waits for the previous one, so the producer never
    overwrites gradients a step is still reading."""
    import torch
    import zero_sharded_optimizer_amd as z
    gbytes = {0: 8, 1: 4, 2: 2, 3: 2}[wl.mode]
    a, b = wl.shard
    L = b - a
    buckets = bucket_edges(L, args.bucket_mib or 25.0, gbytes)
    N = wl.n_workers
    rows = torch.empty(N, L, dtype=grads[0].dtype, device="cuda")
    for k in range(N):
        rows[k].copy_(grads[k])
    grads[:] = [rows[k] for k in range(N)]  # the step reads the rows
    torch.cuda.empty_cache()
    src = rows.clone()
    M = args.overlap_gemm
    A = torch.randn(M, M, device="cuda").to(torch.bfloat16).contiguous() if M else None
    B = torch.randn(M, M, device="cuda").to(torch.bfloat16).contiguous() if M else None
    C = torch.empty(M, M, device="cuda", dtype=torch.bfloat16) if M else None
    main_s = torch.cuda.current_stream()
    prod = torch.cuda.Stream()

    def produce_bucket(lo, hi):
        with torch.cuda.stream(prod):
            if M:
                torch.matmul(A, B, out=C)
            rows[:, lo:hi].copy_(src[:, lo:hi])

    def overlapped(t):
        prod.wait_stream(main_s)
        for lo, hi in buckets:
            produce_bucket(lo, hi)
            ev = torch.cuda.Event()
            ev.record(prod)
            z.zero_step_buckets(hp, param, grads, st, t, [(lo, hi)], [ev], stream=main_s)

    def serial(t):
        prod.wait_stream(main_s)
        for lo, hi in buckets:
            produce_bucket(lo, hi)
        main_s.wait_stream(prod)
        z.zero_step(hp, param, grads, st, t, stream=main_s)

    def producer_only(t):
        prod.wait_stream(main_s)
        for lo, hi in buckets:
            produce_bucket(lo, hi)
        main_s.wait_stream(prod)

    def step_only(t):
        z.zero_step(hp, param, grads, st, t, stream=main_s)

    t = 0
    res = {}
    for name, fn in (("producer", producer_only), ("step", step_only), ("serial", serial),
                     ("overlapped", overlapped)):
        for _ in range(args.warmup):
            t += 1
            fn(t)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            t += 1
            fn(t)
        torch.cuda.synchronize()
        res[name] = (time.perf_counter() - t0) * 1e3 / args.steps
    hidden = (res["serial"] - res["overlapped"]) / res["step"]
    return buckets, res, hidden


def overlap_summary(workload, kt_dir, cmd, bench_json=None):
    """From a rocprofv3 --kernel-trace run of bench.py --overlap: how much of
    the step kernels' time ran while a producer kernel (GEMM or copy) was also
    running, in the overlapped phase (the last zero_step_buckets launches).
    Writes profiles/overlap_<workload>.md."""
    import csv
    import glob
    if not cmd.strip():
        raise SystemExit("--overlap-summary needs --cmd: the exact rocprofv3 command of the run")
    f = glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    ks = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                 for r in rows), key=lambda x: x[0])
    steps = [k for k in ks if STEP_KERNEL in k[2]]
    others = [k for k in ks if STEP_KERNEL not in k[2]]
    with open(bench_json) as jf:
        d = json.loads([ln for ln in jf.read().splitlines() if ln.startswith("{")][-1])
    nb = d["config"]["buckets"]
    per_phase = d["steps"] + d["warmup"]
    # phases in order: producer (no step kernel), step (1 per step), serial (1 per
    # step), overlapped (nb per step): the overlapped launches are the last ones
    ovl = steps[-per_phase * nb:]
    lo_t, hi_t = ovl[0][0], ovl[-1][1]
    prod = [k for k in others if k[1] > lo_t and k[0] < hi_t]
    busy = 0
    overlap = 0
    for s0, s1, _ in ovl:
        busy += s1 - s0
        cuts = sorted((max(s0, p0), min(s1, p1)) for p0, p1, _ in prod if p0 < s1 and p1 > s0)
        cur_s = cur_e = None
        for x0, x1 in cuts:  # union of the producer intervals inside this step kernel
            if cur_e is None or x0 > cur_e:
                if cur_e is not None:
                    overlap += cur_e - cur_s
                cur_s, cur_e = x0, x1
            else:
                cur_e = max(cur_e, x1)
        if cur_e is not None:
            overlap += cur_e - cur_s
    path = os.path.join(ROOT, "profiles", f"overlap_{workload}.md")
    with open(path, "w") as fh:
        fh.write(f"# Bucketed step overlapped with its gradient producer, workload {workload}\n\n")
        fh.write(f"Command (run from the repository root on one MI355X):\n\n```\n{cmd}\n```\n\n")
        ov = d["overlap"]
        fh.write(f"{nb} buckets of {d['config']['bucket_mib']} MiB; producer per bucket: one bf16 "
                 f"GEMM of {d['config']['overlap_gemm']}^3, then the bucket of every worker's "
                 f"gradient written (one strided device copy); each bucket's step enqueued right "
                 f"after, waiting on the device for the bucket's event.\n\n")
        fh.write("| phase | ms per step (wall, the bench line) |\n|---|---|\n")
        for k in ("producer", "step", "serial", "overlapped"):
            fh.write(f"| {k} | {ov[k + '_ms']:.3f} |\n")
        fh.write(f"\nHidden: (serial - overlapped) / step = {ov['hidden_fraction_of_step']:.3f} of "
                 f"the step's time.\n\n")
        fh.write(f"From the trace, overlapped phase: {len(ovl)} step-kernel launches over "
                 f"{(hi_t - lo_t) / 1e6:.3f} ms, {busy / 1e6:.3f} ms of step-kernel time, of which "
                 f"{overlap / 1e6:.3f} ms ({overlap / max(busy, 1):.3f}) ran while a producer "
                 f"kernel was running ({len(prod)} producer kernels in the window).\n\n")
        fh.write("The first 24 kernels of the last overlapped step, by start time (us from its "
                 "first kernel; its producer starts once the previous step's last bucket has "
                 "ended):\n\n| start | end | kernel |\n|---|---|---|\n")
        t_begin = ovl[-nb - 1][1] if len(ovl) > nb else ovl[0][0]
        win = [k for k in ks if k[0] >= t_begin][:24]
        if win:
            base = win[0][0]
            for k0, k1, name in win:
                short = name.replace("(anonymous namespace)::", "").split("(")[0][:90]
                fh.write(f"| {(k0 - base) / 1e3:.1f} | {(k1 - base) / 1e3:.1f} | `{short}` |\n")
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--native-buckets", action="store_true",
                    help="with --bucket-mib: enqueue all buckets in one zero_step_buckets call")
    ap.add_argument("--graph", action="store_true",
                    help="with --bucket-mib: capture the buckets once into a HIP graph "
                         "(zero_step_range_dev, step scalars in device memory) and replay it "
                         "each step")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the copy and streaming-ceiling measurements")
    ap.add_argument("--no-stream-ceilings", action="store_true",
                    help="keep the 4 GiB copy (it calibrates the --pmc counters) but skip the "
                         "streaming-ceiling kernels")
    ap.add_argument("--clip", type=float, default=None, metavar="FRACTION",
                    help="time the clipped step (zero_step_clipped) with max_norm set to "
                         "FRACTION times the first step's global gradient norm")
    ap.add_argument("--bucket-mib", type=float, default=None, metavar="MIB",
                    help="time the bucketed step: zero_step_range over buckets of MIB MiB of "
                         "one worker's gradient, last bucket first")
    ap.add_argument("--with-mean", action="store_true",
                    help="time zero_step_with_mean: the step that also stores the averaged "
                         "gradient (bytes model + sizeof(state) per parameter)")
    ap.add_argument("--overlap", action="store_true",
                    help="time the bucketed step (zero_step_buckets, --bucket-mib, default 25) "
                         "overlapped with a producer stream that writes each bucket's gradients, "
                         "against producer then step serialised")
    ap.add_argument("--overlap-gemm", type=int, default=4096, metavar="M",
                    help="with --overlap: the producer's bf16 GEMM per bucket is M x M x M (0: "
                         "gradient writes only)")
    ap.add_argument("--overlap-summary", metavar="KT_DIR",
                    help="summarise a rocprofv3 --kernel-trace run of --overlap (with "
                         "--bench-json) into profiles/ and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into profiles/ and exit")
    ap.add_argument("--kt-summary", metavar="KT_DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run into profiles/ and exit")
    ap.add_argument("--cmd", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--bench-json", default=None,
                    help="with --kt-summary: the profiled run's bench.py output")
    ap.add_argument("--variant", default=None,
                    help="with --kt-summary: a suffix for the summary's name (e.g. clip)")
    args = ap.parse_args()
    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.workload, *args.pmc_summary, args.cmd, args.variant)))
        return
    if args.kt_summary:
        print(kt_summary(args.workload, args.kt_summary, args.cmd, args.variant, args.bench_json))
        return
    if args.overlap_summary:
        print(overlap_summary(args.workload, args.overlap_summary, args.cmd, args.bench_json))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (all logical workers live in one GPU's HBM); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import zero_sharded_optimizer_amd as z
    from zero_sharded_optimizer_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    a, b = wl.shard
    L = b - a

    # resident inputs
    param, master0 = synth.make_params(wl, "cuda")
    sdt = synth.state_dtype(wl)
    need_master = wl.mode in (2, 3) or wl.rank >= 0
    st = z.States(torch.empty(L, dtype=sdt, device="cuda") if need_master else None,
                  torch.empty(L, dtype=sdt, device="cuda"), torch.empty(L, dtype=sdt, device="cuda"))
    flags = synth.decay_flags(wl)
    mask = z.wd_mask_from_flags(flags) if flags is not None else None
    hp = z.HParams(n=wl.n, n_workers=wl.n_workers, mode=wl.mode, lr=wl.lr, beta1=wl.beta1,
                   beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay, rank=wl.rank,
                   wd_mask=mask)
    z.zero_init_states(hp, param, st)
    if master0 is not None:
        st.master.copy_(master0)
        param[a:b].copy_(master0.to(param.dtype))
        del master0
    grads = synth.make_grads(wl, 1, "cuda")
    torch.cuda.synchronize()

    max_norm = None
    if args.clip is not None:
        if wl.rank >= 0:
            print("--clip needs a full-mode workload", file=sys.stderr)
            sys.exit(2)
        ss = torch.zeros(1, dtype=torch.float64, device="cuda")
        mean = torch.empty(L, dtype=sdt, device="cuda")
        ws = torch.empty(max(1, z.zero_mean_grad_workspace_bytes(hp)), dtype=torch.uint8,
                         device="cuda")
        z.zero_mean_grad(hp, grads, mean, ss, ws)
        max_norm = args.clip * float(ss.item()) ** 0.5
        del mean, ws
        ws = torch.empty(z.zero_step_clipped_workspace_bytes(hp), dtype=torch.uint8, device="cuda")

    if args.overlap:
        if args.clip is not None or args.graph:
            print("--overlap takes neither --clip nor --graph", file=sys.stderr)
            sys.exit(2)
        buckets, ov, hidden = run_overlap(args, wl, hp, param, st, grads)
        out = {
            "metric": METRIC + " (bucketed, overlapped with the gradient producer)",
            "value": L / (ov["overlapped"] * 1e-3), "unit": "params/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ov["overlapped"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": {0: "f64", 1: "f32", 2: "bf16+f32", 3: "f16+f32"}[wl.mode],
            "data": "synthetic (seeded device-side draws; no dataset)",
            "config": {"workload": wl.name, "params_updated_per_step": L,
                       "n_workers": wl.n_workers, "bucket_mib": args.bucket_mib or 25.0,
                       "buckets": len(buckets), "overlap_gemm": args.overlap_gemm,
                       "parallelism": "1 GPU, N logical workers in one HBM"},
            "overlap": {"producer_ms": ov["producer"], "step_ms": ov["step"],
                        "serial_ms": ov["serial"], "overlapped_ms": ov["overlapped"],
                        "hidden_fraction_of_step": hidden},
        }
        print(json.dumps(out), flush=True)
        return

    buckets = None
    if args.bucket_mib is not None:
        gbytes = {0: 8, 1: 4, 2: 2, 3: 2}[wl.mode]
        buckets = bucket_edges(L, args.bucket_mib, gbytes)

    mean_out = None
    if args.with_mean:
        if args.clip is not None or buckets is not None:
            print("--with-mean takes neither --clip nor --bucket-mib", file=sys.stderr)
            sys.exit(2)
        mean_out = torch.empty(L, dtype=sdt, device="cuda")

    graph = None
    if args.graph:
        if buckets is None or args.clip is not None:
            print("--graph needs --bucket-mib (and no --clip)", file=sys.stderr)
            sys.exit(2)
        import numpy as np
        # every step's scalars, prepared up front (they depend only on t)
        total = args.warmup + args.steps
        scal_all = torch.from_numpy(np.concatenate(
            [z.zero_step_scalars(hp, t) for t in range(1, total + 1)])).cuda()
        scal = torch.empty(z.STEP_SCALARS_BYTES, dtype=torch.uint8, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for lo, hi in buckets:
                    z.zero_step_range_dev(hp, param, grads, st, scal, lo, hi)
        torch.cuda.synchronize()

    def one_step(t, stream=None):
        if graph is not None:
            k = z.STEP_SCALARS_BYTES
            scal.copy_(scal_all[(t - 1) * k:t * k])
            graph.replay()
        elif buckets is not None and args.native_buckets:
            z.zero_step_buckets(hp, param, grads, st, t, buckets, stream=stream)
        elif buckets is not None:
            for lo, hi in buckets:
                z.zero_step_range(hp, param, grads, st, t, lo, hi, stream=stream)
        elif mean_out is not None:
            z.zero_step_with_mean(hp, param, grads, st, t, mean_out, stream=stream)
        elif max_norm is None:
            z.zero_step(hp, param, grads, st, t, stream=stream)
        else:
            z.zero_step_clipped(hp, param, grads, st, t, max_norm, ws, sumsq_out=ss,
                                stream=stream)

    for t in range(1, args.warmup + 1):
        one_step(t)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        one_step(args.warmup + 1 + i, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in ev]
    avg_ms = sum(kern_ms) / len(kern_ms)

    if max_norm is not None:
        bpp = bytes_per_param_clipped(wl)
    elif mean_out is not None:
        bpp = bytes_per_param_with_mean(wl)
    else:
        bpp = bytes_per_param(wl)
    algo_bytes = bpp * L
    achieved = algo_bytes / (avg_ms * 1e-3) / 1e9
    if max_norm is None and buckets is None:
        traffic, traffic_src = load_traffic(wl.name + ("_mean" if mean_out is not None else ""),
                                            algo_bytes)
    else:
        traffic, traffic_src = None, None
    dtype = {0: "f64", 1: "f32", 2: "bf16+f32", 3: "f16+f32"}[wl.mode]

    with_mean = mean_out is not None
    del grads, param, st, mean_out
    torch.cuda.empty_cache()
    copy_gbps = None if args.no_copy_ceiling else copy_ceiling()
    ceil = None if args.no_copy_ceiling or args.no_stream_ceilings else stream_ceilings(wl)
    if ceil is not None and ceil["step_streams_GBps"]:
        ceil["step_frac_of_step_streams"] = achieved / ceil["step_streams_GBps"]
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)
    cpu_mt = None if args.no_cpu_baseline else cpu_baseline_threads(wl)

    out = {
        "metric": METRIC,
        "value": L * args.steps / wall,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded device-side draws; no dataset)",
        "config": {"workload": wl.name, "params_updated_per_step": L, "n_workers": wl.n_workers,
                   "mode": dtype, "rank": wl.rank, "lr": wl.lr, "betas": [wl.beta1, wl.beta2],
                   "eps": wl.eps, "weight_decay": wl.weight_decay, "decay": wl.decay,
                   "bytes_per_param": bpp, "parallelism": "1 GPU, N logical workers in one HBM",
                   **({} if max_norm is None else
                      {"clipped": True, "clip_fraction": args.clip, "max_norm": max_norm}),
                   **({} if buckets is None else
                      {"bucket_mib": args.bucket_mib, "buckets": len(buckets)}),
                   **({"graph": True} if graph is not None else {}),
                   **({"with_mean": True} if with_mean else {}),
                   **({"native_buckets": True} if buckets is not None and args.native_buckets
                      else {})},
        "achieved_GBps": achieved,
        "kernel_ms_mean": avg_ms,
        "kernel_ms_median": sorted(kern_ms)[len(kern_ms) // 2],
        "kernel_ms_min": min(kern_ms),
        "copy_ceiling_GBps": copy_gbps,
        "stream_ceilings": ceil,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "traffic_source": traffic_src},
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_mt,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
