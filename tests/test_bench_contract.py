"""bench.py's output contract: one JSON line with the metric, the roofline
object (traffic from counters taken on the current kernel source) and the CPU
baseline, and a clear refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from zero_sharded_optimizer_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


@pytest.mark.parametrize("workload", sorted(synth.WORKLOADS))
def test_traffic_summaries_match_the_current_kernel_source(workload):
    """Each workload's counter summary was taken on the kernel source as it
    stands (the hash of its code, comments and whitespace removed), and its
    traffic is the algorithmic bytes: otherwise the bench line's traffic is null
    and the profiles are stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    assert os.path.exists(path), path
    d = json.load(open(path))
    assert d["kernel_src_sha256_16"] == bench.kernel_hash(), "re-take the counters"
    wl = synth.WORKLOADS[workload]
    algo = bench.bytes_per_param(wl) * wl.length
    assert d["algorithmic_bytes_per_launch"] == pytest.approx(algo)
    assert 0.999 <= d["bytes_per_launch"] / algo <= 1.002


def test_mean_store_traffic_is_one_more_state_value_per_parameter():
    """The counters of zero_step_with_mean on the 8B-model rank share: the fused
    step's 42 B/param plus one fp32 mean written, 46 B/param, on the current
    kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_mixed-rank0-of-8B-n8_mean.json")
    assert os.path.exists(path), path
    d = json.load(open(path))
    assert d["kernel_src_sha256_16"] == bench.kernel_hash(), "re-take the counters"
    wl = synth.WORKLOADS["mixed-rank0-of-8B-n8"]
    assert bench.bytes_per_param_with_mean(wl) == 46
    assert d["algorithmic_bytes_per_launch"] == pytest.approx(46 * wl.length)
    assert 0.999 <= d["bytes_per_launch"] / (46 * wl.length) <= 1.002


def test_every_profile_summary_records_its_command():
    """Every committed profile summary gives the full command that made it (the
    rocprofv3 invocation, with the program after --), so each figure can be
    re-taken; an empty command block fails."""
    import re
    d = os.path.join(ROOT, "profiles")
    files = sorted(os.listdir(d))
    assert files
    for fn in files:
        txt = open(os.path.join(d, fn)).read()
        if fn.endswith(".json"):
            cmd = json.loads(txt).get("command", "")
        else:
            blocks = re.findall(r"```\n(.*?)```", txt, flags=re.S)
            assert blocks, f"{fn}: no command block"
            cmd = blocks[0]
        assert cmd.strip(), f"{fn}: empty command"
        assert "rocprofv3" in cmd, f"{fn}: the command is not a rocprofv3 run"
        for line in cmd.splitlines():
            if line.lstrip().startswith("rocprofv3") or " rocprofv3 " in line:
                assert " -- python" in line or " -- ./" in line, f"{fn}: {line}"


@pytest.mark.gpu
def test_bench_line_on_the_gpu():
    print("[case] bench.py --steps 3 --warmup 1 --no-copy-ceiling", flush=True)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                          "--warmup", "1", "--no-copy-ceiling"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["config"]["workload"] == "mixed-rank0-of-8B-n8" and "model" not in d["config"]
    assert d["config"]["params_updated_per_step"] == 1_000_000_000
    assert d["value"] > 0 and d["unit"] == "params/s" and d["dtype"] == "bf16+f32"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    wl = synth.WORKLOADS["mixed-rank0-of-8B-n8"]
    if bench.load_traffic(wl.name, 42 * wl.length)[0] is None:
        # no counter summary of the current kernel source: traffic is null
        assert r["traffic"] is None and r["traffic_source"] is None
    else:
        assert r["traffic"] == pytest.approx(42 * 1_000_000_000, rel=2e-3)
        assert r["traffic_source"].startswith("profiles/traffic_mixed-rank0-of-8B-n8.json")
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["value"] > 0
    assert c["sample"].startswith(f"first {1 << 26} elements (2^26)")


@pytest.mark.gpu
def test_bench_overlap_line_on_the_gpu():
    """--overlap prints one line whose phases are consistent: the serialised run
    is at least as long as the producer and the step each, and the hidden
    fraction is (serial - overlapped) / step."""
    print("[case] bench.py --overlap on fp32-320M-n8", flush=True)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                          "--warmup", "1", "--workload", "fp32-320M-n8", "--overlap",
                          "--overlap-gemm", "1024"],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    ov = d["overlap"]
    assert d["config"]["buckets"] > 1 and d["value"] > 0
    assert ov["serial_ms"] >= 0.9 * max(ov["producer_ms"], ov["step_ms"])
    assert ov["hidden_fraction_of_step"] == pytest.approx(
        (ov["serial_ms"] - ov["overlapped_ms"]) / ov["step_ms"])


@pytest.mark.gpu
@pytest.mark.parametrize("flags", [["--clip", "0.5"], ["--bucket-mib", "25"],
                                   ["--bucket-mib", "25", "--native-buckets"],
                                   ["--bucket-mib", "25", "--graph"], ["--with-mean"]],
                         ids=["clip", "buckets", "native-buckets", "graph", "with-mean"])
def test_bench_variants_on_the_gpu(flags):
    """The variant runs behind the committed kernel-trace summaries still print
    one valid line (a few steps, no baselines or ceilings)."""
    print(f"[case] bench.py --workload fp32-320M-n8 {' '.join(flags)}", flush=True)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2",
                          "--warmup", "1", "--no-cpu-baseline", "--no-copy-ceiling",
                          "--workload", "fp32-320M-n8", *flags],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert d["value"] > 0 and d["roofline"]["achieved"] > 0
    if "--with-mean" not in flags:
        assert d["roofline"]["traffic"] is None  # no counters for these variants
    if "--clip" in flags:
        assert d["config"]["clipped"] is True
    elif "--with-mean" in flags:
        assert d["config"]["with_mean"] is True and d["config"]["bytes_per_param"] == 60
    else:
        assert d["config"]["bucket_mib"] == 25 and d["config"]["buckets"] > 1
