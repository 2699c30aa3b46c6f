"""bench.py's command-line contract: one GPU only (CPU check), and the one JSON line of a
default run with every field the contract names (GPU check, a short run)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    p = _bench("--gpus", "2", timeout=120)
    assert p.returncode != 0
    assert "one GPU" in json.loads(p.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.gpu
def test_default_run_prints_the_contract_line():
    print("bench.py --steps 2 --warmup 1", flush=True)
    p = _bench("--steps", "2", "--warmup", "1", timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    q = d["roofline_quantize"]
    assert q["bound"] == "hbm" and q["kernel_ms"] > 0 and q["kernel_ms_in_step"] > 0
    assert abs(q["achieved"] - q["bytes_per_launch"] / (q["kernel_ms"] * 1e-3) / 1e9) < 1e-6 * q["achieved"]
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]


@pytest.mark.gpu
def test_column_shard_line():
    """The W4A4 step at one GPU's column shard (N = 28672 / 8 = 3584): one contract line,
    its GEMM roofline priced on the shard's own FLOP."""
    print("bench.py --workload w4a4_shard", flush=True)
    p = _bench("--workload", "w4a4_shard", "--steps", "2", "--warmup", "1", "--settle", "0.2", "--no-cpu",
               timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["flop_per_launch"] == 2.0 * 8192 * 3584 * 8192
    assert abs(r["achieved"] - r["flop_per_launch"] / (r["kernel_ms"] * 1e-3) / 1e12) < 1e-6 * r["achieved"]
    assert d["config"]["N"] == 3584 and "shard" in d["config"]["workload"]


MEMORY_WORKLOADS = [("mxfp4_h32", "quant"), ("mxfp4_h32", "dequant"), ("nvfp4_h16", "quant"),
                    ("nvfp4_h16", "dequant"), ("dualscale_pack", "quant"),
                    ("dualscale_pack", "dequant"), ("arcquant", "quant"), ("arcquant_gamma", "quant"),
                    ("arcquant_mx", "quant"), ("nvfp4_roundtrip", "quant")]


@pytest.mark.gpu
@pytest.mark.parametrize("workload,op", MEMORY_WORKLOADS)
def test_memory_workload_lines(workload, op):
    """Each memory-bound workload prints one contract line with its HBM roofline, timed on
    the second of two passes, the first pass reported beside it."""
    print(f"bench.py --workload {workload} --op {op}", flush=True)
    p = _bench("--workload", workload, "--op", op, "--steps", "5", "--warmup", "1", "--settle", "0.2",
               "--no-cpu", timeout=240)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["achieved"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert r["kernel_ms"] > 0 and r["first_pass_kernel_ms"] > 0 and r["bytes_per_launch"] > 0
    reps = sorted(r["kernel_ms_replays"])
    assert len(reps) == 5 and reps[2] == r["kernel_ms"]              # the median of five replays
    assert abs(r["achieved"] - r["bytes_per_launch"] / (r["kernel_ms"] * 1e-3) / 1e9) < 1e-6 * r["achieved"]
    assert workload in d["config"]["workload"]
