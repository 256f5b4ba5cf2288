"""bench.py's output contract: one JSON line with the fields a benchmark
harness reads (metric, value, unit, steps, warmup, ms_per_step, ...,
config.workload, roofline, cpu_baseline), and a clear refusal of more than
one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.gpu
def test_bench_json_line_contract():
    r = subprocess.run([sys.executable, "-u", BENCH, "--steps", "3", "--warmup", "2"], capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), key
    assert "vs_baseline" in d
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["value"] > 0
    assert d["config"]["workload"] == "t8192_bf16_fwd"
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["achieved"] > 0 and rf["peak"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["cpu_model"] and cb["blas"] and cb["host_cpus"] >= 1


@pytest.mark.gpu
def test_bench_autograd_line():
    # the same contract when the step runs through the torch.autograd layer
    r = subprocess.run([sys.executable, "-u", BENCH, "--workload", "t8192_mxfp8_fwdbwd", "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline", "--autograd"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["config"]["api"] == "torch.autograd layer" and d["config"]["passes"] == "fwd+bwd"
    assert d["value"] > 0 and d["roofline"]["achieved"] > 0 and d["dtype"] == "mxfp8"
