"""The benchmark's reporting contract: the CPU-oracle baseline times what it
ran, --gpus above 1 is refused before anything touches a GPU, and (GPU) one
run prints one JSON line with every field of the contract."""
import json
import os
import re
import subprocess
import sys
import time

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_cpu_baseline_times_the_oracle_it_ran():
    import bench
    cfg = W.WORKLOADS["tiny"]            # RoPE on, first frame position 2
    t = time.perf_counter()
    r = bench.cpu_baseline(cfg, budget_s=0.2)
    wall = time.perf_counter() - t
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    assert 0 < r["seconds"] <= wall + 1e-3
    heads = int(re.search(r"attention for (\d+) of \d+ heads", r["sample"]).group(1))
    assert 1 <= heads <= cfg.n_heads
    flops = W.attn_flops(cfg, W.make_mask(cfg)) * heads / cfg.n_heads
    assert r["value"] == pytest.approx(flops / r["seconds"] / 1e12, rel=1e-2)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_prints_one_contract_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--configs", "tiny,wan13b,bsa_sr"], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    r = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in r, k
    assert r["n_gpus"] == 1 and r["steps"] == 3 and r["warmup"] == 1
    assert r["higher_is_better"] is True and r["data"] == "synthetic" and r["dtype"].startswith("bf16")
    assert r["config"]["workload"] == "wan13b" and r["value"] > 0 and r["ms_per_step"] > 0
    # untimed clock-settling steps ran before the warmup steps, and say so
    assert r["clock_settle"]["untimed_steps"] >= 1 and r["clock_settle"]["seconds"] > 0
    rf = r["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    assert rf["traffic"] is None or rf["traffic"] > 0
    # one record per requested workload; the headline one is the same measurement
    assert sorted(r["configs"]) == ["bsa_sr", "tiny", "wan13b"]
    assert r["configs"]["wan13b"]["attn_ms"] == r["attn_ms"]
    for name, c in r["configs"].items():
        assert c["attn_ms"] > 0 and c["step_ms"] >= c["attn_ms_p10_p90"][0] * 0.5
        assert c["roofline"]["bound"] == ("latency" if name == "tiny" else "mfma")
        assert c["roofline"]["frac"] > 0
    assert set(r["clocks"]) >= {"before", "after"}
