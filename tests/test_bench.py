"""The benchmark's contract: its refusal of several GPUs (CPU) and the JSON record of a short run (GPU)."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    # Exits with status 2 and says why, before any GPU call.
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_host_cpu_names_the_model_and_cpu_count():
    sys.path.insert(0, ROOT)
    import bench
    desc = bench.host_cpu()
    assert f"{os.cpu_count()} logical CPUs" in desc and "usable" in desc
    model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][:1]
    if model:
        assert desc.startswith(model[0])


def test_ring_and_head_scales_need_one_workload():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--ring"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert p.returncode == 2 and "--config" in p.stderr


@pytest.mark.gpu
def test_short_run_prints_one_json_record():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "1", "--steps", "16",
                        "--warmup", "2", "--no-cpu-baseline", "--no-append"], capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 16 and rec["warmup"] == 2 and rec["value"] > 0
    assert rec["config"]["workload"].startswith("tiny-f32") and rec["config"]["kernel_stamped_steps"] == 16
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    assert rec["config"]["kernel_us"]["mean"] > 0 and rec["cpu_baseline"] is None


@pytest.mark.gpu
def test_default_run_times_every_workload_with_the_verify_step_as_headline():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "12", "--warmup", "2",
                        "--no-cpu-baseline", "--no-append"], capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    assert rec["config"]["workload"].startswith("verify5-bf16")
    configs = rec["config"]["configs"]
    assert sorted(configs) == ["C1", "C2", "C3", "C4", "C5"]
    for name, c in configs.items():
        assert c["kernel_stamped_steps"] >= 10, name
        assert c["kernel_us"]["mean"] > 0 and 0 < c["frac"] < 1, name
        assert c["step_us"] > 0 and c["queries_per_s"] > 0, name
    assert configs["C5"]["frac"] == rec["roofline"]["frac"]
    assert abs(rec["value"] - configs["C5"]["queries_per_s"]) < 1e-6 * rec["value"]
    assert "traffic_source" in rec["roofline"]
