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


def test_host_cpu_names_the_cpu_count():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.host_cpu().endswith(f"{os.cpu_count()} logical CPUs")


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
    assert rec["config"]["workload"].startswith("tiny-f32") and rec["config"]["kernel_stamped_steps"] == 2
    roof = rec["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-12
    assert rec["config"]["kernel_us"]["mean"] > 0 and rec["cpu_baseline"] is None
