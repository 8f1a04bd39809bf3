"""The C ABI used from plain C: tests/c/decode_from_c.c builds against include/pa.h and libpa.so with
gcc (-std=c11, every warning an error) and, on a GPU, runs a decode step checked against the oracle."""

from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_94_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(tmp_path) -> str:
    exe = str(tmp_path / "decode_from_c")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", os.path.join(ROOT, "tests", "c", "decode_from_c.c"),
           "-o", exe, f"-L{PKG}", "-lpa", f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib"]
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stderr[-3000:]
    return exe


def test_header_is_c11_and_links(tmp_path):
    assert os.path.exists(_compile(tmp_path))


@pytest.mark.gpu
def test_decode_from_plain_c(tmp_path):
    exe = _compile(tmp_path)
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(p.stdout, p.stderr)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "max|err| vs fp64 oracle" in p.stdout and "invalid" in p.stdout.lower()
