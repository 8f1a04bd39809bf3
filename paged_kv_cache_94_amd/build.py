"""Build libpa.so (the HIP kernels plus the C-ABI) for gfx950, in-tree.

Every HIP source is compiled by hipcc for gfx950 only, with packed-fp32
instructions disabled, and linked into paged_kv_cache_94_amd/libpa.so. The
library carries the hash of the sources it was built from (pa_build_id);
the binding refuses a library whose hash differs from its sources'.
Run as ``python -m paged_kv_cache_94_amd.build``.
"""

from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "pa_error.cpp", "pa_alloc.cpp", "pa_valu.hip", "pa_mfma.hip", "pa_aux.hip", "pa_write.hip",
           "pa_prefill.hip"]
SOURCE_SUFFIXES = (".cpp", ".hip", ".h")


def source_hash(root: str = ROOT) -> str:
    """16 hex digits of a SHA-256 over the library's sources and headers (names and contents)."""
    h = hashlib.sha256()
    for sub in (os.path.join("paged_kv_cache_94_amd", "csrc"), "include"):
        d = os.path.join(root, sub)
        for name in sorted(os.listdir(d)):
            if name.endswith(SOURCE_SUFFIXES):
                h.update(f"{sub}/{name}\0".encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
                h.update(b"\0")
    return h.hexdigest()[:16]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


# Libraries: the release library; a diagnostic copy of the same sources
# compiled with PA_STAMPS, whose matrix-core kernel records per-workgroup
# phase timestamps into pa_args.debug_stamps (bench.py --stamps); and the
# read-ceiling probe, a load-only kernel over a workload's cache tiles
# (bench.py --ceiling).
VARIANTS = {
    "release": {"lib": LIB, "objdir": BUILD, "flags": [], "sources": SOURCES},
    "stamps": {"lib": os.path.join(PKG, "libpa_stamps.so"), "objdir": os.path.join(PKG, "_build_stamps"),
               "flags": ["-DPA_STAMPS"], "sources": SOURCES},
    "probe": {"lib": os.path.join(PKG, "libpa_probe.so"), "objdir": os.path.join(PKG, "_build_probe"),
              "flags": [], "sources": ["pa_probe.hip"]},
}
STAMPS_LIB = VARIANTS["stamps"]["lib"]
PROBE_LIB = VARIANTS["probe"]["lib"]
ALL_VARIANTS = ("release", "stamps", "probe")


def _compile(src: str, extra: list, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + COMMON + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags: list | None = None, variants=("release",)) -> str:
    """Compile every source and link each requested variant; returns the release library's path."""
    extra = list(extra_flags or []) + [f'-DPA_BUILD_ID="{source_hash()}"']
    jobs = [(v, src) for v in variants for src in VARIANTS[v]["sources"]]
    for v in variants:
        os.makedirs(VARIANTS[v]["objdir"], exist_ok=True)
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    # The matrix-core kernels take longest: start them first.
    jobs.sort(key=lambda j: j[1] != "pa_mfma.hip")
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda j: (j[0], _compile(j[1], extra + VARIANTS[j[0]]["flags"], VARIANTS[j[0]]["objdir"])),
                           jobs))
    for v in variants:
        target = VARIANTS[v]["lib"]
        tmp = target + ".tmp%d" % os.getpid()
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for vv, o in objs if vv == v]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"linking {os.path.basename(target)} failed:\n{res.stdout}\n{res.stderr}")
        os.replace(tmp, target)
        if verbose:
            print(f"built {target}")
    return LIB


if __name__ == "__main__":
    # python -m paged_kv_cache_94_amd.build [--all] [extra hipcc flags...]
    argv = sys.argv[1:]
    variants = ALL_VARIANTS if "--all" in argv else ("release",)
    build(verbose=True, extra_flags=[a for a in argv if a != "--all"], variants=variants)
