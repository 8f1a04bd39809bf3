#!/usr/bin/env python3
"""Paged decode-attention benchmark on one MI355X.

One step = one paged decode-attention call (attention kernel, plus the
split-combine kernel when the key range is split) over one batch of a
synthetic workload, inputs resident in HBM. By default every workload of the
set is timed in one run, each with the same number of steps:

  C5 verify5-bf16          (the headline: the largest single-GPU workload)
                           256 sequences x 5 query tokens (speculative verify,
                           causal within the 5), 32 query heads on 8 KV heads,
                           head_dim 128, bf16, lognormal lengths (median 1024)
  C1 tiny-f32              2 sequences (37, 70 tokens), fp32, 4 / 2 heads, D 64
  C2 gemma4-12b-local-bf16 32 sequences, 16 / 8 heads, D 256, window 1024
  C3 gemma4-12b-global-bf16 16 sequences of 4K-32K, 16 heads on 1 KV head,
                           D 256, values are the keys
  C4 gqa70b-int8kv         64 sequences, 64 / 8 heads, D 128, int8 cache

Blocks are 16 tokens, randomly permuted in a pool of total need + 10%.
Between steps the call rotates over several device copies of the cache (and
its own block table) so that no step finds its cache in the 256 MB
Infinity Cache from the previous one: every step reads from HBM.

Prints ONE JSON line on stdout (the run's record); diagnostics go to stderr.
  value     = the headline workload's queries per second over the K timed
              steps (query = one token of one sequence through all heads of
              the layer)
  roofline  = algorithmic bytes of a step / mean duration of the attention
              kernel; on every max(1, K // 16)-th timed step (--event-every)
              the library stamps a pair of HIP events from that kernel's own
              dispatch on the launch stream (hipExtLaunchKernel), the same
              start/end timestamps a kernel trace reports. The events are
              created without the system-scope fence
              (hipEventDisableSystemFence), whose cache writeback and
              invalidation would cost every stamped step GPU time and slow
              the kernel after it. traffic = HBM bytes per launch from
              rocprofv3 counters (traffic_source names the summary), or null
              when no counter pass matches the current kernel sources and plan
  config.configs = the same figures for every workload of the run
  cpu_baseline = the fp64 oracle on the host's cores, same workload
  block_allocator = host time of the block allocator's work for one step
              of the same batch (grow every sequence by its q_len new
              tokens, then export the int32 block table and lengths)
  kv_append = the KV append (pa_cache_write) into the same cache, timed
              apart from the step: once with the step's own new tokens
              (B x q_len) and once with a prefill-sized chunk of tokens
              scattered over the pool, each timed by events that the
              append kernel's own dispatch stamps
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attention queries/s and achieved KV HBM GB/s (% of MI355X peak)"

# HBM bytes per launch of the timed kernel, from two rocprofv3 counter passes
# over this benchmark (FETCH_SIZE, then WRITE_SIZE: KiB per dispatch, mean
# over the run's launches of the kernel). Each is scaled by what the same
# counter read, in the same run, for a plain 1 GiB device-to-device copy
# (--calibrate-copy): FETCH_SIZE read 524314 KiB for 1048576 KiB read (factor
# 2.0), WRITE_SIZE 1048576 KiB for 1048576 KiB written (factor 1.0). A figure
# holds only for the kernel sources and the launch plan it was taken with;
# for anything else the record's traffic is null.
MEASURED_TRAFFIC = {
    1: {"source": "profiles/pa_valu_kernel-tiny_f32-hbm_counters.txt", "kernel_sources": "ea299d4735d08495",
        "plan": {"kernel": 0, "rows": 2, "waves_per_group": 8, "splits": 1, "grid": 4, "balanced": 0, "pieces": 0, "queue": 0},
        "fetch_kib": 89, "fetch_factor": 2.0, "write_kib": 2, "write_factor": 1.0},
    2: {"source": "profiles/pa_valu_kernel-gemma4_12b_local_bf16-hbm_counters.txt", "kernel_sources": "ea299d4735d08495",
        "plan": {"kernel": 0, "rows": 2, "waves_per_group": 8, "splits": 1, "grid": 256, "balanced": 0, "pieces": 0, "queue": 0},
        "fetch_kib": 132874, "fetch_factor": 2.0, "write_kib": 256, "write_factor": 1.0},
    3: {"source": "profiles/pa_mfma_kernel-gemma4_12b_global_bf16-hbm_counters.txt", "kernel_sources": "25f2214b36e1fb52",
        "plan": {"kernel": 1, "rows": 16, "waves_per_group": 8, "splits": 57, "grid": 256, "balanced": 1, "pieces": 0, "queue": 0},
        "fetch_kib": 61373, "fetch_factor": 2.0, "write_kib": 4209, "write_factor": 1.0},
    4: {"source": "profiles/pa_mfma_kernel-gqa70b_int8kv-hbm_counters.txt", "kernel_sources": "25f2214b36e1fb52",
        "plan": {"kernel": 1, "rows": 8, "waves_per_group": 4, "splits": 4, "grid": 512, "balanced": 1, "pieces": 0, "queue": 0},
        "fetch_kib": 189700, "fetch_factor": 2.0, "write_kib": 3810, "write_factor": 1.0},
    5: {"source": "profiles/pa_mfma_kernel-verify5_bf16-hbm_counters.txt", "kernel_sources": "25f2214b36e1fb52",
        "plan": {"kernel": 1, "rows": 20, "waves_per_group": 4, "splits": 16, "grid": 512, "balanced": 2, "pieces": 4096, "queue": 1},
        "fetch_kib": 838642, "fetch_factor": 2.0, "write_kib": 35638, "write_factor": 1.0},
}
KERNEL_SOURCES = {0: ("pa_device.h", "pa_common.h", "pa_valu.hip"), 1: ("pa_device.h", "pa_common.h", "pa_mfma.hip")}


def kernel_sources_sha(kernel: int) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_kv_cache_94_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(config: int, plan: dict):
    m = MEASURED_TRAFFIC.get(config)
    if m is None or kernel_sources_sha(plan["kernel"]) != m["kernel_sources"]:
        return None
    if any(plan[k] != v for k, v in m["plan"].items()):
        return None
    return (m["fetch_kib"] * m["fetch_factor"] + m["write_kib"] * m["write_factor"]) * 1024
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 << 20         # Infinity Cache


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=0, choices=[0, 1, 2, 3, 4, 5],
                    help="0 (default): every workload, the speculative-verify step (5, the largest) as the "
                         "headline; 1-5: that workload alone")
    ap.add_argument("--copies", type=int, default=0,
                    help="cache copies rotated across steps (0: enough to exceed 4x the Infinity Cache)")
    ap.add_argument("--num-splits", type=int, default=0, help="force the context split count (0: library plan)")
    ap.add_argument("--tuning", default="",
                    help="launch-plan overrides (pa_tuning fields), e.g. partition=queue,pieces_per_wg=8; the record "
                         "notes them (experiments only: the library's own plan is the default)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the headline's oracle baseline")
    ap.add_argument("--cpu-seconds-others", type=float, default=3.0,
                    help="budget for the oracle baseline of each other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the KV append timing")
    ap.add_argument("--ring", action="store_true",
                    help="window workloads: lay each sequence's cache out as a ring of window/16 blocks")
    ap.add_argument("--head-scales", action="store_true", help="int8 workload: one scale per KV head")
    ap.add_argument("--prefill", type=int, default=0, choices=[0, 1, 2, 3],
                    help="time a paged prefill workload instead of a decode step (1 local layer, 2 global, 3 int8)")
    ap.add_argument("--event-every", type=int, default=0,
                    help="decode: stamp the attention kernel's dispatch with a HIP event pair on every Nth timed "
                         "step (0: every max(1, steps // 16)-th, so at least 10 samples from 10 steps on; a pair "
                         "on every step adds GPU and host time to each step)")
    ap.add_argument("--stamps", action="store_true",
                    help="load libpa_stamps.so (the same sources built with PA_STAMPS) and, after the timed steps, "
                         "record one launch's per-workgroup phase timestamps for each matrix-core workload")
    ap.add_argument("--ceiling", action="store_true",
                    help="after each workload's timed steps, stream its cache tiles with the load-only probe "
                         "(libpa_probe.so) on the same cache copies: the read rate this part gives that access "
                         "pattern, the kernel's practical ceiling")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy 3x (a known-size kernel for counter scaling)")
    return ap.parse_args()


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence.

    torch.cuda.Event records with a system-scope fence, which writes back and
    invalidates the caches at each record: ~4.5 us of GPU time per stamped
    step on MI355X, and a slower start for the kernel that follows (the
    Gemma4-like global-layer step, 16 sequences of 4K-32K tokens on one KV
    head, measured 29.2 us after one vs 26.8 us without). The
    event is made through the process's HIP runtime (the one torch loaded,
    which libpa's kernels also run on); only its handle is handed to libpa,
    whose launch stamps it from the kernel's own dispatch.
    """

    FLAGS = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)
    _hip = None

    def __init__(self, torch):
        import ctypes
        if TimingEvent._hip is None:
            torch.cuda.init()
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._torch = torch
        h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self) -> None:
        import ctypes
        stream = self._torch.cuda.current_stream().cuda_stream
        rc = TimingEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                  ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        # At interpreter shutdown the runtime may already be gone: nothing to release then.
        try:
            import ctypes
            if TimingEvent._hip is not None and getattr(self, "cuda_event", None):
                TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))
        except Exception:
            pass


def event_pair(torch):
    return TimingEvent(torch), TimingEvent(torch)


def host_cpu() -> str:
    """The host's CPU as lscpu names it (model name, family/model/stepping, sockets,
    cores, threads) and the logical CPUs this process may run on."""
    fields = {}
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    if "Model name" not in fields:
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        fields["Model name"] = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    desc = fields.get("Model name", "unknown CPU")
    ids = [f"{k.lower()} {fields[k]}" for k in ("CPU family", "Model", "Stepping") if k in fields]
    topo = [f"{fields[k]} {k.lower()}" for k in ("Socket(s)", "Core(s) per socket", "Thread(s) per core")
            if k in fields]
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    parts = [desc] + ([", ".join(ids)] if ids else []) + ([", ".join(topo)] if topo else [])
    return "; ".join(parts) + f"; {fields.get('CPU(s)', os.cpu_count())} logical CPUs, {usable} usable"


def time_steps(torch, np, calls, steps: int, every: int):
    """Launch `steps` steps back to back (call i % len(calls)); stamp every `every`-th.
    Returns (seconds per step, mean stamped kernel seconds, stamped kernel ms list)."""
    ev = {i: event_pair(torch) for i in range(0, steps, every)}
    for a, b in ev.values():   # materialise the underlying HIP events before handing their handles over
        a.record()
        b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % len(calls)].launch(timing=ev.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in ev.values()]
    return elapsed / steps, sum(kern_ms) / len(kern_ms) / 1e3, kern_ms


def measure_append(pa, accounting, torch, np, x, k, v, ks, vs, *, reps: int) -> dict:
    """Time pa_cache_write for the step's own tokens and for a prefill-sized chunk."""
    dev = k.device
    src = "f32" if x.kv_dtype == "f32" else "bf16"
    tdt = torch.float32 if src == "f32" else torch.bfloat16
    bs = 16
    step_slots = []
    R = x.ring_blocks
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        for pos in range(L - x.q_len, L):
            entry = (pos // bs) % R if R else pos // bs
            step_slots.append(int(x.block_table[b, entry]) * bs + pos % bs)
    rng = np.random.default_rng(1234)
    chunk = min(16384, x.num_blocks * bs)
    cases = {"step": np.asarray(step_slots, dtype=np.int64),
             "chunk": rng.permutation(x.num_blocks * bs)[:chunk].astype(np.int64)}
    out = {}
    for name, slots in cases.items():
        T = int(slots.size)
        kn = torch.randn((T, x.num_kv_heads, x.head_dim), device=dev).to(tdt)
        vn = kn if x.v_aliases_k else torch.randn_like(kn, dtype=torch.float32).to(tdt)
        sl = torch.from_numpy(slots).to(dev)
        for _ in range(3):
            pa.cache_write(kn, vn, sl, k, v, ks, vs)
        evs = [event_pair(torch) for _ in range(reps)]
        for a, b in evs:   # materialise the HIP events before the kernel stamps them
            a.record()
            b.record()
        torch.cuda.synchronize()
        for a, b in evs:
            pa.cache_write(kn, vn, sl, k, v, ks, vs, timing=(a, b))
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        mean = sum(us) / len(us)
        nbytes = accounting.append_bytes(T, num_kv_heads=x.num_kv_heads, head_dim=x.head_dim, src_dtype=src,
                                         kv_dtype=x.kv_dtype, v_shares_k=x.v_aliases_k)
        out[name] = {"tokens": T, "src_dtype": src, "alg_bytes": nbytes, "us_mean": mean,
                     "us_p50": us[len(us) // 2], "GBps": nbytes / (mean * 1e-6) / 1e9}
    return out


def measure_allocator(np, x, *, steps: int) -> dict:
    """Host microseconds per step of the block allocator for this batch (binding included)."""
    from paged_kv_cache_94_amd.allocator import BlockAllocator
    bs = 16
    grow = (steps + 20) * x.q_len
    need = int(sum(-(-(int(L) + grow) // bs) for L in x.seq_lens))
    al = BlockAllocator(need + x.batch, bs, prefix_cache=True)
    rng = np.random.default_rng(7)
    ids = list(range(x.batch))
    for b in ids:
        al.add(b, x.ring_blocks)
        al.append(b, int(x.seq_lens[b]), rng.integers(0, 32000, int(x.seq_lens[b])).astype(np.int32))
    mb = x.ring_blocks or int(-(-(int(x.seq_lens.max()) + grow) // bs))
    counts = [x.q_len] * x.batch
    toks = rng.integers(0, 32000, (steps + 20, x.batch * x.q_len)).astype(np.int32)
    for i in range(20):                      # warm up the binding and the allocator's tables
        al.append_batch(ids, counts, toks[steps + i])
        al.block_table(ids, mb)
    t0 = time.perf_counter()
    for i in range(steps):
        al.append_batch(ids, counts, toks[i])
        al.block_table(ids, mb)
    us = (time.perf_counter() - t0) / steps * 1e6
    al.close()
    return {"sequences": x.batch, "tokens_per_step": x.batch * x.q_len, "us_per_step": us,
            "what": "append_batch + block_table through the Python (ctypes) binding, host only; "
                    "the binding's call overhead dominates"}


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, published


def main_prefill(args) -> int:
    """One step = one pa_prefill call over the workload's packed chunks (inputs resident in HBM)."""
    import numpy as np
    import torch

    import paged_kv_cache_94_amd as pa
    from paged_kv_cache_94_amd import accounting
    from workloads import PREFILL_CONFIGS, make_prefill_config

    if not os.path.exists(pa.library_path()):
        from paged_kv_cache_94_amd import build
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = PREFILL_CONFIGS[args.prefill]
    x = make_prefill_config(args.prefill)
    acct = accounting.for_inputs(x)
    log(f"workload {x.name}: B={x.batch} chunk {cfg['chunk']} history {cfg['hist']} Hq={x.num_q_heads} "
        f"Hkv={x.num_kv_heads} D={x.head_dim} window={x.window} kv={x.kv_dtype}; "
        f"{acct['flops'] / 1e12:.3f} TFLOP per step")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, qs, lens, table = to_dev(x.q), to_dev(x.q_start), to_dev(x.seq_lens), to_dev(x.block_table)
    k = to_dev(x.k_pool)
    v = k if x.v_aliases_k else to_dev(x.v_pool)
    ks = None if x.k_scale is None else to_dev(x.k_scale)
    vs = None if x.v_scale is None else to_dev(x.v_scale)
    out = torch.empty_like(q)
    kw = dict(max_q_len=int(np.diff(x.q_start).max()), window=x.window, scale=x.scale, max_seq_len=x.max_seq_len,
              k_scale=ks, v_scale=vs)
    ev = [event_pair(torch) for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        pa.prefill(out, q, qs, k, v, table, lens, **kw)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        pa.prefill(out, q, qs, k, v, table, lens, timing=ev[i], **kw)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    kern_s = sum(kern_ms) / len(kern_ms) / 1e3
    tflops = acct["flops"] / kern_s / 1e12
    ms_per_step = elapsed / args.steps * 1e3
    value = acct["queries"] * args.steps / elapsed
    log(f"prefill kernel: mean {kern_s * 1e6:.1f} us -> {tflops:.1f} TFLOP/s = "
        f"{tflops / MFMA_BF16_PEAK_TFLOPS * 100:.1f}% of bf16 MFMA peak; step {ms_per_step * 1e3:.1f} us, "
        f"{value:.4g} query tokens/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle   # the CPU baseline leg is the only part of the benchmark that uses the oracle
        prob = oracle.Problem.from_inputs(x)
        threads = oracle.default_threads()
        rng = np.random.default_rng(0)
        total_rows = acct["queries"] * x.num_q_heads
        n, spent, done = 256, 0.0, 0
        while spent < args.cpu_seconds and done < total_rows:
            rows = rng.integers(0, total_rows, n).astype(np.int64)
            c0 = time.perf_counter()
            oracle.attention(prob, rows=rows, threads=threads)
            spent += time.perf_counter() - c0
            done += n
        cpu = {"value": done / x.num_q_heads / spent, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{done} (query token, head) rows drawn uniformly from the workload, fp64, "
                         f"{spent:.1f} s; value = rows/s / Hq"}
        log(f"cpu baseline: {cpu['value']:.4g} query tokens/s on {threads} threads")

    rec = {
        "metric": "paged prefill query tokens/s and matrix-core TFLOP/s (% of MI355X bf16 peak)",
        "value": value,
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if x.kv_dtype == "bf16" else "int8 cache, bf16 q",
        "data": "synthetic",
        "config": {"workload": f"{x.name}: B={x.batch}, chunk={cfg['chunk']}, history {cfg['hist']}, "
                               f"Hq={x.num_q_heads}, Hkv={x.num_kv_heads}, D={x.head_dim}, window={x.window} "
                               f"(seed {100 + args.prefill})",
                   "flops_per_step": acct["flops"], "kernel_us": kern_s * 1e6},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


CONFIG_ORDER = (5, 1, 2, 3, 4)   # the headline (largest single-GPU workload) first, then the others


def run_decode(idx: int, args, *, cpu_seconds: float, one_core: bool, extras: bool) -> dict:
    """Time the decode step of workload `idx` and return its record."""
    import numpy as np
    import torch

    import paged_kv_cache_94_amd as pa
    from paged_kv_cache_94_amd import accounting
    from workloads import CONFIGS, make_config

    dev = torch.device("cuda:0")
    cfg = CONFIGS[idx]
    t0 = time.time()
    x = make_config(idx, ring=args.ring, head_scales=args.head_scales)
    acct = accounting.for_inputs(x)
    log(f"[{idx}] workload {x.name}: B={x.batch} q_len={x.q_len} Hq={x.num_q_heads} Hkv={x.num_kv_heads} "
        f"D={x.head_dim} window={x.window} kv={x.kv_dtype} pool={x.num_blocks} blocks "
        f"(generated in {time.time() - t0:.1f}s)")
    log(f"[{idx}] algorithmic bytes/step {acct['alg_bytes'] / 1e6:.1f} MB, touched KV "
        f"{acct['touched_kv_bytes'] / 1e6:.1f} MB, flops/step {acct['flops'] / 1e9:.2f} G")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    copies = args.copies or max(1, min(8, math.ceil(4 * MALL_BYTES / max(1, acct["alg_bytes"]))))
    q = to_dev(x.q)
    lens = to_dev(x.seq_lens)
    k0 = to_dev(x.k_pool)
    v0 = k0 if x.v_aliases_k else to_dev(x.v_pool)
    ks0 = None if x.k_scale is None else to_dev(x.k_scale)
    vs0 = None if x.v_scale is None else (ks0 if x.v_scale is x.k_scale else to_dev(x.v_scale))
    table0 = to_dev(x.block_table)
    entry = "verify" if x.q_len > 1 else ("decode_int8" if x.kv_dtype == "int8" else "decode")
    out = torch.empty_like(q)
    calls = []
    for c in range(copies):
        if c == 0:
            k, v, ks, vs, table = k0, v0, ks0, vs0, table0
        else:
            k = torch.empty_like(k0).copy_(k0)
            v = k if x.v_aliases_k else torch.empty_like(v0).copy_(v0)
            ks = None if ks0 is None else torch.empty_like(ks0).copy_(ks0)
            vs = None if vs0 is None else (ks if vs0 is ks0 else torch.empty_like(vs0).copy_(vs0))
            table = table0.clone()
        calls.append(pa.Prepared(entry, out, q, k, v, table, lens, window=x.window, scale=x.scale,
                                 max_seq_len=x.max_seq_len, k_scale=ks, v_scale=vs, num_splits=args.num_splits,
                                 ring_blocks=x.ring_blocks, tuning=tuning_of(args, x)))
    plan = pa.plan(q, k0, v0, table0, lens, window=x.window, scale=x.scale, max_seq_len=x.max_seq_len,
                   k_scale=ks0, v_scale=vs0, num_splits=args.num_splits, ring_blocks=x.ring_blocks,
                   tuning=tuning_of(args, x))
    log(f"[{idx}] plan: {plan}; {copies} cache copies rotated")

    # The timed steps run back to back; every `every`-th one also carries a
    # pair of HIP events stamped by the attention kernel's own dispatch
    # (hipExtLaunchKernel), whose mean is the kernel duration below.
    every = args.event_every or max(1, args.steps // 16)
    for i in range(args.warmup):
        calls[i % copies].launch()
    torch.cuda.synchronize()
    step_s, kern_s, kern_ms = time_steps(torch, np, calls, args.steps, every)
    elapsed = step_s * args.steps
    srt = sorted(kern_ms)
    pct = {k: srt[min(len(srt) - 1, int(f * len(srt)))] * 1e3 for k, f in (("p10", 0.1), ("p50", 0.5), ("p90", 0.9))}
    queries = acct["queries"]
    value = queries * args.steps / elapsed
    achieved = acct["alg_bytes"] / kern_s / 1e9
    step_gbs = acct["alg_bytes"] / step_s / 1e9
    log(f"[{idx}] attention kernel: mean {kern_s * 1e6:.2f} us over {len(kern_ms)} stamped steps (p10 "
        f"{pct['p10']:.2f}, median {pct['p50']:.2f}, p90 {pct['p90']:.2f}) -> {achieved:.0f} GB/s = "
        f"{achieved / HBM_PEAK_GBS * 100:.1f}% of peak; whole step {step_s * 1e6:.2f} us -> {step_gbs:.0f} GB/s, "
        f"{value:.4g} queries/s")

    traffic = None if (args.ring or args.head_scales or args.num_splits or args.stamps) else \
        measured_traffic(idx, plan)
    stamps = phase_stamps(torch, calls[0], plan, kern_s, acct["alg_bytes"]) if args.stamps and plan["kernel"] == 1 \
        else None
    rec = {
        "workload": f"{x.name}: B={x.batch}, q_len={x.q_len}, Hq={x.num_q_heads}, Hkv={x.num_kv_heads}, "
                    f"D={x.head_dim}, block=16, window={x.window}, kv={x.kv_dtype}, lens {cfg['lens']} "
                    f"(seed {idx})",
        "batch": x.batch,
        "q_len": x.q_len,
        "dtype": {"f32": "f32", "bf16": "bf16", "int8": "int8 cache, bf16 q"}[x.kv_dtype],
        "alg_bytes_per_step": acct["alg_bytes"],
        "queries_per_step": queries,
        "kernel": ("pa_valu_kernel" if plan["kernel"] == 0 else "pa_mfma_kernel"),
        "kernel_us": {"mean": kern_s * 1e6, **pct},
        "kernel_stamped_steps": len(kern_ms),
        "achieved_GBps": achieved,
        "frac": achieved / HBM_PEAK_GBS,
        "step_us": step_s * 1e6,
        "step_GBps": step_gbs,
        "queries_per_s": value,
        "ms_per_step": step_s * 1e3,
        "plan": {k: plan[k] for k in ("kernel", "rows", "waves_per_group", "splits", "grid", "balanced", "pieces",
                                      "queue")},
        "tuning": tuning_of(args, x),
        "cache_copies": copies,
        "traffic": traffic,
        "traffic_source": (MEASURED_TRAFFIC[idx]["source"] if traffic is not None else
                           "null: no counter pass matches these kernel sources and this plan"),
    }
    if stamps is not None:
        rec["stamps"] = stamps
        log_stamps(idx, stamps)
    if args.ceiling:
        rec["ceiling"] = read_ceiling(torch, np, x, calls, args.steps, kern_s)
        c = rec["ceiling"]
        log(f"[{idx}] read ceiling: {c['kv_bytes'] / 1e6:.1f} MB of cache tiles; " +
            "; ".join(f"{r['workgroups']}x{r['waves']}w depth {r['depth']}: {r['us']:.2f} us = {r['TBps']:.2f} TB/s"
                      for r in c["runs"]) +
            f"; the attention kernel reads them at {c['kernel_TBps']:.2f} TB/s = {c['kernel_share']:.1%} of the best")

    if extras:
        # Warm: every step re-reads the same cache copy, so the Infinity Cache
        # (256 MB) can serve what of it fits. Reported beside the cold figures, never as them.
        if copies > 1:
            wsteps = max(8, args.steps // 2)
            w_step, w_kern, _ = time_steps(torch, np, calls[:1], wsteps, every)
            rec["warm"] = {"what": "every step re-reads one cache copy (the Infinity Cache may hold part of it)",
                           "steps": wsteps, "kernel_us": w_kern * 1e6, "ms_per_step": w_step * 1e3,
                           "queries_per_s": queries / w_step, "kernel_GBps": acct["alg_bytes"] / w_kern / 1e9}
            log(f"[{idx}] warm (one cache copy): attention kernel {w_kern * 1e6:.2f} us, step {w_step * 1e6:.2f} us")
        rec["block_allocator"] = measure_allocator(np, x, steps=200)
        log(f"[{idx}] block allocator: {rec['block_allocator']['us_per_step']:.1f} us of host time per step")
        if not args.no_append:
            rec["kv_append"] = measure_append(pa, accounting, torch, np, x, k0, v0, ks0, vs0, reps=50)
            for name, r in rec["kv_append"].items():
                log(f"[{idx}] kv append ({name}): {r['tokens']} tokens {r['src_dtype']} -> {x.kv_dtype}: "
                    f"{r['us_mean']:.2f} us -> {r['GBps']:.0f} GB/s")

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[{idx}] copy calibration: 3 x 1 GiB device-to-device copies done")

    del calls, out, q, lens, k0, v0, ks0, vs0, table0, k, v, ks, vs, table
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(np, x, queries, cpu_seconds=cpu_seconds, one_core=one_core)
        log(f"[{idx}] cpu baseline: {rec['cpu_baseline']['value']:.4g} queries/s on "
            f"{rec['cpu_baseline']['cores']} threads")
    return rec


STAMP_TICKS_PER_US = 100.0   # s_memrealtime counts at 100 MHz on MI300-class parts (checked against events below)


def phase_stamps(torch, call, plan: dict, kern_s: float, alg_bytes: int) -> dict:
    """One launch with the phase stamps of libpa_stamps.so on; per-workgroup phase statistics in us.

    Slots per workgroup (include/pa.h, pa_args.debug_stamps): 0 entry, 1 partition known, 2 exit,
    3 segment count, then per segment s at 4 + 5s: start, first block consumed, block loop done,
    result written, block count. Times are from the earliest workgroup entry. stream_TBps: the
    algorithmic bytes spread over each segment's [start, block loop done] in proportion to its
    blocks, summed over workgroups in 5 us bins -- the rate at which the kernel pulls its data.
    """
    import numpy as np
    slots = 64
    buf = torch.zeros(plan["grid"] * slots, dtype=torch.int64, device="cuda")
    call.args.debug_stamps = buf.data_ptr()
    ev = event_pair(torch)
    for a in ev:
        a.record()
    for _ in range(2):
        buf.zero_()
        call.launch(timing=ev)
    torch.cuda.synchronize()
    call.args.debug_stamps = None
    st = buf.view(plan["grid"], slots).cpu().numpy().astype(np.int64)
    kern_us = ev[0].elapsed_time(ev[1]) * 1e3
    t0 = st[:, 0].min()
    us = (st - t0) / STAMP_TICKS_PER_US
    per_seg = 5
    nseg = np.minimum(st[:, 3], (slots - 4) // per_seg)
    starts, streams, merges, gaps, firsts, spans = [], [], [], [], [], []
    for w in range(st.shape[0]):
        n = int(nseg[w])
        raw = st[w, 4:4 + per_seg * n].reshape(n, per_seg) if n else np.zeros((0, per_seg), dtype=np.int64)
        seg = us[w, 4:4 + per_seg * n].reshape(n, per_seg) if n else np.zeros((0, per_seg))
        for k in range(n):
            spans.append((seg[k, 0], seg[k, 2], int(raw[k, 4])))
        starts.append(float((seg[:, 1] - seg[:, 0]).sum()))
        streams.append(float((seg[:, 2] - seg[:, 1]).sum()))
        merges.append(float((seg[:, 3] - seg[:, 2]).sum()))
        gaps.append(float((seg[1:, 0] - seg[:-1, 3]).sum()) if n > 1 else 0.0)
        if n:
            firsts.append(float(seg[0, 1]))

    def q(v):
        v = np.sort(np.asarray(v, dtype=np.float64))
        if v.size == 0:
            return None
        return {"p10": float(v[int(0.1 * (v.size - 1))]), "p50": float(v[int(0.5 * (v.size - 1))]),
                "p90": float(v[int(0.9 * (v.size - 1))]), "max": float(v[-1])}

    span_us = float(us[:, 2].max())
    # Streaming rate over time: each segment's share of the bytes, spread over [start, loop done].
    total_blocks = sum(b for _, _, b in spans) or 1
    bin_us = 5.0
    bins = np.zeros(int(span_us // bin_us) + 2)
    for t0s, t1s, blocks in spans:
        nbytes = alg_bytes * blocks / total_blocks
        a, b = max(0.0, t0s), max(t0s + 1e-3, t1s)
        i0, i1 = int(a // bin_us), int(b // bin_us)
        for i in range(i0, i1 + 1):
            lo, hi = max(a, i * bin_us), min(b, (i + 1) * bin_us)
            if hi > lo:
                bins[i] += nbytes * (hi - lo) / (b - a)
    rate = [round(float(x) / (bin_us * 1e-6) / 1e12, 2) for x in bins]
    return {
        "what": "one launch of libpa_stamps.so (same sources, PA_STAMPS); us from the first workgroup entry",
        "kernel_us_events": kern_us, "span_us_stamps": span_us,
        "stamp_rate_check": span_us / kern_us if kern_us > 0 else None,
        "workgroups": int(st.shape[0]), "segments_per_wg": q(nseg),
        "entry": q(us[:, 0]), "partition_known": q(us[:, 1]), "first_block_consumed": q(firsts), "exit": q(us[:, 2]),
        "sum_segment_starts": q(starts), "sum_streaming": q(streams), "sum_merges_and_writes": q(merges),
        "sum_between_segments": q(gaps),
        "stream_TBps_per_5us": rate,
    }


def log_stamps(idx: int, s: dict) -> None:
    log(f"[{idx}] phase stamps ({s['workgroups']} workgroups; kernel {s['kernel_us_events']:.1f} us by events, "
        f"{s['span_us_stamps']:.1f} us by stamps), us from the first entry: p10 / p50 / p90 / max")
    for key in ("segments_per_wg", "entry", "partition_known", "first_block_consumed", "exit", "sum_segment_starts",
                "sum_streaming", "sum_merges_and_writes", "sum_between_segments"):
        v = s[key]
        if v is not None:
            log(f"[{idx}]   {key:24s} {v['p10']:8.2f} {v['p50']:8.2f} {v['p90']:8.2f} {v['max']:8.2f}")
    log(f"[{idx}]   streaming TB/s per 5 us: {' '.join(f'{x:.1f}' for x in s['stream_TBps_per_5us'])}")


def tuning_of(args, x):
    """The --tuning overrides as a dict (None without any); they apply to the matrix-core workloads only."""
    if not args.tuning:
        return None
    mfma = x.kv_dtype == "int8" or (x.kv_dtype == "bf16" and x.num_q_heads // x.num_kv_heads * x.q_len > 512 // x.head_dim)
    if not mfma:
        return None
    out = {}
    for item in args.tuning.split(","):
        k, v = item.split("=")
        out[k.strip()] = v.strip() if k.strip() == "partition" else int(v)
    return out


def tile_list(np, x):
    """The (block, KV head) tiles one step reads, as ids phys * Hkv + g, in (sequence, KV head, block) order."""
    ids = []
    R = x.ring_blocks
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        lo = max(0, L - x.q_len - x.window + 1) if x.window > 0 else 0
        blocks = np.arange(lo // 16, (L - 1) // 16 + 1)
        phys = x.block_table[b, (blocks % R) if R else blocks].astype(np.int64)
        for g in range(x.num_kv_heads):
            ids.append(phys * x.num_kv_heads + g)
    return np.concatenate(ids).astype(np.int32) if ids else np.zeros(0, dtype=np.int32)


def read_ceiling(torch, np, x, calls, steps: int, kern_s: float) -> dict:
    """Stream the step's cache tiles with the load-only probe (libpa_probe.so), rotating over the cache copies."""
    import ctypes
    from paged_kv_cache_94_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build(variants=("probe",))
    lib = ctypes.CDLL(build.PROBE_LIB)
    V, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.pa_probe_read.argtypes = [V, V, V, I32, I32, I32, I32, I32, I32, V, V, V, V]
    lib.pa_probe_read.restype = ctypes.c_int
    tiles_h = tile_list(np, x)
    tiles = torch.from_numpy(tiles_h).to("cuda")
    elem = {"f32": 4, "bf16": 2, "int8": 1}[x.kv_dtype]
    row_bytes = x.head_dim * elem
    two = not x.v_aliases_k
    kv_bytes = int(tiles_h.size) * 16 * row_bytes * (2 if two else 1)
    pools = [(c._keep[2], c._keep[3]) for c in calls]
    runs = []
    for wgs, waves, depth in ((512, 4, 2), (256, 8, 2), (512, 4, 3)):
        sink = torch.empty(wgs * waves * 64, dtype=torch.int32, device="cuda")
        n = max(8, min(steps, 40))
        evs = [event_pair(torch) for _ in range(n)]
        for a, b in evs:
            a.record()
            b.record()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream().cuda_stream
        for i in range(-2, n):   # two untimed warm-up launches
            k, v = pools[i % len(pools)]
            ev = evs[i] if i >= 0 else (None, None)
            rc = lib.pa_probe_read(k.data_ptr(), v.data_ptr() if two else None, tiles.data_ptr(), int(tiles_h.size),
                                   row_bytes, x.num_kv_heads, wgs, waves, depth, sink.data_ptr(),
                                   ev[0].cuda_event if ev[0] else None, ev[1].cuda_event if ev[1] else None, stream)
            if rc != 0:
                raise RuntimeError(f"pa_probe_read failed ({rc})")
        torch.cuda.synchronize()
        us = sum(a.elapsed_time(b) for a, b in evs) / n * 1e3
        runs.append({"workgroups": wgs, "waves": waves, "depth": depth, "us": us, "TBps": kv_bytes / us / 1e6})
    best = max(r["TBps"] for r in runs)
    kernel_tbps = kv_bytes / kern_s / 1e12
    return {"what": "load-only probe over the same cache tiles and copies: each cached row read front to back in "
                    "16-byte non-temporal pieces, as the matrix-core kernel loads them; KV bytes only",
            "kv_bytes": kv_bytes, "tiles": int(tiles_h.size), "runs": runs, "best_TBps": best,
            "kernel_TBps": kernel_tbps, "kernel_share": kernel_tbps / best}


def cpu_baseline(np, x, queries: int, *, cpu_seconds: float, one_core: bool) -> dict:
    """The fp64 oracle on the host's cores over the same batch (a baseline, not the target)."""
    import oracle   # the CPU baseline leg is the only part of the benchmark that uses the oracle
    prob = oracle.Problem.from_inputs(x)
    threads = oracle.default_threads()
    reps, spent = 0, 0.0
    while reps < 1 or spent < cpu_seconds:
        c0 = time.perf_counter()
        oracle.attention(prob, threads=threads)
        spent += time.perf_counter() - c0
        reps += 1
        if reps >= 1000:
            break
    cpu = {"value": queries * reps / spent, "unit": "queries/s", "cores": threads, "kind": "oracle",
           "sample": f"the whole {x.name} batch ({x.batch} sequences x {x.q_len} query token(s), all "
                     f"{x.num_q_heads} heads), fp64, repeated {reps} times in {spent:.1f} s",
           "host_cpu": host_cpu()}
    if one_core and threads > 1:
        # The same oracle on one core, over a bounded slice of the batch's rows.
        rows_total = queries * x.num_q_heads
        rng = np.random.default_rng(0)
        n1, spent1, done1 = 64, 0.0, 0
        while spent1 < cpu_seconds / 3 and done1 < rows_total:
            rows = rng.integers(0, rows_total, n1).astype(np.int64)
            c0 = time.perf_counter()
            oracle.attention(prob, rows=rows, threads=1)
            spent1 += time.perf_counter() - c0
            done1 += n1
        cpu["one_core"] = {"value": done1 / x.num_q_heads / spent1, "unit": "queries/s", "cores": 1,
                           "sample": f"{done1} (query, head) rows drawn uniformly from the batch, fp64, "
                                     f"{spent1:.1f} s; value = rows/s / Hq"}
    return cpu


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "decode attention shards by sequence or KV head with no exchange, so a multi-GPU figure "
              "would be N independent copies of this one.", file=sys.stderr)
        return 2

    if args.prefill:
        return main_prefill(args)
    if (args.ring or args.head_scales) and args.config == 0:
        print("--ring and --head-scales apply to one workload: pass --config 2 (ring) or 4 (head scales)",
              file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_94_amd as pa
    from paged_kv_cache_94_amd import _lib, build

    if args.stamps:
        if not os.path.exists(build.STAMPS_LIB):
            build.build(variants=("stamps",))
        _lib.load(build.STAMPS_LIB)   # every call of this process goes to the stamps build
        log(f"loaded {build.STAMPS_LIB}")
    elif not os.path.exists(pa.library_path()):
        build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(torch.device("cuda:0"))

    order = CONFIG_ORDER if args.config == 0 else (args.config,)
    head = order[0]
    recs = {}
    for idx in order:
        cpu_s = 0.0 if args.no_cpu_baseline else (args.cpu_seconds if idx == head else args.cpu_seconds_others)
        recs[idx] = run_decode(idx, args, cpu_seconds=cpu_s, one_core=idx == head, extras=idx == head)
    h = recs[head]

    roofline = {"bound": "hbm", "kernel": h["kernel"], "achieved": h["achieved_GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": h["frac"], "traffic": h["traffic"], "traffic_source": h["traffic_source"]}
    config = {"workload": h["workload"], "batch": h["batch"], "q_len": h["q_len"],
              "alg_bytes_per_step": h["alg_bytes_per_step"], "kernel_us": h["kernel_us"],
              "kernel_stamped_steps": h["kernel_stamped_steps"], "step_GBps": h["step_GBps"],
              "cache_copies": h["cache_copies"], "plan": h["plan"]}
    if len(order) > 1:
        # Every workload of the set, timed in this same run (the headline's own entry included).
        keep = ("workload", "dtype", "alg_bytes_per_step", "kernel", "kernel_us", "kernel_stamped_steps",
                "achieved_GBps", "frac", "step_us", "step_GBps", "queries_per_s", "plan", "cache_copies", "traffic",
                "traffic_source", "cpu_baseline")
        config["configs"] = {f"C{i}": {k: recs[i][k] for k in keep if k in recs[i]} for i in sorted(recs)}
    rec = {
        "metric": METRIC,
        "value": h["queries_per_s"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": h.get("cpu_baseline"),
        "warm": h.get("warm"),
        "kv_append": h.get("kv_append"),
        "block_allocator": h.get("block_allocator"),
    }
    if args.ceiling:
        rec["ceiling"] = {f"C{i}": recs[i]["ceiling"] for i in sorted(recs) if "ceiling" in recs[i]}
    if args.stamps:
        rec["stamps"] = {f"C{i}": recs[i]["stamps"] for i in sorted(recs) if "stamps" in recs[i]}
        rec["library"] = "libpa_stamps.so (diagnostic build with phase stamps)"
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
