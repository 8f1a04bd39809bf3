"""A prepared decode step captured in a HIP graph and replayed.

A serving loop marshals a step once (``pa.Prepared``) and replays it from a
graph. The library allocates nothing and issues no memset in a call, and the
piece queue returns its counters to zero itself, so the captured kernels must
give the same results on every replay. Each case captures one launch, then
replays it several times. Before each replay the queries are replaced with
new contents and the output is poisoned, both by eager work on the same
stream, with a synchronisation after each replay. Every replay is compared
with the oracle for the queries it saw, and with an eager launch of the same
step.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_94_amd as pa
from tests.gpu_util import TOL, Dev, max_err, to_torch
from workloads import make_inputs

pytestmark = pytest.mark.gpu
REPLAYS = 4


def _case(name):
    rng = np.random.default_rng(11)
    if name == "queue":             # many units: pieces handed out through the device queue
        lens = np.clip(np.round(np.exp(rng.normal(np.log(300), 0.8, 160))), 16, 3000).astype(int)
        return make_inputs(lens, q_len=1, num_q_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                           kv_dtype="bf16", seed=21, poison=True), {}, dict(queue=1)
    if name == "splits":            # forced context splits, merged by the combine kernel
        return make_inputs([700, 2000, 33, 1200], q_len=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                           q_dtype="bf16", kv_dtype="bf16", seed=22, poison=True), dict(num_splits=4), dict(balanced=0)
    if name == "vector":            # fp32, small groups: the vector kernel
        return make_inputs([37, 500, 129, 16], q_len=1, num_q_heads=8, num_kv_heads=4, head_dim=64, q_dtype="f32",
                           kv_dtype="f32", window=100, seed=23, poison=True), {}, dict(kernel=0)
    return make_inputs([60, 900, 2500, 17, 400], q_len=1, num_q_heads=64, num_kv_heads=8, head_dim=128,
                       q_dtype="bf16", kv_dtype="int8", seed=24, poison=True), {}, dict(kernel=1)


def _entry(x):
    return "verify" if x.q_len > 1 else ("decode_int8" if x.kv_dtype == "int8" else "decode")


@pytest.mark.parametrize("name", ["queue", "splits", "vector", "int8"])
def test_graph_replays_match_eager_and_oracle(name):
    x, call_kw, plan_expect = _case(name)
    dev = Dev(x)
    plan = dev.plan(**call_kw)
    print(f"graph {name}: plan {plan}", flush=True)
    for k, v in plan_expect.items():
        assert plan[k] == v, (k, plan)
    if name == "splits":
        assert plan["splits"] > 1

    out = torch.full_like(dev.q, float("nan"))
    prep = pa.Prepared(_entry(x), out, dev.q, dev.k, dev.v, dev.table, dev.lens, window=x.window, scale=x.scale,
                       max_seq_len=x.max_seq_len, k_scale=dev.ks, v_scale=dev.vs, **call_kw)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        prep.launch()                # warm-up outside the capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        prep.launch()

    rows = None
    n_rows = x.q.shape[0] * x.q.shape[1] * x.q.shape[2]
    if n_rows > 2000:
        rows = np.random.default_rng(5).choice(n_rows, size=2000, replace=False).astype(np.int64)
    for r in range(REPLAYS):
        q_host = np.roll(x.q, shift=r + 1, axis=0) if r % 2 == 0 else np.roll(x.q, shift=r, axis=2)
        with torch.cuda.stream(stream):
            dev.q.copy_(to_torch(q_host))
            out.fill_(float("nan"))
            graph.replay()
        stream.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        with torch.cuda.stream(stream):
            out.fill_(float("nan"))
            prep.launch()
        stream.synchronize()
        eager = out.float().cpu().numpy().astype(np.float64)
        xr = dataclasses.replace(x, q=np.ascontiguousarray(q_host))
        ref = oracle.attention(oracle.Problem.from_inputs(xr), rows=rows)
        flat = got.reshape(-1, x.head_dim)
        assert not np.isnan(got).any(), r
        err = max_err(flat if rows is None else flat[rows], ref.reshape(-1, x.head_dim))
        print(f"graph {name}: replay {r} max|err| vs oracle {err:.3g}, vs eager {max_err(got, eager):.3g}", flush=True)
        assert err <= TOL[x.kv_dtype], (r, err)
        assert max_err(got, eager) <= TOL[x.kv_dtype], r
