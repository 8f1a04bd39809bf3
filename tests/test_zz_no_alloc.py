"""pa_verify_noalloc (the library's static scratch array) against pa_verify (a caller workspace).

Both run the same plan and kernels, so their outputs must agree bit for bit;
both are also held to the fp64 oracle's tolerance on sampled rows. Two calls
in a row share the scratch array, the second on a smaller input with a
different partition, and a third needs no workspace at all.
"""

from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_94_amd as pa
from tests.gpu_util import TOL, Dev, max_err
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _both(x, **kw):
    dev = Dev(x)
    args = dict(window=x.window, scale=x.scale, max_seq_len=x.max_seq_len, k_scale=dev.ks, v_scale=dev.vs, **kw)
    ref_out = torch.full_like(dev.q, float("nan"))
    pa.verify(ref_out, dev.q, dev.k, dev.v, dev.table, dev.lens, **args)
    out = torch.full_like(dev.q, float("nan"))
    pa.verify_noalloc(out, dev.q, dev.k, dev.v, dev.table, dev.lens, **args)
    torch.cuda.synchronize()
    return dev.plan(**kw), out.float().cpu().numpy().astype(np.float64), ref_out.float().cpu().numpy().astype(np.float64)


def _sampled_rows(x, n, seed):
    total = x.batch * x.q_len * x.num_q_heads
    return np.unique(np.random.default_rng(seed).integers(0, total, n)).astype(np.int64)


def test_noalloc_matches_verify_on_consecutive_calls():
    # Call 1: 300 verify sequences, pieces handed out through the queue in the scratch array.
    lens = np.random.default_rng(1).integers(16, 3000, 300).tolist()
    big = make_inputs(lens, q_len=5, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
                      poison=True, seed=zlib.crc32(b"noalloc-big"))
    plan, got, ref = _both(big)
    _log(f"call 1: plan {plan}")
    assert plan["queue"] == 1 and 0 < plan["workspace_bytes"] <= 64 << 20
    assert not np.isnan(got).any()
    np.testing.assert_array_equal(got, ref)
    rows = _sampled_rows(big, 3000, 2)
    o = oracle.attention(oracle.Problem.from_inputs(big), rows=rows)
    assert max_err(got.reshape(-1, big.head_dim)[rows], o.reshape(-1, big.head_dim)) <= TOL["bf16"]

    # Call 2, right after on the same scratch: a smaller global-layer problem cut into one piece per
    # workgroup (asked for through the tuning).
    small = make_inputs([3000, 700, 4100], q_len=1, num_q_heads=16, num_kv_heads=1, head_dim=256, q_dtype="bf16",
                        kv_dtype="bf16", alias_v=True, poison=True, seed=zlib.crc32(b"noalloc-small"))
    plan2, got2, ref2 = _both(small, tuning={"partition": "pieces"})
    _log(f"call 2: plan {plan2}")
    assert plan2["balanced"] == 2 and plan2["queue"] == 0 and 0 < plan2["workspace_bytes"] < plan["workspace_bytes"]
    np.testing.assert_array_equal(got2, ref2)
    assert max_err(got2, oracle.attention(oracle.Problem.from_inputs(small))) <= TOL["bf16"]

    # Call 3: the queue again after the pieces partition (its counters must still start at zero).
    plan3, got3, ref3 = _both(big)
    assert plan3["queue"] == 1
    np.testing.assert_array_equal(got3, got)


def test_noalloc_int8_and_unsplit_calls():
    x = make_inputs([90, 300, 17, 1500], q_len=1, num_q_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                    kv_dtype="int8", poison=True, seed=zlib.crc32(b"noalloc-int8"))
    plan, got, ref = _both(x)
    assert plan["workspace_bytes"] > 0
    np.testing.assert_array_equal(got, ref)
    assert max_err(got, oracle.attention(oracle.Problem.from_inputs(x))) <= TOL["int8"]
    # The tiny fp32 problem needs no workspace: the scratch array is not touched.
    y = make_inputs([37, 70], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="f32", kv_dtype="f32",
                    poison=True, seed=3)
    plan, got, ref = _both(y)
    assert plan["workspace_bytes"] == 0
    np.testing.assert_array_equal(got, ref)
    assert max_err(got, oracle.attention(oracle.Problem.from_inputs(y))) <= TOL["f32"]
