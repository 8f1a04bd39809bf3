"""Calls on a stream other than torch's current one, and the queue-header check.

The binding allocates and zero-fills a call's workspace on the stream the
kernels run on. The piece queue needs that workspace's header at zero when
its kernel starts. Here the current stream is kept busy with a long matrix
product while the call goes to a side stream: a fill queued behind that
product would still be pending when the side stream's kernel claims its
first pieces. Outputs must match the fp64 oracle.
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

QUEUE = {"partition": "queue"}


def _verify_case(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(16, 2000, 40).tolist()
    return make_inputs(lens, q_len=5, num_q_heads=32, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                       kv_dtype="bf16", poison=True, seed=seed)


def _busy_current_stream():
    a = torch.randn(6144, 6144, device="cuda")
    return a @ a   # a few ms of work queued on the current stream


def test_queue_partition_on_a_side_stream():
    x = _verify_case(zlib.crc32(b"side-stream"))
    dev = Dev(x)
    assert dev.plan(tuning=QUEUE)["queue"] == 1
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    side = torch.cuda.Stream()
    for _ in range(3):
        out = torch.full_like(dev.q, float("nan"))
        torch.cuda.synchronize()
        busy = _busy_current_stream()
        pa.verify(out, dev.q, dev.k, dev.v, dev.table, dev.lens, window=x.window, scale=x.scale,
                  max_seq_len=x.max_seq_len, stream=side, tuning=QUEUE)
        side.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        del busy
        torch.cuda.synchronize()
        assert not np.isnan(got).any()
        assert max_err(got, ref) <= TOL["bf16"]


def test_prepared_call_launched_on_a_side_stream():
    x = _verify_case(zlib.crc32(b"prepared-side"))
    dev = Dev(x)
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    out = torch.full_like(dev.q, float("nan"))
    call = pa.Prepared("verify", out, dev.q, dev.k, dev.v, dev.table, dev.lens, window=x.window, scale=x.scale,
                       max_seq_len=x.max_seq_len, tuning=QUEUE)
    side = torch.cuda.Stream()
    for _ in range(2):
        busy = _busy_current_stream()
        call.launch(stream=side)
        side.synchronize()
        del busy
        got = out.float().cpu().numpy().astype(np.float64)
        assert max_err(got, ref) <= TOL["bf16"]
        out.fill_(float("nan"))
        torch.cuda.synchronize()


def test_validate_flags_a_queue_header_that_is_not_zero():
    x = _verify_case(zlib.crc32(b"queue-header"))
    dev = Dev(x)
    need = dev.plan(tuning=QUEUE)["workspace_bytes"]
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    kw = dict(window=x.window, max_seq_len=x.max_seq_len, workspace=ws)
    st = pa.validate(dev.q, dev.k, dev.v, dev.table, dev.lens, tuning=QUEUE, **kw)
    assert st.cpu().tolist() == [0] * (x.batch + 1)
    # A "done" counter left behind (shard 3: int32 index 16 * (8 + 3)).
    ws.view(torch.int32)[16 * 11] = 2
    st = pa.validate(dev.q, dev.k, dev.v, dev.table, dev.lens, tuning=QUEUE, **kw).cpu().tolist()
    assert st[0] == pa.BAD_WORKSPACE and st[1:] == [0] * x.batch
    # A plan that does not use the queue does not look at the header.
    st = pa.validate(dev.q, dev.k, dev.v, dev.table, dev.lens, tuning={"partition": "list"}, **kw).cpu().tolist()
    assert st[0] == 0
    # Once the counters are back at zero the call itself is correct on this workspace.
    ws.zero_()
    got = dev.run_f64(workspace=ws, tuning=QUEUE)
    assert max_err(got, oracle.attention(oracle.Problem.from_inputs(x))) <= TOL["bf16"]
    assert not ws[:4096].any().item()
