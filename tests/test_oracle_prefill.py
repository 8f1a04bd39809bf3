"""Pins for the oracle's prefill (packed, per-sequence query counts), CPU only.

A prefill chunk (Lab 5, "Flash Attention": q_len > 1 with the sequence's
history already in the cache) is checked against torch's float64
scaled_dot_product_attention on contiguous copies with an explicit causal /
window band mask, sequence by sequence, and against the oracle's own
uniform-q_len path run on each sequence alone (bit-identical: the same
rows with the same keys).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests.refs import dense_sdpa_packed
from workloads import make_inputs

# (history lens, q_lens, Hq, Hkv, D, window, q_dtype, kv_dtype)
CASES = [
    ([0, 10, 33], [37, 5, 16], 4, 2, 64, 0, "f32", "f32"),
    ([0, 0, 100], [1, 64, 70], 8, 1, 128, 0, "bf16", "bf16"),
    ([5, 200, 17], [90, 33, 0], 8, 2, 64, 40, "bf16", "bf16"),
    ([64, 3], [48, 129], 16, 2, 128, 0, "bf16", "int8"),
    ([300], [100], 6, 3, 64, 16, "f32", "f32"),
]


def _case(c, seed, **kw):
    hist, ql, hq, hkv, d, w, qd, kd = c
    lens = [h + q for h, q in zip(hist, ql)]
    return make_inputs(lens, q_len=1, q_lens=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_dtype=qd,
                       kv_dtype=kd, window=w, seed=seed, poison=True, **kw)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_prefill_matches_torch_sdpa(i):
    x = _case(CASES[i], 300 + i)
    got = oracle.attention(oracle.Problem.from_inputs(x))
    assert got.shape == x.q.shape and not np.isnan(got).any()
    np.testing.assert_allclose(got, dense_sdpa_packed(x), rtol=0, atol=1e-12)


@pytest.mark.parametrize("i", range(len(CASES)))
def test_prefill_equals_each_sequence_alone(i):
    x = _case(CASES[i], 400 + i)
    got = oracle.attention(oracle.Problem.from_inputs(x))
    for b in range(x.batch):
        a, e = int(x.q_start[b]), int(x.q_start[b + 1])
        if e == a:
            continue
        one = oracle.Problem(x.q[a:e][None], x.k_pool, x.v_pool, x.block_table[b:b + 1], x.seq_lens[b:b + 1],
                             q_len=e - a, window=x.window, scale=x.scale, k_scale=x.k_scale, v_scale=x.v_scale)
        assert oracle.attention(one)[0].tobytes() == got[a:e].tobytes()


def test_prefill_rows_subset_and_visits():
    x = _case(CASES[2], 7)
    p = oracle.Problem.from_inputs(x)
    full = oracle.attention(p)
    rows = np.array([0, 17, 5 * 8 + 3, full.shape[0] * 8 - 1], dtype=np.int64)
    sub = oracle.attention(p, rows=rows)
    np.testing.assert_array_equal(sub, full.reshape(-1, full.shape[-1])[rows])
    vis = oracle.visited_blocks(p)
    for b in range(x.batch):
        L, ql = int(x.seq_lens[b]), int(x.q_start[b + 1] - x.q_start[b])
        want = np.zeros(x.block_table.shape[1], np.int32)
        if ql:
            lo = max(0, L - ql - x.window + 1) if x.window > 0 else 0
            want[lo // 16:(L - 1) // 16 + 1] = 1
        np.testing.assert_array_equal(vis[b], want)
