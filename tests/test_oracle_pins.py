"""Pins for the fp64 oracle: checks against things other than itself.

* torch's float64 scaled_dot_product_attention on contiguous copies built by
  numpy fancy indexing, with an explicit band mask and torch's own GQA head
  expansion (tests/refs.py), over many tiny shapes and window boundaries;
* closed forms: a single visible key returns its value, window 1 returns the
  query's own value, equal keys or a zero query return the mean of the visible
  values, all-ones values return ones;
* invariants: relabelling physical blocks, a window at least as long as the
  sequence, verify rows against single-token decode steps, expanding KV heads
  to one per query head, int8 with unit scales against fp32;
* hand-derived golden fixtures (tests/golden/*.json, each with its citation).
"""

from __future__ import annotations

import zlib

import glob
import json
import os

import numpy as np
import pytest

import oracle
from tests.refs import band_mask, contiguous_cache, dense_sdpa, storage_to_f64
from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(x, **kw):
    return oracle.attention(oracle.Problem.from_inputs(x), **kw)


# (lens, q_len, Hq, Hkv, D, window, q_dtype, kv_dtype)
SDPA_CASES = [
    ([37, 70], 1, 4, 2, 64, 0, "f32", "f32"),
    ([1, 16, 17, 33], 1, 4, 2, 64, 0, "f32", "f32"),
    ([80, 45, 16], 1, 8, 1, 128, 0, "bf16", "bf16"),
    ([64, 65, 79], 1, 16, 16, 64, 1, "f32", "f32"),
    ([64, 65, 79], 1, 4, 4, 64, 15, "bf16", "bf16"),
    ([64, 65, 79], 1, 4, 2, 64, 16, "bf16", "bf16"),
    ([64, 65, 79], 1, 4, 2, 64, 17, "f32", "f32"),
    ([50, 51, 52], 1, 2, 1, 256, 49, "bf16", "bf16"),
    ([50, 51, 52], 1, 2, 1, 256, 51, "bf16", "bf16"),
    ([50, 51, 52], 1, 2, 1, 256, 53, "bf16", "bf16"),
    ([40, 77], 1, 16, 1, 256, 0, "bf16", "bf16"),
    ([23, 48, 61], 1, 8, 2, 128, 0, "bf16", "int8"),
    ([23, 48, 61], 1, 8, 2, 128, 20, "bf16", "int8"),
    ([5, 16, 17, 44], 5, 8, 2, 128, 0, "bf16", "bf16"),
    ([5, 16, 17, 44], 5, 8, 2, 64, 7, "f32", "f32"),
    ([6, 30, 80], 3, 6, 3, 64, 16, "bf16", "int8"),
]


@pytest.mark.parametrize("case", SDPA_CASES, ids=lambda c: "L%s_q%d_h%d-%d_d%d_w%d_%s_%s" % (
    "-".join(map(str, c[0])), c[1], c[2], c[3], c[4], c[5], c[6], c[7]))
def test_matches_torch_sdpa(case):
    lens, q_len, Hq, Hkv, D, window, qd, kvd = case
    x = make_inputs(lens, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    q_dtype=qd, kv_dtype=kvd, window=window, seed=zlib.crc32(repr(case).encode()),
                    poison=True)
    got = run(x)
    ref = dense_sdpa(x)
    assert not np.isnan(got).any()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    x = make_inputs([30, 50, 17], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="bf16", kv_dtype="bf16", window=9, seed=3)
    full = run(x)
    rows = np.array([0, 5, 7, 23, 11], dtype=np.int64)
    part = run(x, rows=rows)
    np.testing.assert_array_equal(part, full.reshape(-1, 64)[rows])


def test_single_key_returns_value():
    x = make_inputs([1, 1, 1], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", seed=11)
    got = run(x)
    for b in range(3):
        _, v = contiguous_cache(x, b)
        for h in range(4):
            np.testing.assert_array_equal(got[b, 0, h], v[0, h // 2])


def test_window_one_returns_own_value():
    x = make_inputs([9, 40, 77], q_len=1, num_q_heads=4, num_kv_heads=4, head_dim=128,
                    q_dtype="bf16", kv_dtype="bf16", window=1, seed=12)
    got = run(x)
    for b in range(3):
        _, v = contiguous_cache(x, b)
        np.testing.assert_array_equal(got[b, 0], v[-1])


def _mean_visible_values(x, b, t, h):
    _, v = contiguous_cache(x, b)
    L = v.shape[0]
    vis = band_mask(L, x.q_len, x.window)[t]
    return v[vis, h // x.group].mean(axis=0)


def test_equal_keys_give_mean_value():
    x = make_inputs([33, 70], q_len=3, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", window=20, seed=13)
    x.k_pool[...] = x.k_pool[0, 0, 0]  # one key vector everywhere
    got = run(x)
    for b in range(2):
        for t in range(3):
            for h in range(4):
                np.testing.assert_allclose(got[b, t, h], _mean_visible_values(x, b, t, h), atol=1e-13)


def test_zero_query_gives_mean_value():
    x = make_inputs([18, 47], q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    q_dtype="bf16", kv_dtype="bf16", seed=14)
    x.q[...] = 0
    got = run(x)
    for b in range(2):
        for h in range(8):
            np.testing.assert_allclose(got[b, 0, h], _mean_visible_values(x, b, 0, h), atol=1e-13)


def test_unit_values_give_ones():
    x = make_inputs([25, 61, 3], q_len=2, num_q_heads=4, num_kv_heads=1, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", window=11, seed=15)
    x.v_pool[...] = 1.0
    np.testing.assert_allclose(run(x), 1.0, atol=1e-14)


def test_block_permutation_invariance():
    x = make_inputs([37, 70, 5], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="bf16", kv_dtype="bf16", window=30, seed=16)
    base = run(x)
    rng = np.random.default_rng(99)
    perm = rng.permutation(x.num_blocks)           # new position of old block i is perm[i]
    y_k = np.empty_like(x.k_pool)
    y_v = np.empty_like(x.v_pool)
    y_k[perm] = x.k_pool
    y_v[perm] = x.v_pool
    x.k_pool, x.v_pool = y_k, y_v
    x.block_table = perm[x.block_table].astype(np.int32)
    np.testing.assert_array_equal(run(x), base)


def test_long_window_equals_global():
    x = make_inputs([37, 70], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", window=0, seed=17)
    base = run(x)
    for w in (70, 71, 1000):
        x.window = w
        np.testing.assert_array_equal(run(x), base)


def test_verify_rows_equal_sequential_decode():
    q_len = 5
    x = make_inputs([5, 21, 64, 90], q_len=q_len, num_q_heads=8, num_kv_heads=2, head_dim=128,
                    q_dtype="bf16", kv_dtype="bf16", window=19, seed=18)
    full = run(x)
    for t in range(q_len):
        p = oracle.Problem(x.q[:, t:t + 1], x.k_pool, x.v_pool, x.block_table,
                           x.seq_lens - (q_len - 1 - t), q_len=1, window=x.window, scale=x.scale)
        np.testing.assert_array_equal(oracle.attention(p)[:, 0], full[:, t])


def test_gqa_equals_expanded_heads():
    x = make_inputs([29, 64], q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=64,
                    q_dtype="bf16", kv_dtype="bf16", window=0, seed=19)
    base = run(x)
    kx = np.repeat(x.k_pool, 4, axis=2)
    vx = np.repeat(x.v_pool, 4, axis=2)
    p = oracle.Problem(x.q, kx, vx, x.block_table, x.seq_lens, q_len=1, window=0, scale=x.scale)
    np.testing.assert_array_equal(oracle.attention(p), base)


def test_int8_unit_scales_equal_fp32():
    x = make_inputs([33, 47], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=128,
                    q_dtype="f32", kv_dtype="int8", window=0, seed=20)
    x.k_scale[...] = 1.0
    x.v_scale[...] = 1.0
    got = run(x)
    p = oracle.Problem(x.q, x.k_pool.astype(np.float32), x.v_pool.astype(np.float32),
                       x.block_table, x.seq_lens, q_len=1, window=0, scale=x.scale)
    np.testing.assert_array_equal(got, oracle.attention(p))


def test_int8_scales_apply_per_token():
    # Doubling one token's key scale equals doubling that key's codes' value in fp32.
    x = make_inputs([20], q_len=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
                    q_dtype="f32", kv_dtype="int8", seed=21)
    blk, slot = x.block_table[0, 0], 7
    kf = x.k_pool.astype(np.float32) * x.k_scale.transpose(0, 2, 1)[..., None]
    vf = x.v_pool.astype(np.float32) * x.v_scale.transpose(0, 2, 1)[..., None]
    x.k_scale[blk, :, slot] *= 2.0
    kf[blk, slot] *= 2.0
    got = run(x)
    p = oracle.Problem(x.q, kf.astype(np.float32), vf.astype(np.float32), x.block_table, x.seq_lens,
                       q_len=1, window=0, scale=x.scale)
    np.testing.assert_allclose(got, oracle.attention(p), atol=1e-6)


def test_visited_blocks_closed_form():
    # The oracle lists visible keys one by one; compare with the interval they must form.
    for window, q_len in ((0, 1), (1, 1), (16, 1), (17, 1), (33, 5), (100, 5)):
        x = make_inputs([1, 15, 16, 17, 31, 32, 33, 90], q_len=min(q_len, 1) if q_len == 1 else q_len,
                        num_q_heads=2, num_kv_heads=1, head_dim=64, q_dtype="f32", kv_dtype="f32",
                        window=window, seed=22) if q_len == 1 else \
            make_inputs([5, 15, 16, 17, 31, 32, 33, 90], q_len=q_len, num_q_heads=2, num_kv_heads=1,
                        head_dim=64, q_dtype="f32", kv_dtype="f32", window=window, seed=22)
        vis = oracle.visited_blocks(oracle.Problem.from_inputs(x))
        for b, L in enumerate(x.seq_lens):
            first = max(0, L - q_len - window + 1) if window > 0 else 0
            expect = np.zeros(x.max_blocks, dtype=np.int32)
            expect[first // 16:(L - 1) // 16 + 1] = 1
            np.testing.assert_array_equal(vis[b], expect)


def test_gather_matches_fancy_indexing():
    x = make_inputs([37, 70, 3], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="bf16", kv_dtype="bf16", window=21, seed=23)
    p = oracle.Problem.from_inputs(x)
    for which, pool in ((0, x.k_pool), (1, x.v_pool)):
        got = oracle.gather(p, which, dst_tokens=24, fill=0)
        for b, L in enumerate(x.seq_lens):
            first = max(0, L - x.q_len - x.window + 1)
            nblk = (L + 15) // 16
            rows = pool[x.block_table[b, :nblk]].reshape(nblk * 16, 2, 64)[first:L]
            np.testing.assert_array_equal(got[b, :L - first], rows)
            assert not got[b, L - first:].any()


def test_rejects_bad_inputs():
    x = make_inputs([20], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", seed=24)
    x.block_table[0, 1] = x.num_blocks  # out of the pool
    with pytest.raises(oracle.OracleError):
        run(x)
    y = make_inputs([20], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", seed=24)
    y.seq_lens[0] = 10_000  # longer than the block table can map
    with pytest.raises(oracle.OracleError):
        run(y)


def _golden_problem(d):
    lens = d["seq_lens"]
    assert len(lens) == 1
    L = lens[0]
    k_tok = np.asarray(d["k_tokens"], dtype=np.float32)   # [L, Hkv, D]
    v_tok = np.asarray(d["v_tokens"], dtype=np.float32)
    nblk = (L + 15) // 16
    num_blocks = nblk + 2
    phys = np.arange(num_blocks)[::-1][:nblk].astype(np.int32)   # deliberately not the identity
    k_pool = np.full((num_blocks, 16, d["Hkv"], d["D"]), np.nan, dtype=np.float32)
    v_pool = np.full_like(k_pool, np.nan)
    for j in range(L):
        k_pool[phys[j // 16], j % 16] = k_tok[j]
        v_pool[phys[j // 16], j % 16] = v_tok[j]
    q = np.asarray(d["q"], dtype=np.float32)
    return oracle.Problem(q, k_pool, v_pool, phys[None, :], np.array(lens, dtype=np.int32),
                          q_len=d["q_len"], window=d["window"], scale=d["scale"])


@pytest.mark.parametrize("path", sorted(p for p in glob.glob(os.path.join(GOLDEN, "*.json"))
                                        if "k_tokens" in open(p).read()),
                         ids=os.path.basename)
def test_golden_closed_forms(path):
    d = json.load(open(path))
    assert d["citation"]
    got = oracle.attention(_golden_problem(d))
    np.testing.assert_allclose(got, np.asarray(d["expected"]), rtol=0, atol=d["tolerance"])
