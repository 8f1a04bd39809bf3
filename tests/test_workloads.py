"""The seeded input generator: shapes, block assignment, poison and the int8 encoding."""

from __future__ import annotations

import numpy as np
import pytest

from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_config, make_inputs


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.0e38, 0.0, -0.0], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    # 1+2^-8 is the midpoint of 1 and 1+2^-7: ties go to the even mantissa (1.0);
    # 1+3*2^-8 is the midpoint of 1+2^-7 and 1+2^-6: ties go to 1+2^-6.
    np.testing.assert_array_equal(got[:4], [1.0, 1.0, 1.0 + 2**-6, -2.5])
    assert np.isfinite(got[4]) and got[5] == 0.0
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_tiny_config_layout():
    x = make_config(1)
    assert x.q.shape == (2, 1, 4, 64) and x.q.dtype == np.float32
    assert x.k_pool.shape == (16, 16, 2, 64)
    assert x.block_table.shape == (2, 5)
    np.testing.assert_array_equal(x.seq_lens, [37, 70])
    used = np.concatenate([x.block_table[0, :3], x.block_table[1, :5]])
    assert len(set(used.tolist())) == 8 and used.min() >= 0 and used.max() < 16


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_named_config_shapes(idx):
    c = CONFIGS[idx]
    x = make_config(idx, batch=3)
    assert x.q.shape == (3, c["q_len"], c["Hq"], c["D"])
    assert x.k_pool.shape[1:] == (16, c["Hkv"], c["D"])
    assert x.max_blocks == (c["max_len"] + 15) // 16
    need = int(((x.seq_lens + 15) // 16).sum())
    assert x.num_blocks >= need + 1
    assert x.v_aliases_k == bool(c.get("alias_v"))
    if c["kv_dtype"] == "int8":
        assert x.k_pool.dtype == np.int8 and x.k_scale.shape == (x.num_blocks, c["Hkv"], 16)
        assert np.abs(x.k_pool).max() <= 127


def test_pool_assignment_is_a_permutation():
    x = make_inputs([1, 16, 17, 100], q_len=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
                    q_dtype="f32", kv_dtype="f32", seed=5)
    used = np.concatenate([x.block_table[b, :(L + 15) // 16] for b, L in enumerate(x.seq_lens)])
    assert len(np.unique(used)) == used.size


def test_int8_encoding_bounds():
    x = make_inputs([40], q_len=1, num_q_heads=2, num_kv_heads=2, head_dim=128, q_dtype="bf16",
                    kv_dtype="int8", seed=6)
    # Every (token, head) row uses the full code range at its largest magnitude.
    assert np.all(np.abs(x.k_pool).max(axis=-1) == 127)
    assert np.all(x.k_scale > 0)


def test_poison_marks_only_unusable_slots():
    x = make_inputs([20, 40], q_len=1, num_q_heads=2, num_kv_heads=1, head_dim=64, q_dtype="f32",
                    kv_dtype="f32", window=10, seed=7, poison=True)
    for b, L in enumerate(x.seq_lens):
        nblk = (L + 15) // 16
        rows = x.k_pool[x.block_table[b, :nblk]].reshape(-1, 1, 64)
        first = L - 10
        assert np.isnan(rows[:first]).all()
        assert np.isfinite(rows[first:L]).all()
        assert np.isnan(rows[L:]).all()
        assert np.isnan(x.k_pool[x.block_table[b, nblk:]]).all()


def test_generation_is_deterministic():
    a = make_config(4, batch=2)
    b = make_config(4, batch=2)
    np.testing.assert_array_equal(a.k_pool, b.k_pool)
    np.testing.assert_array_equal(a.v_scale, b.v_scale)
    np.testing.assert_array_equal(a.block_table, b.block_table)
