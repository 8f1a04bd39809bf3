"""Pins for the oracle's KV append (oracle_cache_write), CPU only.

The append writes each new token's K and V rows, all KV heads, to global
slot s = block * 16 + slot; float caches take the rows unchanged, int8
caches take per-(token, head) codes rint(x / scale), scale = max|x| / 127 in
binary32 (tiniestgpt notes, KV cache quantization: one scale per token per
head). Each check below holds for the definition whatever the data:
copies match numpy fancy indexing bit for bit, untouched slots stay as they
were, codes stay in [-127, 127] with the row's largest magnitude at +-127,
integer multiples of a power of two come back exactly, the dequantized row is
within half a scale step of the input, negating the input negates the codes,
and the scale of head g lands at [block][g][slot].
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits

BS = 16


def _pools(nb, hkv, d, kind, fill):
    if kind == "int8":
        kp = np.full((nb, BS, hkv, d), fill, dtype=np.int8)
        ks = np.full((nb, hkv, BS), np.nan, dtype=np.float32)
        return kp, kp.copy(), ks, ks.copy()
    dt = np.float32 if kind == "f32" else np.uint16
    kp = np.full((nb, BS, hkv, d), fill, dtype=dt)
    return kp, kp.copy(), None, None


def _rows(rng, T, hkv, d, kind):
    x = rng.standard_normal((T, hkv, d)).astype(np.float32) * 3.0
    return f32_to_bf16_bits(x) if kind == "bf16" else x


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_float_append_is_a_copy(kind):
    rng = np.random.default_rng(1)
    nb, hkv, d, T = 6, 3, 64, 20
    fill = np.uint16(0x7FC0) if kind == "bf16" else np.float32(np.nan)
    kp, vp, _, _ = _pools(nb, hkv, d, kind, fill)
    k, v = _rows(rng, T, hkv, d, kind), _rows(rng, T, hkv, d, kind)
    slots = rng.permutation(nb * BS)[:T].astype(np.int64)
    slots[[3, 11]] = -1
    ek, ev = kp.copy(), vp.copy()
    live = slots >= 0
    ek.reshape(nb * BS, hkv, d)[slots[live]] = k[live]
    ev.reshape(nb * BS, hkv, d)[slots[live]] = v[live]
    oracle.cache_write(k, v, slots, kp, vp)
    assert kp.tobytes() == ek.tobytes() and vp.tobytes() == ev.tobytes()


def _int8_case(x, slots, nb=4):
    T, hkv, d = x.shape
    kp, vp, ks, vs = _pools(nb, hkv, d, "int8", 99)
    oracle.cache_write(x, x.copy(), slots, kp, vp, ks, vs)
    return kp, vp, ks, vs


def _codes_scales(kp, ks, slots, hkv):
    """Codes [T, Hkv, D] and scales [T, Hkv] of the written tokens."""
    blk, slot = slots // BS, slots % BS
    return kp[blk, slot], np.stack([ks[b, :, s] for b, s in zip(blk, slot)])


def test_int8_codes_in_range_with_the_peak_at_127():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((12, 2, 128)).astype(np.float32)
    slots = np.arange(12, dtype=np.int64) * 3
    kp, _, ks, _ = _int8_case(x, slots, nb=3)
    codes, _ = _codes_scales(kp, ks, slots, 2)
    assert codes.min() >= -127 and codes.max() <= 127
    peak = np.abs(x).argmax(axis=-1)
    got = np.take_along_axis(codes, peak[..., None], axis=-1)[..., 0]
    np.testing.assert_array_equal(np.abs(got), 127)
    np.testing.assert_array_equal(np.sign(got), np.sign(np.take_along_axis(x, peak[..., None], axis=-1)[..., 0]))


def test_int8_zero_row_has_unit_scale_and_zero_codes():
    x = np.zeros((2, 2, 64), np.float32)
    x[1, 1, 5] = 0.75          # the other rows stay all-zero
    slots = np.array([7, 40], np.int64)
    kp, _, ks, _ = _int8_case(x, slots)
    codes, scales = _codes_scales(kp, ks, slots, 2)
    assert scales[0, 0] == 1.0 and scales[0, 1] == 1.0 and scales[1, 0] == 1.0
    assert not codes[0].any() and not codes[1, 0].any()


def test_int8_exact_multiples_come_back_exactly():
    rng = np.random.default_rng(3)
    k = rng.integers(-127, 128, size=(5, 2, 64)).astype(np.float32)
    k[..., 0] = np.where(rng.random((5, 2)) < 0.5, 127.0, -127.0)   # the peak sets scale = step
    step = np.float32(2.0 ** -6)
    x = k * step
    slots = np.array([0, 17, 18, 50, 63], np.int64)
    kp, _, ks, _ = _int8_case(x, slots)
    codes, scales = _codes_scales(kp, ks, slots, 2)
    np.testing.assert_array_equal(codes, k.astype(np.int8))
    np.testing.assert_array_equal(scales, np.full((5, 2), step, np.float32))


def test_int8_dequantized_row_is_within_half_a_step():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((16, 4, 128)) * rng.uniform(0.01, 10, size=(16, 4, 1))).astype(np.float32)
    slots = rng.permutation(64)[:16].astype(np.int64)
    kp, _, ks, _ = _int8_case(x, slots)
    codes, scales = _codes_scales(kp, ks, slots, 4)
    err = np.abs(codes.astype(np.float64) * scales[..., None] - x.astype(np.float64))
    assert np.all(err <= 0.5 * scales[..., None].astype(np.float64) * (1 + 1e-6))


def test_int8_negation_negates_codes():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 2, 64)).astype(np.float32)
    slots = np.arange(6, dtype=np.int64)
    kp, _, ks, _ = _int8_case(x, slots)
    kn, _, ksn, _ = _int8_case(-x, slots)
    np.testing.assert_array_equal(kn[0, :6], -kp[0, :6])
    np.testing.assert_array_equal(ksn, ks)


def test_int8_scale_of_head_g_lands_at_block_head_slot():
    # Head g's row is (g + 1) times a base row: its scale is (g + 1) * max|base| / 127.
    base = np.linspace(-1.0, 1.0, 64, dtype=np.float32)
    x = np.stack([base * np.float32(g + 1) for g in range(3)])[None]    # [1, 3, 64]
    slot = np.array([2 * BS + 9], np.int64)
    kp, _, ks, _ = _int8_case(x, slot)
    for g in range(3):
        assert ks[2, g, 9] == np.float32(g + 1) / np.float32(127.0)
    assert np.isnan(ks[2, :, 8]).all() and np.isnan(ks[2, :, 10]).all()


def test_int8_bf16_source_and_skipped_tokens():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 2, 64)).astype(np.float32)
    xb = f32_to_bf16_bits(x)
    slots = np.array([3, -1, 20, -5], np.int64)
    kp, vp, ks, vs = _pools(3, 2, 64, "int8", 99)
    oracle.cache_write(xb, xb.copy(), slots, kp, vp, ks, vs)
    # bf16 rows widen exactly, so they quantize like the fp32 rows they hold
    xw = (xb.astype(np.uint32) << 16).view(np.float32)
    kq, _, ksq, _ = _int8_case(xw, slots, nb=3)
    assert kp.tobytes() == kq.tobytes()
    np.testing.assert_array_equal(ks, ksq)
    written = np.zeros((3, BS), bool)
    written[0, 3] = written[1, 4] = True
    assert (kp[~written] == 99).all() and np.isnan(ks.transpose(0, 2, 1)[~written]).all()
