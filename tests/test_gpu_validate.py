"""GPU check of pa_validate: the device-side precondition check of lengths and table entries.

Expected bits are computed here in plain Python from the definitions in
include/pa.h: 1 when seq_len < q_len, 2 when seq_len > max_seq_len (or, in a
linear table, beyond max_blocks_per_seq * 16), 4 when a table entry of a
block the step reads -- logical blocks from the first visible key's block to
(seq_len - 1) / 16, ring entries modulo ring_blocks -- is outside
[0, num_blocks). Entries a step does not read never raise a bit. For an int8
cache: 8 when a K or V scale of a key some query sees (first visible key of
query 0 to seq_len - 1, in a valid block) is NaN or infinite, 16 when such a
V scale is 255 or more in magnitude; scales of other slots never raise a bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_94_amd as pa
from tests.gpu_util import to_torch
from workloads import make_inputs

pytestmark = pytest.mark.gpu
BS = 16


def _expected(lens, table, q_len, window, max_seq_len, num_blocks, ring=0):
    out = []
    for b, L in enumerate(lens):
        bits = 0
        if L < q_len:
            bits |= 1
        if L > max_seq_len or (ring == 0 and L > table.shape[1] * BS):
            bits |= 2
        if L >= 1:
            p0 = L - min(q_len, L)
            lo = max(0, p0 - window + 1) if window > 0 else 0
            hi = (L - 1) // BS if ring else min((L - 1) // BS, table.shape[1] - 1)
            for i in range(lo // BS, hi + 1):
                e = table[b, i % ring if ring else i]
                if e < 0 or e >= num_blocks:
                    bits |= 4
        out.append(bits)
    return [int(np.bitwise_or.reduce(out)) if out else 0] + out


def _scale_bits(ks, vs):
    bits = 0 if np.isfinite(ks) and np.isfinite(vs) else 8
    return bits | (16 if abs(vs) >= 255 else 0)


def _expected_scales(lens, table, q_len, window, num_blocks, ks, vs, ring=0):
    """Scale bits per sequence; ks / vs are [nb, Hkv, 16] (per token) or [Hkv] (per head)."""
    out = []
    for b, L in enumerate(lens):
        bits = 0
        p0 = L - min(q_len, L)
        lo = max(0, p0 - window + 1) if window > 0 else 0
        end = L if ring else min(L, table.shape[1] * BS)
        for j in range(lo, end):
            if ks.ndim == 1:
                for h in range(ks.shape[0]):
                    bits |= _scale_bits(ks[h], vs[h])
                continue
            e = table[b, (j // BS) % ring if ring else j // BS]
            if 0 <= e < num_blocks:
                for h in range(ks.shape[1]):
                    bits |= _scale_bits(ks[e, h, j % BS], vs[e, h, j % BS])
        out.append(bits)
    return [int(np.bitwise_or.reduce(out)) if out else 0] + out


def _run(x, lens, table, max_seq_len, ring=0, ks=None, vs=None):
    st = pa.validate(to_torch(x.q), to_torch(x.k_pool), to_torch(x.v_pool), to_torch(table),
                     to_torch(np.asarray(lens, np.int32)), window=x.window, max_seq_len=max_seq_len,
                     ring_blocks=ring, k_scale=None if ks is None else to_torch(ks),
                     v_scale=None if vs is None else to_torch(vs))
    torch.cuda.synchronize()
    return st.cpu().numpy().tolist()


@pytest.mark.parametrize("window", [0, 40])
def test_valid_inputs_raise_nothing(window):
    x = make_inputs([2, 37, 70, 300, 16], q_len=2 if window else 1, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="bf16", kv_dtype="bf16", window=window, seed=3, poison=True)
    got = _run(x, list(x.seq_lens), x.block_table, x.max_seq_len)
    assert got == [0] * (x.batch + 1)


def test_each_broken_precondition_is_flagged():
    x = make_inputs([50, 60, 70, 80, 90, 100], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                    q_dtype="bf16", kv_dtype="bf16", window=30, seed=4, poison=False, max_blocks=12)
    nb = x.k_pool.shape[0]
    lens = [int(v) for v in x.seq_lens]
    table = x.block_table.copy()
    lens[0] = 1                               # shorter than q_len
    lens[1] = 150                             # longer than max_seq_len (100), still inside the row
    table[2, (70 - 1) // BS] = nb             # a block the step reads: out of range
    table[3, 11] = -7                         # past the sequence's blocks: never read
    table[4, 0] = 10 ** 6                     # before the window: never read
    lens[5] = 12 * BS + 5                     # beyond the table row (and max_seq_len)
    exp = _expected(lens, table, 2, 30, 100, nb)
    assert exp[1:] == [1, 2, 4, 0, 0, 2]
    assert _run(x, lens, table, 100) == exp


def test_ring_entries_are_checked_modulo_the_ring():
    x = make_inputs([20, 100, 400], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="bf16",
                    kv_dtype="bf16", window=48, seed=5, poison=False, ring=True)
    R = x.ring_blocks
    nb = x.k_pool.shape[0]
    lens = [int(v) for v in x.seq_lens]
    table = x.block_table.copy()
    assert _run(x, lens, table, 400, ring=R) == [0, 0, 0, 0]
    table[2, ((400 - 1) // BS) % R] = nb + 3    # the ring entry holding the newest keys
    exp = _expected(lens, table, 1, 48, 400, nb, ring=R)
    assert exp[1:] == [0, 0, 4]
    assert _run(x, lens, table, 400, ring=R) == exp


@pytest.mark.parametrize("window,head_scales,ring", [(0, False, False), (40, False, False), (40, False, True),
                                                     (0, True, False)])
def test_int8_scales_of_unseen_slots_raise_nothing(window, head_scales, ring):
    """Poisoned caches hold NaN scales in every slot no query sees (tails, before the window)."""
    x = make_inputs([2, 37, 70, 300, 16], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="bf16",
                    kv_dtype="int8", window=window, seed=6, poison=True, head_scales=head_scales, ring=ring)
    if not head_scales:
        assert np.isnan(x.k_scale).any() and np.isnan(x.v_scale).any()
    lens = list(x.seq_lens)
    exp = _expected_scales(lens, x.block_table, 2, window, x.k_pool.shape[0], x.k_scale, x.v_scale,
                           ring=x.ring_blocks)
    assert exp == [0] * (x.batch + 1)
    assert _run(x, lens, x.block_table, x.max_seq_len, ring=x.ring_blocks, ks=x.k_scale, vs=x.v_scale) == exp
    # Without the scales only lengths and table entries are checked.
    assert _run(x, lens, x.block_table, x.max_seq_len, ring=x.ring_blocks) == exp


def test_int8_bad_scales_are_flagged():
    x = make_inputs([50, 60, 70, 80, 90], q_len=2, num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="bf16",
                    kv_dtype="int8", window=30, seed=7, poison=True)
    nb = x.k_pool.shape[0]
    lens = [int(v) for v in x.seq_lens]
    ks, vs = x.k_scale.copy(), x.v_scale.copy()
    t = x.block_table

    def at(b, j):                             # the scale slot of sequence b's key j
        return t[b, j // BS], j % BS

    e, s = at(0, 49)
    ks[e, 1, s] = np.inf                      # newest key, K scale infinite
    e, s = at(1, 60 - 2 - 30 + 1)
    vs[e, 0, s] = np.nan                      # first visible key, V scale NaN
    e, s = at(2, 55)
    vs[e, 1, s] = -300.0                      # a seen V scale too large for the prefill
    e, s = at(3, 80 - 2 - 30)
    vs[e, 0, s] = 1e6                         # one key before the window: never seen
    ks[e, 0, s] = np.nan
    e, s = at(4, 89)
    vs[e, 0, s] = 255.0                       # exactly the bound
    exp = _expected_scales(lens, t, 2, 30, nb, ks, vs)
    assert exp[1:] == [8, 8, 16, 0, 16]
    assert _run(x, lens, t, x.max_seq_len, ks=ks, vs=vs) == exp


def test_int8_per_head_scales_flag_every_sequence():
    x = make_inputs([5, 40, 1], q_len=1, num_q_heads=4, num_kv_heads=2, head_dim=64, q_dtype="bf16",
                    kv_dtype="int8", seed=8, poison=True, head_scales=True)
    ks, vs = x.k_scale.copy(), x.v_scale.copy()
    vs[1] = 400.0
    exp = _expected_scales(list(x.seq_lens), x.block_table, 1, 0, x.k_pool.shape[0], ks, vs)
    assert exp == [16, 16, 16, 16]
    assert _run(x, list(x.seq_lens), x.block_table, x.max_seq_len, ks=ks, vs=vs) == exp
    ks[0] = -np.inf
    assert _run(x, list(x.seq_lens), x.block_table, x.max_seq_len, ks=ks, vs=vs) == [24, 24, 24, 24]
