"""Pins for the oracle's ring cache and per-head int8 scales, CPU only.

Ring (Lab 5, "Ring KV Cache"): position t lives in ring slot t mod 16R. The
pins build ring pools from a linear problem with their own code (copy each
position still held by the ring to slot t mod 16R of fresh blocks, poison
every other slot) and require the oracle to give bit-identical attention,
raw gathers and visit sets, before the ring wraps, exactly at capacity,
long after, with windows that are and are not multiples of the block size,
and for verify steps. Per-head scales (tiniestgpt notes, per_head
granularity): an int8 cache with one scale per head must equal the same
cache with that scale repeated for every token; the append with a given
head scale must produce clamp(rint(x / s)).
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
from workloads import make_inputs

BS = 16


def ring_inputs(x, rng):
    """The same inputs with each sequence's cache in a ring of R blocks (built here, not by the oracle)."""
    R = -(-(x.window + x.q_len - 1) // BS)
    C = R * BS
    B = x.batch
    nb = B * R + 1
    perm = rng.permutation(nb).astype(np.int32)
    poison_blk = int(perm[-1])
    table = perm[:B * R].reshape(B, R).copy()
    kp = np.empty((nb,) + x.k_pool.shape[1:], dtype=x.k_pool.dtype)
    if x.kv_dtype == "int8":
        kp[:] = 127
    elif x.kv_dtype == "bf16":
        kp[:] = 0x7FC0
    else:
        kp[:] = np.nan
    vp = kp.copy()
    ks = vs = None
    if x.k_scale is not None:
        ks = np.full((nb,) + x.k_scale.shape[1:], np.nan, dtype=np.float32)
        vs = ks.copy()
    for b in range(B):
        L = int(x.seq_lens[b])
        for t in range(max(0, L - C), L):
            src_blk, src_slot = int(x.block_table[b, t // BS]), t % BS
            e, slot = (t % C) // BS, t % BS
            dst = int(table[b, e])
            kp[dst, slot] = x.k_pool[src_blk, src_slot]
            vp[dst, slot] = x.v_pool[src_blk, src_slot]
            if ks is not None:
                ks[dst, :, slot] = x.k_scale[src_blk, :, src_slot]
                vs[dst, :, slot] = x.v_scale[src_blk, :, src_slot]
        used = min(R, -(-L // BS))
        table[b, used:] = poison_blk
    return dataclasses.replace(x, k_pool=kp, v_pool=vp, k_scale=ks, v_scale=vs, block_table=table, ring_blocks=R)


def _ringify(x, rng):
    y = ring_inputs(x, rng)
    return oracle.Problem.from_inputs(y), y.ring_blocks


# (lens, q_len, Hq, Hkv, D, window, q_dtype, kv_dtype)
RING_CASES = [
    ([5, 47, 48, 49, 64, 65, 200, 511], 1, 4, 2, 64, 48, "f32", "f32"),    # before, at and past capacity
    ([30, 100, 257], 1, 8, 2, 128, 37, "bf16", "bf16"),                    # window not a multiple of 16
    ([16, 17, 90, 300], 5, 8, 2, 64, 32, "bf16", "bf16"),                  # verify: ring holds W + 4
    ([70, 129, 400], 1, 8, 1, 128, 64, "bf16", "int8"),
    ([3, 4, 33, 1000], 3, 6, 3, 64, 16, "f32", "f32"),
]


def _case(c, seed):
    lens, ql, hq, hkv, d, w, qd, kd = c
    return make_inputs(lens, q_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_dtype=qd,
                       kv_dtype=kd, window=w, seed=seed, poison=True)


@pytest.mark.parametrize("i", range(len(RING_CASES)))
def test_ring_equals_linear(i):
    x = _case(RING_CASES[i], 100 + i)
    ring, _ = _ringify(x, np.random.default_rng(7 + i))
    lin = oracle.Problem.from_inputs(x)
    a, b = oracle.attention(lin), oracle.attention(ring)
    assert not np.isnan(a).any()
    assert a.tobytes() == b.tobytes()
    tokens = x.window + x.q_len - 1
    for which in (0, 1):
        assert oracle.gather(lin, which, tokens).tobytes() == oracle.gather(ring, which, tokens).tobytes()


@pytest.mark.parametrize("i", range(len(RING_CASES)))
def test_ring_visits_closed_form(i):
    x = _case(RING_CASES[i], 200 + i)
    ring, R = _ringify(x, np.random.default_rng(3))
    vis = oracle.visited_blocks(ring)
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        lo = max(0, L - x.q_len - x.window + 1)
        want = np.zeros(R, np.int32)
        for i_log in range(lo // BS, (L - 1) // BS + 1):
            want[i_log % R] += 1
        np.testing.assert_array_equal(vis[b], want)


def test_ring_generator_poisons_exactly_the_unseen_slots():
    # The workload generator's own ring layout: the oracle reads no poisoned slot (no NaN out), and
    # each sequence's ring blocks keep exactly as many clean slots as the step has visible keys.
    for c in RING_CASES:
        if c[7] == "int8":
            continue
        y = make_inputs(c[0], q_len=c[1], num_q_heads=c[2], num_kv_heads=c[3], head_dim=c[4], q_dtype=c[6],
                        kv_dtype=c[7], window=c[5], seed=5, poison=True, ring=True)
        R = -(-(c[5] + c[1] - 1) // BS)
        assert y.ring_blocks == R and y.block_table.shape[1] == R
        out = oracle.attention(oracle.Problem.from_inputs(y))
        assert not np.isnan(out).any()
        pool = y.k_pool.view(np.uint16) if c[7] == "bf16" else y.k_pool.view(np.uint32)
        nan = (pool == 0x7FC0) if c[7] == "bf16" else np.isnan(y.k_pool)
        for b, L in enumerate(y.seq_lens):
            used = min(R, -(-int(L) // BS))
            clean = int((~nan[y.block_table[b, :used], :, 0, 0]).sum())
            assert clean == min(int(L), c[5] + c[1] - 1)


def test_ring_preconditions():
    x = _case(RING_CASES[2], 1)
    ring, R = _ringify(x, np.random.default_rng(1))
    s = ring.struct
    s.ring_blocks = R - 1                       # cannot hold W + q_len - 1 keys
    with pytest.raises(oracle.OracleError):
        oracle.attention(ring)
    s.ring_blocks, s.window = R, 0              # a ring needs a window
    with pytest.raises(oracle.OracleError):
        oracle.attention(ring)


def _per_head(x, rng):
    """The same int8 cache with one scale per head, and its per-token twin (scale repeated)."""
    hkv = x.num_kv_heads
    sk = rng.uniform(0.01, 0.2, hkv).astype(np.float32)
    sv = rng.uniform(0.01, 0.2, hkv).astype(np.float32)
    nb = x.k_pool.shape[0]
    tk = np.broadcast_to(sk[None, :, None], (nb, hkv, BS)).copy()
    tv = np.broadcast_to(sv[None, :, None], (nb, hkv, BS)).copy()
    head = oracle.Problem(x.q, x.k_pool, x.v_pool, x.block_table, x.seq_lens, q_len=x.q_len, window=x.window,
                          scale=x.scale, k_scale=sk, v_scale=sv)
    tok = oracle.Problem(x.q, x.k_pool, x.v_pool, x.block_table, x.seq_lens, q_len=x.q_len, window=x.window,
                         scale=x.scale, k_scale=tk, v_scale=tv)
    return head, tok


@pytest.mark.parametrize("window,q_len", [(0, 1), (20, 1), (0, 4)])
def test_per_head_scales_equal_repeated_per_token_scales(window, q_len):
    x = make_inputs([9, 40, 77], q_len=q_len, num_q_heads=8, num_kv_heads=4, head_dim=64, q_dtype="bf16",
                    kv_dtype="int8", window=window, seed=31)
    head, tok = _per_head(x, np.random.default_rng(2))
    assert oracle.attention(head).tobytes() == oracle.attention(tok).tobytes()


def test_per_head_scales_differ_by_head():
    # Two heads with the same codes and different scales give different outputs, head by head.
    x = make_inputs([40], q_len=1, num_q_heads=2, num_kv_heads=2, head_dim=64, q_dtype="f32", kv_dtype="int8",
                    seed=3)
    x.k_pool[:, :, 1] = x.k_pool[:, :, 0]
    x.v_pool[:, :, 1] = x.v_pool[:, :, 0]
    x.q[:, :, 1] = x.q[:, :, 0]
    sk = np.array([0.05, 0.05], np.float32)
    sv = np.array([0.05, 0.1], np.float32)
    out = oracle.attention(oracle.Problem(x.q, x.k_pool, x.v_pool, x.block_table, x.seq_lens, q_len=1, window=0,
                                          scale=x.scale, k_scale=sk, v_scale=sv))
    np.testing.assert_allclose(out[0, 0, 1], 2 * out[0, 0, 0], rtol=1e-13)


def test_per_head_append_codes():
    rng = np.random.default_rng(8)
    hkv, d, nb, T = 3, 64, 4, 10
    s = np.array([0.5, 0.03125, 2.0], np.float32)
    x = (rng.standard_normal((T, hkv, d)) * 3).astype(np.float32)
    x[0, 0, :4] = [0.25, 0.75, -0.25, 1000.0]       # ties at s = 0.5 -> 0, 2, -0; saturation -> 127
    x[1, 1, :2] = [-1e9, 1e-30]
    slots = rng.permutation(nb * BS)[:T].astype(np.int64)
    kp = np.full((nb, BS, hkv, d), 99, np.int8)
    vp = kp.copy()
    ks, vs = s.copy(), s.copy()
    oracle.cache_write(x, x.copy(), slots, kp, vp, ks, vs)
    assert ks.tobytes() == s.tobytes() and vs.tobytes() == s.tobytes()      # given scales stay as they are
    want = np.clip(np.rint(x / s[None, :, None]), -127, 127).astype(np.int8)
    np.testing.assert_array_equal(kp.reshape(-1, hkv, d)[slots], want)
    np.testing.assert_array_equal(vp.reshape(-1, hkv, d)[slots], want)
    assert list(want[0, 0, :4]) == [0, 2, 0, 127] and list(want[1, 1, :2]) == [-127, 0]
    untouched = np.setdiff1d(np.arange(nb * BS), slots)
    assert (kp.reshape(-1, hkv, d)[untouched] == 99).all()
