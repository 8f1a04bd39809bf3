"""Several decode steps driven by the block allocator, on the GPU, against the oracle.

The allocator (C++, host) hands out slot ids and block tables; the KV append
(pa_cache_write) writes each step's rows, skipping positions a prefix-cache
hit already holds; decode reads through the allocator's tables. The host
mirror applies the oracle's append to the same slots, so after every step
the device pools must equal the mirror bit for bit and decode must match
the oracle's attention over the mirror.

Synthetic K/V rows are a function of the token's whole prefix (a seeded draw
keyed by a CRC of the prefix ids), as real keys and values are: that is what
makes sharing a prefix block correct, and the dense check below confirms
every sequence sees, through its table, exactly the rows of its own prefix.
"""

from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_94_amd as pa
from paged_kv_cache_94_amd.allocator import BlockAllocator
from tests.gpu_util import TOL, max_err, to_torch
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
BS = 16
HQ, HKV, D = 8, 2, 128


def _log(msg):
    print(msg, flush=True)


def _rows_for(prefix_ids):
    """K and V rows [Hkv, D] (fp32) of the last token of this prefix."""
    key = zlib.crc32(np.asarray(prefix_ids, dtype=np.int32).tobytes())
    r = np.random.default_rng(key)
    return r.standard_normal((2, HKV, D)).astype(np.float32)


def _host(t):
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


class Engine:
    def __init__(self, kv, num_blocks, rng, ring_blocks=0, window=0):
        self.kv = kv
        self.rng = rng
        self.ring = ring_blocks
        self.window = window
        self.alloc = BlockAllocator(num_blocks, BS, prefix_cache=True)
        self.nb = num_blocks
        if kv == "int8":
            self.kp = np.full((num_blocks, BS, HKV, D), 77, dtype=np.int8)
            self.ks = np.full((num_blocks, HKV, BS), np.nan, dtype=np.float32)
            self.vs = self.ks.copy()
        else:
            self.kp = np.full((num_blocks, BS, HKV, D), 0x7FC0, dtype=np.uint16)
            self.ks = self.vs = None
        self.vp = self.kp.copy()
        self.dk, self.dv = to_torch(self.kp), to_torch(self.vp)
        self.dks = None if self.ks is None else to_torch(self.ks)
        self.dvs = None if self.vs is None else to_torch(self.vs)
        self.tokens = {}
        self.hit_tokens = 0

    def _write(self, seq_tokens, slots):
        """Rows for each (sequence prefix) at its slot; slot -1 is skipped by both sides."""
        k = np.stack([_rows_for(p)[0] for p in seq_tokens])
        v = np.stack([_rows_for(p)[1] for p in seq_tokens])
        src = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        pa.cache_write(to_torch(src[0]), to_torch(src[1]), torch.from_numpy(slots).cuda(), self.dk, self.dv,
                       self.dks, self.dvs)
        oracle.cache_write(src[0], src[1], slots, self.kp, self.vp, self.ks, self.vs)

    def grow(self, seq_ids, new_tokens):
        counts = [len(t) for t in new_tokens]
        flat = [x for t in new_tokens for x in t]
        slots, cached = self.alloc.append_batch(seq_ids, counts, flat)
        prefixes = []
        for s, t in zip(seq_ids, new_tokens):
            base = self.tokens.setdefault(s, [])
            for j in range(len(t)):
                prefixes.append(tuple(base + t[:j + 1]))
            base += t
        self.hit_tokens += int(cached.sum())
        self._write(prefixes, slots)

    def add(self, sid, prompt):
        self.alloc.add(sid, self.ring)
        self.grow([sid], [prompt])

    def release(self, sid):
        self.alloc.release(sid)
        del self.tokens[sid]

    def check(self):
        sids = sorted(self.tokens)
        lens = [len(self.tokens[s]) for s in sids]
        mb = self.ring if self.ring else max(-(-n // BS) for n in lens)
        table, seq_lens = self.alloc.block_table(sids, mb)
        assert seq_lens.tolist() == lens
        torch.cuda.synchronize()
        for got, exp in ((self.dk, self.kp), (self.dv, self.vp), (self.dks, self.ks), (self.dvs, self.vs)):
            if exp is not None:
                assert _host(got).tobytes() == exp.tobytes()
        if self.kv == "bf16":   # every sequence sees its own prefix's rows through its table
            for i, s in enumerate(sids):
                held = range(max(0, lens[i] - self.ring * BS), lens[i]) if self.ring else range(lens[i])
                for pos in held:
                    entry = (pos // BS) % self.ring if self.ring else pos // BS
                    blk, slot = table[i, entry], pos % BS
                    want = f32_to_bf16_bits(_rows_for(self.tokens[s][:pos + 1]))
                    assert (self.kp[blk, slot] == want[0]).all() and (self.vp[blk, slot] == want[1]).all()
        B = len(sids)
        q32 = self.rng.standard_normal((B, 1, HQ, D)).astype(np.float32)
        q = f32_to_bf16_bits(q32)
        dq = to_torch(q)
        out = torch.full_like(dq, float("nan"))
        dt, dl = torch.from_numpy(table).cuda(), torch.from_numpy(seq_lens).cuda()
        kw = dict(max_seq_len=max(lens), window=self.window, ring_blocks=self.ring)
        if self.kv == "int8":
            pa.decode_int8(out, dq, self.dk, self.dv, dt, dl, self.dks, self.dvs, **kw)
        else:
            pa.decode(out, dq, self.dk, self.dv, dt, dl, **kw)
        torch.cuda.synchronize()
        prob = oracle.Problem(q, self.kp, self.vp, table, seq_lens, q_len=1, window=self.window, scale=D ** -0.5,
                              k_scale=self.ks, v_scale=self.vs, ring_blocks=self.ring)
        ref = oracle.attention(prob)
        got = out.float().cpu().numpy().astype(np.float64)
        assert not np.isnan(got).any()
        return max_err(got, ref)


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_allocator_append_decode_steps(kv):
    rng = np.random.default_rng(2024 if kv == "bf16" else 2025)
    eng = Engine(kv, num_blocks=48, rng=rng)
    stems = [[int(t) for t in np.random.default_rng(s).integers(0, 50, 80)] for s in range(2)]
    next_id = 0
    for i in range(5):
        n = int(rng.integers(18, 75))
        k = int(rng.integers(0, n + 1))
        eng.add(next_id, stems[i % 2][:k] + [int(t) for t in rng.integers(50, 99, n - k)])
        next_id += 1
    worst = 0.0
    for step in range(10):
        if step in (3, 6):
            eng.release(sorted(eng.tokens)[0])
            n = int(rng.integers(20, 60))
            eng.add(next_id, stems[step % 2][:n])     # a stem prefix: its leading blocks may hit
            next_id += 1
        sids = sorted(eng.tokens)
        eng.grow(sids, [[int(rng.integers(0, 99))] for _ in sids])
        err = eng.check()
        worst = max(worst, err)
        _log(f"{kv} step {step}: B={len(sids)} free={eng.alloc.num_free()} max|err|={err:.2e}")
        assert err <= TOL[kv]
    q, h = eng.alloc.stats()
    _log(f"{kv}: prefix blocks queried {q}, hit {h}; {eng.hit_tokens} tokens served from cache")
    assert h > 0 and eng.hit_tokens > 0


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_ring_allocator_decode_steps(kv):
    # A window layer (W = 48) whose sequences live in rings of 3 blocks: prompts longer and shorter
    # than the ring, then 40 decode steps, so every ring wraps several times.
    rng = np.random.default_rng(77 if kv == "bf16" else 78)
    eng = Engine(kv, num_blocks=24, rng=rng, ring_blocks=3, window=48)
    for sid, n in enumerate([5, 30, 47, 48, 49, 120]):
        eng.add(sid, [int(t) for t in rng.integers(0, 99, n)])
    assert eng.alloc.num_free() == 24 - (1 + 2 + 3 + 3 + 3 + 3)
    for step in range(40):
        if step == 20:
            eng.release(2)
            eng.add(100, [int(t) for t in rng.integers(0, 99, 70)])
        sids = sorted(eng.tokens)
        eng.grow(sids, [[int(rng.integers(0, 99))] for _ in sids])
        err = eng.check()
        if step % 10 == 0:
            _log(f"ring {kv} step {step}: free={eng.alloc.num_free()} max|err|={err:.2e}")
        assert err <= TOL[kv]
    assert eng.alloc.num_free() == 24 - 6 * 3
