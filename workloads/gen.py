"""Seeded synthetic paged-KV inputs.

Layouts (all row-major, shared by every consumer):

* ``q``           ``[B, q_len, Hq, D]``      float32, or uint16 holding bf16 bits
* ``k_pool``      ``[num_blocks, 16, Hkv, D]`` float32 / uint16 (bf16 bits) / int8
* ``v_pool``      same shape and dtype; may be the very same array as ``k_pool``
* ``k_scale``     ``[num_blocks, Hkv, 16]``   float32, int8 caches only (one per token per head; a
                                              block's 16 scales of one head are contiguous)
* ``v_scale``     same
* ``block_table`` ``[B, max_blocks]``         int32, logical block -> physical block
* ``seq_lens``    ``[B]``                     int32, cached tokens including this step's queries

The pool layout ``[block][slot][head][dim]`` and the block table are the
ones described in the tiniestgpt inference notes ("PagedAttention: why it is
needed"). The five named configurations are synthetic stand-ins for a
Gemma4-12B local layer, a Gemma4-12B global layer (Lab 5, "Sliding Window
Attention" and "Grouped Query Attention"), a 70B-class GQA layer with an int8
cache, and a speculative-verify step.

Draw order for every configuration: lengths -> block permutation -> Q -> K
-> V -> int8 encoding. The int8 encoding (symmetric, one scale per token per
head, ``scale = max|x| / 127``, round half to even, clamp to [-127, 127], a
zero row gets scale 1) is part of the input recipe: both the kernels and the
oracle consume the stored codes and scales, never the float draws.

``poison=True`` fills every cache slot that a correct kernel must not use
(unused pool blocks, slots past a sequence's end, keys older than the window)
with NaN (bf16/f32) or NaN scales (int8), and points unused block-table
entries at an unused, NaN-filled block, so a stray read shows up as NaN in
the output instead of faulting.
"""

from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

BLOCK_SIZE = 16

_BF16_QNAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns the uint16 bit pattern."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 22

    def conv(s: int) -> None:
        u = flat_in[s:s + step].view(np.uint32)
        rounded = (u + (((u >> 16) & 1) + 0x7FFF)) >> 16
        res = rounded.astype(np.uint16)
        nan = np.isnan(flat_in[s:s + step])
        if nan.any():
            res[nan] = _BF16_QNAN
        flat_out[s:s + step] = res

    starts = range(0, flat_in.size, step)
    if len(starts) <= 1:
        for s in starts:
            conv(s)
    else:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
            list(ex.map(conv, starts))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _encode_int8_per_head(x: np.ndarray):
    """Symmetric int8 codes with one float32 scale per KV head (axis 2) over the whole pool."""
    amax = np.abs(x).max(axis=(0, 1, 3))
    scale = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    codes = np.rint(x / scale[None, None, :, None]).clip(-127, 127).astype(np.int8)
    return codes, scale


def _encode_int8_per_token(x: np.ndarray):
    """Symmetric int8 codes with one float32 scale per row of the last axis."""
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    codes = np.rint(x / scale[..., None]).clip(-127, 127).astype(np.int8)
    return codes, scale


@dataclasses.dataclass
class PagedInputs:
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    block_table: np.ndarray
    seq_lens: np.ndarray
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    scale: float
    q_dtype: str          # "f32" | "bf16"
    kv_dtype: str         # "f32" | "bf16" | "int8"
    block_size: int = BLOCK_SIZE
    name: str = "custom"
    seed: int = 0
    ring_blocks: int = 0  # > 0: each table row is a ring of this many blocks (window layers)
    q_start: Optional[np.ndarray] = None  # prefill: [B+1] offsets of packed queries q [total, Hq, D]

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def v_aliases_k(self) -> bool:
        return self.v_pool is self.k_pool

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


_CHUNK = 1 << 22


def _standard_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 N(0,1) draws of ``shape``.

    One 63-bit key is taken from ``rng`` (so the caller's draw order is
    kept); the array is then filled in fixed chunks of 4 Mi elements, chunk c
    from its own generator seeded with (key, c). The result depends only on
    the key, never on how many threads fill it.
    """
    key = int(rng.integers(0, 2**63 - 1))
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n_chunks = (flat.size + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        g = np.random.default_rng([key, c])
        seg = flat[c * _CHUNK:(c + 1) * _CHUNK]
        g.standard_normal(out=seg, dtype=np.float32)

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        import concurrent.futures as cf
        workers = max(1, min(16, os.cpu_count() or 1))
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def _draw_kv(rng: np.random.Generator, shape, kv_dtype: str, head_scales: bool = False):
    x = _standard_normal(rng, shape)
    if kv_dtype == "f32":
        return x, None
    if kv_dtype == "bf16":
        return f32_to_bf16_bits(x), None
    if kv_dtype == "int8" and head_scales:
        return _encode_int8_per_head(x)                   # scale [Hkv]
    if kv_dtype == "int8":
        codes, scale = _encode_int8_per_token(x)          # scale [blocks, 16, Hkv]
        return codes, np.ascontiguousarray(scale.transpose(0, 2, 1))
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def _poison_slots(pool: np.ndarray, scale: Optional[np.ndarray], blocks, slots, kv_dtype: str):
    """Overwrite pool[blocks, slots] (all heads, all dims) with NaN, or NaN scales for int8.

    Per-head int8 scales are shared by every token, so there only the codes
    are poisoned (to 127, which moves any score that reads them)."""
    if kv_dtype == "int8":
        pool[blocks, slots] = 127
        if scale.ndim == 3:
            scale[blocks, :, slots] = np.nan
    elif kv_dtype == "bf16":
        pool[blocks, slots] = _BF16_QNAN
    else:
        pool[blocks, slots] = np.nan


def make_inputs(seq_lens: Sequence[int], *, q_len: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, q_dtype: str, kv_dtype: str, window: int = 0,
                scale: Optional[float] = None, seed: int = 0, rng: Optional[np.random.Generator] = None,
                num_blocks: Optional[int] = None, pool_slack: float = 1.1,
                max_blocks: Optional[int] = None, alias_v: bool = False, poison: bool = False,
                name: str = "custom", ring: bool = False, head_scales: bool = False,
                q_lens: Optional[Sequence[int]] = None) -> PagedInputs:
    """Build one seeded paged-cache problem.

    ``seq_lens`` counts cached tokens including this step's ``q_len`` queries.
    Physical blocks are handed to sequences consecutively from one random
    permutation of the pool ids.

    ``ring`` (window layers only): each sequence owns a ring of
    R = ceil((window + q_len - 1) / 16) blocks and position t lives in ring
    slot t mod 16R (Lab 5, "Ring KV Cache"); the table has R columns.
    ``head_scales`` (int8 only): one scale per KV head for the whole pool.
    ``q_lens`` (prefill): per-sequence query counts; queries are packed one
    sequence after another, q is [sum(q_lens), Hq, D] with offsets q_start,
    and query t of sequence b sits at seq_lens[b] - q_lens[b] + t. ``q_len``
    is then ignored and set to max(q_lens).
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int64)
    if lens.ndim != 1:
        raise ValueError("seq_lens must be 1-D")
    qls = np.full(lens.size, q_len, dtype=np.int64) if q_lens is None else np.asarray(q_lens, dtype=np.int64)
    if q_lens is not None:
        if qls.shape != lens.shape or np.any(qls < 0):
            raise ValueError("q_lens must be [B], >= 0")
        q_len = int(qls.max()) if qls.size else 1
    if np.any(lens < qls) or np.any(lens < 1):
        raise ValueError("every sequence must hold at least its query tokens (and one token)")
    B = int(lens.size)
    bs = BLOCK_SIZE
    nblk = (lens + bs - 1) // bs
    ring_blocks = 0
    if ring:
        if window <= 0:
            raise ValueError("a ring cache needs a window")
        ring_blocks = -(-(window + q_len - 1) // bs)
        nblk = np.minimum(nblk, ring_blocks)
        if max_blocks is None:
            max_blocks = ring_blocks
    if head_scales and kv_dtype != "int8":
        raise ValueError("per-head scales are for int8 caches")
    need = int(nblk.sum())
    if num_blocks is None:
        num_blocks = max(need + 1, int(math.ceil(pool_slack * need)))
    if num_blocks <= need:
        raise ValueError("pool too small")
    if max_blocks is None:
        max_blocks = int(nblk.max()) if B else 1
    if max_blocks < (int(nblk.max()) if B else 0):
        raise ValueError("max_blocks too small for the longest sequence")
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)

    perm = rng.permutation(num_blocks).astype(np.int32)
    unused = perm[need:]
    table = np.zeros((B, max(1, max_blocks)), dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        table[b, :n] = perm[off:off + n]
        off += n

    q_start = None
    if q_lens is not None:
        q_start = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
        qf = _standard_normal(rng, (int(q_start[-1]), num_q_heads, head_dim))
    else:
        qf = _standard_normal(rng, (B, q_len, num_q_heads, head_dim))
    if q_dtype == "f32":
        q = qf
    elif q_dtype == "bf16":
        q = f32_to_bf16_bits(qf)
    else:
        raise ValueError(f"unknown q dtype {q_dtype!r}")
    del qf

    shape = (num_blocks, bs, num_kv_heads, head_dim)
    k_pool, k_scale = _draw_kv(rng, shape, kv_dtype, head_scales)
    if alias_v:
        v_pool, v_scale = k_pool, k_scale
    else:
        v_pool, v_scale = _draw_kv(rng, shape, kv_dtype, head_scales)

    if poison:
        pools = [(k_pool, k_scale)] if alias_v else [(k_pool, k_scale), (v_pool, v_scale)]
        poison_block = int(unused[0])
        for b in range(B):
            n = int(nblk[b])
            table[b, n:] = poison_block
        for pool, sc in pools:
            _poison_slots(pool, sc, unused, slice(None), kv_dtype)
            if ring_blocks:
                _poison_ring(pool, sc, table, lens, nblk, ring_blocks, qls, window, kv_dtype)
                continue
            for b in range(B):
                L = int(lens[b])
                n = int(nblk[b])
                tail = L - (n - 1) * bs
                if tail < bs:
                    _poison_slots(pool, sc, table[b, n - 1], slice(tail, bs), kv_dtype)
                if window > 0:
                    first_key = max(0, L - int(qls[b]) - window + 1)
                    full = first_key // bs
                    if full:
                        _poison_slots(pool, sc, table[b, :full], slice(None), kv_dtype)
                    if first_key % bs:
                        _poison_slots(pool, sc, table[b, full], slice(0, first_key % bs), kv_dtype)

    return PagedInputs(q=q, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale, v_scale=v_scale,
                       block_table=table, seq_lens=lens.astype(np.int32), q_len=q_len,
                       num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                       window=int(window), scale=float(scale), q_dtype=q_dtype, kv_dtype=kv_dtype,
                       name=name, seed=seed, ring_blocks=ring_blocks, q_start=q_start)


def _poison_ring(pool, sc, table, lens, nblk, R, qls, window, kv_dtype):
    """Poison every ring slot that holds no key a query of the step may see.

    Ring slot e*16 + s holds the newest position t <= L-1 with t = e*16 + s
    (mod 16R); it is visible when t >= L - q_len - window + 1 (and t >= 0)."""
    bs = BLOCK_SIZE
    C = R * bs
    for b in range(table.shape[0]):
        L = int(lens[b])
        lo = max(0, L - int(qls[b]) - window + 1)
        for e in range(int(nblk[b])):
            r = e * bs + np.arange(bs)
            t = (L - 1) - ((L - 1 - r) % C)
            bad = np.nonzero((t < lo) | (t < 0))[0]
            if bad.size:
                _poison_slots(pool, sc, int(table[b, e]), bad, kv_dtype)


# The five workloads. Each entry fixes the shape; lengths are drawn from the
# config's own generator (seed = config number) before anything else.
CONFIGS = {
    1: dict(name="tiny-f32", B=2, q_len=1, Hq=4, Hkv=2, D=64, window=0, q_dtype="f32",
            kv_dtype="f32", lens="fixed:37,70", num_blocks=16, max_len=70),
    2: dict(name="gemma4-12b-local-bf16", B=32, q_len=1, Hq=16, Hkv=8, D=256, window=1024,
            q_dtype="bf16", kv_dtype="bf16", lens="uniform:512,8192", max_len=8192),
    3: dict(name="gemma4-12b-global-bf16", B=16, q_len=1, Hq=16, Hkv=1, D=256, window=0,
            q_dtype="bf16", kv_dtype="bf16", lens="uniform:4096,32768", max_len=32768, alias_v=True),
    4: dict(name="gqa70b-int8kv", B=64, q_len=1, Hq=64, Hkv=8, D=128, window=0,
            q_dtype="bf16", kv_dtype="int8", lens="uniform:1024,4096", max_len=4096),
    5: dict(name="verify5-bf16", B=256, q_len=5, Hq=32, Hkv=8, D=128, window=0,
            q_dtype="bf16", kv_dtype="bf16", lens="lognormal:1024,1.0,16,16384", max_len=16384),
}


# Prefill chunks (Lab 5, "Flash Attention": prefill with q_len > 1 over cached
# history, global and window layers). Each sequence brings `chunk` query
# tokens after a history drawn from `hist`; shapes are those of the decode
# workloads' layers.
PREFILL_CONFIGS = {
    1: dict(name="gemma4-12b-local-prefill", B=4, chunk=2048, hist="uniform:0,6144", Hq=16, Hkv=8, D=256,
            window=1024, kv_dtype="bf16"),
    2: dict(name="gemma4-12b-global-prefill", B=2, chunk=4096, hist="uniform:0,4096", Hq=16, Hkv=1, D=256,
            window=0, kv_dtype="bf16", alias_v=True),
    3: dict(name="gqa70b-int8kv-prefill", B=4, chunk=2048, hist="uniform:0,2048", Hq=64, Hkv=8, D=128,
            window=0, kv_dtype="int8"),
}


def make_prefill_config(idx: int, *, poison: bool = False) -> PagedInputs:
    """One of the prefill workloads, seeded with 100 + its number."""
    c = PREFILL_CONFIGS[idx]
    rng = np.random.default_rng(100 + idx)
    hist = _draw_lens(c["hist"], c["B"], rng)
    q_lens = np.full(c["B"], c["chunk"], dtype=np.int64)
    return make_inputs(hist + q_lens, q_len=1, q_lens=q_lens, num_q_heads=c["Hq"], num_kv_heads=c["Hkv"],
                       head_dim=c["D"], q_dtype="bf16", kv_dtype=c["kv_dtype"], window=c["window"], rng=rng,
                       alias_v=c.get("alias_v", False), poison=poison, name=c["name"], seed=100 + idx)


def _draw_lens(spec: str, B: int, rng: np.random.Generator) -> np.ndarray:
    kind, arg = spec.split(":", 1)
    if kind == "fixed":
        lens = np.array([int(v) for v in arg.split(",")], dtype=np.int64)
        assert lens.size == B
        return lens
    if kind == "uniform":
        lo, hi = (int(v) for v in arg.split(","))
        return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = arg.split(",")
        x = rng.lognormal(mean=math.log(float(median)), sigma=float(sigma), size=B)
        return np.clip(np.rint(x), int(lo), int(hi)).astype(np.int64)
    raise ValueError(spec)


def make_config(idx: int, *, poison: bool = False, batch: Optional[int] = None, ring: bool = False,
                head_scales: bool = False) -> PagedInputs:
    """One of the five named workloads, seeded with its own number.

    ``batch`` keeps only the first ``batch`` sequences of the drawn length
    list (a smaller problem with the same length distribution and pool rule).
    ``ring`` lays a window layer's cache out as rings; ``head_scales`` gives
    an int8 cache one scale per KV head.
    """
    c = CONFIGS[idx]
    rng = np.random.default_rng(idx)
    lens = _draw_lens(c["lens"], c["B"], rng)
    if batch is not None:
        lens = lens[:batch]
    num_blocks = c.get("num_blocks")
    max_blocks = None if ring else (c["max_len"] + BLOCK_SIZE - 1) // BLOCK_SIZE
    name = c["name"] + ("-ring" if ring else "") + ("-headscale" if head_scales else "")
    return make_inputs(lens, q_len=c["q_len"], num_q_heads=c["Hq"], num_kv_heads=c["Hkv"],
                       head_dim=c["D"], q_dtype=c["q_dtype"], kv_dtype=c["kv_dtype"],
                       window=c["window"], rng=rng, num_blocks=num_blocks,
                       max_blocks=max_blocks, alias_v=c.get("alias_v", False), poison=poison,
                       name=name, seed=idx, ring=ring, head_scales=head_scales)
