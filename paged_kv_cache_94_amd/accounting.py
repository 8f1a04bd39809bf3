"""Bytes and flops a paged decode-attention step must move and compute.

The cache-size rule is the CS336 lecture 10 study guide's KV formula,
M_KV = 2 * layers * tokens * n_kv * d_h * bytes_per_element (K and V), and
the tiniestgpt notes' "KV bytes per token" line. The per-call algorithmic
byte count applies it to exactly the keys a step must read:

    alg_bytes = sum_b T_b * Hkv * D * (e_K + e_V * [V not shared with K])
              + sum_b T_b * Hkv * 8 * [int8 cache]       (two fp32 scales per token per head)
              + bytes(Q) + bytes(out)
              + 4 * sum_b touched_blocks_b + 4 * B        (block-table entries, seq_lens)

with T_b the keys some query of sequence b may see (min(L_b, W + q_len - 1)
under a window W, else L_b). Keys outside the window, the tail of the last
block and the split partials are not counted: a kernel that moves them pays
for them in achieved bandwidth.

Flops: 4 * D per (query row, visible key) -- a multiply-add for q.k and
another for p.v, as in the study guide's attention intensity estimate
(4 * B * S * T * D for T queries over S keys).
"""

from __future__ import annotations

import numpy as np

BLOCK = 16


def kv_bytes_per_token_per_layer(n_kv: int, d_h: int, bytes_per_elem: int) -> int:
    """K and V bytes one token adds to one layer's cache."""
    return 2 * n_kv * d_h * bytes_per_elem


def kv_cache_bytes(layers: int, tokens: int, n_kv: int, d_h: int, bytes_per_elem: int) -> int:
    """M_KV for one sequence (CS336 lecture 10 study guide, KV cache size)."""
    return layers * tokens * kv_bytes_per_token_per_layer(n_kv, d_h, bytes_per_elem)


def visible_keys(seq_lens, q_len: int, window: int) -> np.ndarray:
    """Keys at least one query of each sequence may see."""
    L = np.asarray(seq_lens, dtype=np.int64)
    if window > 0:
        return np.minimum(L, window + q_len - 1)
    return L


def touched_blocks(seq_lens, q_len: int, window: int) -> np.ndarray:
    """Whole 16-token blocks holding a visible key, per sequence."""
    L = np.asarray(seq_lens, dtype=np.int64)
    first = np.maximum(0, L - q_len - window + 1) if window > 0 else np.zeros_like(L)
    return (L - 1) // BLOCK - first // BLOCK + 1


_ELEM = {"f32": 4, "bf16": 2, "int8": 1}


def step_bytes(seq_lens, *, q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int, q_dtype: str,
               kv_dtype: str, window: int, v_shares_k: bool, token_scales: bool = True) -> int:
    """Algorithmic HBM bytes of one step (see the module docstring)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B = int(L.size)
    T = int(visible_keys(L, q_len, window).sum())
    e_kv = _ELEM[kv_dtype]
    e_q = _ELEM[q_dtype]
    kv = T * num_kv_heads * head_dim * e_kv * (1 if v_shares_k else 2)
    if kv_dtype == "int8":   # per-token scales; per-head ones are 8 bytes per head in all
        kv += (T if token_scales else 1) * num_kv_heads * 4 * (1 if v_shares_k else 2)
    qo = 2 * B * q_len * num_q_heads * head_dim * e_q
    meta = 4 * int(touched_blocks(L, q_len, window).sum()) + 4 * B
    return int(kv + qo + meta)


def touched_kv_bytes(seq_lens, *, q_len: int, num_kv_heads: int, head_dim: int, kv_dtype: str, window: int,
                     v_shares_k: bool, token_scales: bool = True) -> int:
    """Cache bytes in the whole blocks a block-skipping kernel reads."""
    nblk = int(touched_blocks(seq_lens, q_len, window).sum())
    per_tok = num_kv_heads * head_dim * _ELEM[kv_dtype] + (num_kv_heads * 4 if kv_dtype == "int8" and token_scales
                                                           else 0)
    return nblk * BLOCK * per_tok * (1 if v_shares_k else 2)


def step_flops(seq_lens, *, q_len: int, num_q_heads: int, head_dim: int, window: int) -> int:
    """4 * D per (query row, visible key)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    total = 0
    for t in range(q_len):
        p = L - q_len + t
        lo = np.maximum(0, p - window + 1) if window > 0 else np.zeros_like(p)
        total += int((p - lo + 1).sum())
    return 4 * head_dim * num_q_heads * total


def append_bytes(tokens: int, *, num_kv_heads: int, head_dim: int, src_dtype: str, kv_dtype: str,
                 v_shares_k: bool) -> int:
    """Algorithmic HBM bytes of one KV append of `tokens` rows per KV head.

    Each (token, head) row is read once in the source dtype and written once
    in the cache dtype, for K and for V unless V is K; an int8 cache adds
    one fp32 scale per row; each token's int64 slot id is read once.
    """
    per_row = head_dim * (_ELEM[src_dtype] + _ELEM[kv_dtype]) + (4 if kv_dtype == "int8" else 0)
    return int(tokens * (8 + num_kv_heads * per_row * (1 if v_shares_k else 2)))


def prefill_flops(seq_lens, q_lens, *, num_q_heads: int, head_dim: int, window: int) -> int:
    """4 * D per (query row, visible key) for packed chunks: query t of a chunk of n
    sits at L - n + t and sees min(p + 1, W) keys (p + 1 without a window)."""
    total = 0
    for L, n in zip(np.asarray(seq_lens, dtype=np.int64), np.asarray(q_lens, dtype=np.int64)):
        p = np.arange(L - n, L)
        vis = p + 1 if window <= 0 else np.minimum(p + 1, window)
        total += int(vis.sum())
    return 4 * head_dim * num_q_heads * total


def for_inputs(x) -> dict:
    """Byte / flop accounting for a PagedInputs-like object."""
    if getattr(x, "q_start", None) is not None:   # packed prefill chunks
        q_lens = np.diff(x.q_start)
        e = _ELEM[x.kv_dtype] * (1 if x.v_pool is x.k_pool else 2)
        keys = sum(int(min(L, x.window + n - 1)) if x.window > 0 else int(L) for L, n in zip(x.seq_lens, q_lens))
        kv = keys * x.num_kv_heads * x.head_dim * e
        return {
            "alg_bytes": int(kv + 2 * x.q.size * 2),
            "flops": prefill_flops(x.seq_lens, q_lens, num_q_heads=x.num_q_heads, head_dim=x.head_dim,
                                   window=x.window),
            "queries": int(x.q_start[-1]),
        }
    kw = dict(q_len=x.q_len, num_kv_heads=x.num_kv_heads, head_dim=x.head_dim, kv_dtype=x.kv_dtype,
              window=x.window, v_shares_k=x.v_pool is x.k_pool,
              token_scales=x.k_scale is None or x.k_scale.ndim == 3)
    return {
        "alg_bytes": step_bytes(x.seq_lens, num_q_heads=x.num_q_heads, q_dtype=x.q_dtype, **kw),
        "touched_kv_bytes": touched_kv_bytes(x.seq_lens, **kw),
        "flops": step_flops(x.seq_lens, q_len=x.q_len, num_q_heads=x.num_q_heads, head_dim=x.head_dim,
                            window=x.window),
        "queries": int(x.seq_lens.size) * x.q_len,
    }
