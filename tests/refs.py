"""Independent CPU references used to pin the oracle (tests only).

``dense_sdpa`` rebuilds each sequence's cache as a contiguous tensor with
numpy fancy indexing (the "gather first, then run ordinary attention"
formulation of the Lab 5 handout's "Paged Attention" section), then calls
torch's own scaled_dot_product_attention in float64 with an explicit boolean
band mask (the "compute, then mask" formulation of the handout's "Sliding
Window Attention" section) and torch's own GQA head expansion. None of it
goes through the oracle's index arithmetic.
"""

from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def storage_to_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def contiguous_cache(x, b: int):
    """K, V of sequence b as [L, Hkv, D] float64 (int8 dequantized)."""
    L = int(x.seq_lens[b])
    nblk = (L + x.block_size - 1) // x.block_size
    blocks = x.block_table[b, :nblk]
    k = storage_to_f64(x.k_pool[blocks]).reshape(nblk * x.block_size, x.num_kv_heads, x.head_dim)[:L]
    v = storage_to_f64(x.v_pool[blocks]).reshape(nblk * x.block_size, x.num_kv_heads, x.head_dim)[:L]
    if x.kv_dtype == "int8":
        # scales are [block, head, slot]: bring slots next to blocks, then flatten tokens
        ks = x.k_scale[blocks].transpose(0, 2, 1).astype(np.float64).reshape(-1, x.num_kv_heads)[:L]
        vs = x.v_scale[blocks].transpose(0, 2, 1).astype(np.float64).reshape(-1, x.num_kv_heads)[:L]
        k = k * ks[..., None]
        v = v * vs[..., None]
    return k, v


def band_mask(L: int, q_len: int, window: int) -> np.ndarray:
    """[q_len, L] bool: True where query t may see key j."""
    pos = np.arange(L - q_len, L)[:, None]
    keys = np.arange(L)[None, :]
    ok = keys <= pos
    if window > 0:
        ok &= keys > pos - window
    return ok


def dense_sdpa(x) -> np.ndarray:
    """[B, q_len, Hq, D] float64 via torch SDPA on contiguous copies."""
    q_all = storage_to_f64(x.q)
    out = np.empty(q_all.shape, dtype=np.float64)
    for b in range(x.batch):
        k, v = contiguous_cache(x, b)
        L = k.shape[0]
        mask_np = band_mask(L, x.q_len, x.window)
        # Keys no query may see can hold anything (the tests poison them with NaN);
        # zero them so the mask, not the arithmetic on them, removes them.
        unseen = ~mask_np.any(axis=0)
        k[unseen] = 0.0
        v[unseen] = 0.0
        q = torch.from_numpy(q_all[b]).permute(1, 0, 2)[None]          # [1, Hq, q_len, D]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()  # [1, Hkv, L, D]
        vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
        mask = torch.from_numpy(mask_np)[None, None]
        o = F.scaled_dot_product_attention(q, kt, vt, attn_mask=mask, scale=x.scale,
                                           enable_gqa=x.num_q_heads != x.num_kv_heads)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


def dense_sdpa_packed(x) -> np.ndarray:
    """[total, Hq, D] float64 for packed (prefill) queries, sequence by sequence, as dense_sdpa."""
    q_all = storage_to_f64(x.q)
    out = np.empty(q_all.shape, dtype=np.float64)
    for b in range(x.batch):
        a, e = int(x.q_start[b]), int(x.q_start[b + 1])
        if e == a:
            continue
        k, v = contiguous_cache(x, b)
        L = k.shape[0]
        mask_np = band_mask(L, e - a, x.window)
        unseen = ~mask_np.any(axis=0)
        k[unseen] = 0.0
        v[unseen] = 0.0
        q = torch.from_numpy(q_all[a:e]).permute(1, 0, 2)[None]
        kt = torch.from_numpy(k).permute(1, 0, 2)[None].contiguous()
        vt = torch.from_numpy(v).permute(1, 0, 2)[None].contiguous()
        mask = torch.from_numpy(mask_np)[None, None]
        o = F.scaled_dot_product_attention(q, kt, vt, attn_mask=mask, scale=x.scale,
                                           enable_gqa=x.num_q_heads != x.num_kv_heads)
        out[a:e] = o[0].permute(1, 0, 2).numpy()
    return out
