"""Pools past 4 GiB: the kernels address blocks at the top of a large pool.

A small problem's blocks are moved to the top of a device pool of more than
4.5 GiB per tensor, and its block table is shifted to match. The lower blocks
are never written or read. Every cache row (and, for int8, every scale) that
the kernels touch then lies beyond byte 2^32 of its allocation, so 32-bit
offset arithmetic anywhere on the path would read or write the wrong place.
The append, decode (vector and matrix-core kernels, bf16 and int8), the
verify step and prefill run there. Their results are compared with the
oracle on the small problem: bit for bit for the append, to the attention
tolerance for the rest.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_94_amd as pa
from tests.gpu_util import TOL, Dev, max_err, to_torch
from workloads import f32_to_bf16_bits, make_inputs

pytestmark = pytest.mark.gpu
LARGE = int(4.5 * 2**30)
BS = 16


def _lift(dev: Dev, x) -> int:
    """Move dev's pools (and per-token scales) to the top of pools of more than LARGE bytes; return the shift."""
    nb = x.k_pool.shape[0]
    block_bytes = dev.k[0].numel() * dev.k.element_size()
    total = max(nb, LARGE // block_bytes + 1)
    off = total - nb

    def big(t):
        if t is None or t.dim() == 1:            # absent, or one scale per KV head
            return t
        out = torch.empty((total,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        out[off:].copy_(t)
        return out

    v_alias, s_alias = dev.v is dev.k, dev.vs is dev.ks
    dev.k = big(dev.k)
    dev.v = dev.k if v_alias else big(dev.v)
    dev.ks = big(dev.ks)
    dev.vs = dev.ks if s_alias else big(dev.vs)
    dev.table = dev.table + off
    assert dev.k.numel() * dev.k.element_size() > LARGE
    return off


def _free(dev: Dev):
    dev.k = dev.v = dev.ks = dev.vs = None
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv,q_len,Hq,Hkv,D,kernel", [
    ("bf16", 1, 16, 8, 128, 0),      # vector kernel
    ("bf16", 1, 16, 1, 256, 1),      # matrix-core kernel, one KV head
    ("int8", 1, 64, 8, 128, 1),      # int8 cache, per-token scales
    ("bf16", 5, 32, 8, 128, 1),      # verify step
])
def test_attention_at_the_top_of_a_large_pool(kv, q_len, Hq, Hkv, D, kernel):
    x = make_inputs([37, 300, 1000, 16, 129], q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                    q_dtype="bf16", kv_dtype=kv, seed=90 + D + q_len, poison=True)
    dev = Dev(x)
    off = _lift(dev, x)
    print(f"large pool {kv} q_len={q_len} Hq={Hq} Hkv={Hkv} D={D}: block shift {off}", flush=True)
    assert dev.plan()["kernel"] == kernel
    got = dev.run_f64()
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    _free(dev)
    assert not np.isnan(got).any()
    err = max_err(got, ref)
    assert err <= TOL[kv], err


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_prefill_at_the_top_of_a_large_pool(kv):
    x = make_inputs([40, 700, 1300], q_len=1, q_lens=[40, 300, 17], num_q_heads=16, num_kv_heads=8, head_dim=128,
                    q_dtype="bf16", kv_dtype=kv, seed=95, poison=True)
    dev = Dev(x)
    off = _lift(dev, x)
    print(f"large pool prefill {kv}: block shift {off}", flush=True)
    out = torch.full_like(dev.q, float("nan"))
    pa.prefill(out, dev.q, to_torch(x.q_start), dev.k, dev.v, dev.table, dev.lens, max_q_len=x.q_len,
               window=x.window, scale=x.scale, max_seq_len=x.max_seq_len, k_scale=dev.ks, v_scale=dev.vs)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    _free(dev)
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    assert not np.isnan(got).any()
    err = max_err(got, ref)
    assert err <= TOL[kv], err


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_append_at_the_top_of_a_large_pool(kv):
    """Append each sequence's last token into the lifted pools; the lifted region must match the oracle's pools."""
    x = make_inputs([37, 300, 129, 16], q_len=1, num_q_heads=16, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                    kv_dtype=kv, seed=97, poison=False)
    rng = np.random.default_rng(97)
    T = x.batch
    slots = np.asarray([int(x.block_table[b, (L - 1) // BS]) * BS + (L - 1) % BS
                        for b, L in enumerate(x.seq_lens)], dtype=np.int64)
    k = rng.standard_normal((T, x.num_kv_heads, x.head_dim)).astype(np.float32)
    v = rng.standard_normal((T, x.num_kv_heads, x.head_dim)).astype(np.float32)
    if kv == "bf16":                              # bf16 rows (as bit patterns) into a bf16 pool
        k, v = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    dev = Dev(x)
    off = _lift(dev, x)
    print(f"large pool append {kv}: block shift {off}, top slot byte offset "
          f"{(int(slots.max()) + off * BS) * x.num_kv_heads * x.head_dim * dev.k.element_size()}", flush=True)
    dk, dv = to_torch(k), to_torch(v)
    pa.cache_write(dk, dv, to_torch(slots + off * BS), dev.k, dev.v, dev.ks, dev.vs)
    torch.cuda.synchronize()
    oracle.cache_write(k, v, slots, x.k_pool, x.v_pool, x.k_scale, x.v_scale)
    pairs = [(dev.k, x.k_pool), (dev.v, x.v_pool), (dev.ks, x.k_scale), (dev.vs, x.v_scale)]
    for got, exp in pairs:
        if exp is not None:
            top = got[off:].contiguous()
            host = top.view(torch.int16) if top.dtype == torch.bfloat16 else top
            assert host.cpu().numpy().tobytes() == exp.tobytes()
    got = dev.run_f64()
    _free(dev)
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    assert not np.isnan(got).any()
    assert max_err(got, ref) <= TOL[kv]
