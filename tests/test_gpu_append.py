"""GPU parity of the KV append (pa_cache_write) against the oracle's append.

The append is integer / byte work once the binary32 quantizer has decided
the codes, and both sides decide them in binary32 with round-half-even, so
every comparison here is bit for bit: pool bytes, int8 codes, scales, and
the untouched rest of the pools. The last tests append a decode (or verify)
step's own tokens and then run the attention over the updated cache against
the oracle, to the attention tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_94_amd as pa
from tests.gpu_util import TOL, Dev, max_err, to_torch
from workloads import f32_to_bf16_bits, make_config, make_inputs

pytestmark = pytest.mark.gpu
BS = 16


def _log(msg):
    print(msg, flush=True)


def _host(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _rows(rng, T, hkv, d, src, edge=True):
    # Attention tests draw N(0, 1) like the workloads (the attention tolerance assumes
    # outputs of that size: bf16 rounding alone is 2^-9 relative) and leave out the edge
    # rows: all zero (scale 1), exact round-half ties at scale 1, wide dynamic range, one
    # subnormal row, one row of equal magnitudes.
    x = (rng.standard_normal((T, hkv, d)) * (2.0 if edge else 1.0)).astype(np.float32)
    if edge and T > 5:
        x[0] = 0.0
        x[1] = 0.5 * ((np.arange(d) % 9) - 4.0)                      # multiples of 0.5: 2.5 -> 2, -3.5 -> -4
        x[1, :, 0] = 127.0
        x[2] = (rng.standard_normal((hkv, d)) * np.float32(1e-3)).astype(np.float32)
        x[2, :, 1] = 3.0e4
        x[3] = np.float32(1e-39) * np.sign(rng.standard_normal((hkv, d))).astype(np.float32)
        x[4] = -7.0
    return f32_to_bf16_bits(x) if src == "bf16" else x


def _empty_pools(nb, hkv, d, kv):
    if kv == "int8":
        kp = np.full((nb, BS, hkv, d), 99, dtype=np.int8)
        ks = np.full((nb, hkv, BS), np.nan, dtype=np.float32)
        return kp, kp.copy(), ks, ks.copy()
    if kv == "bf16":
        kp = np.full((nb, BS, hkv, d), 0x7FC0, dtype=np.uint16)
    else:
        kp = np.full((nb, BS, hkv, d), np.nan, dtype=np.float32)
    return kp, kp.copy(), None, None


def _dev(a):
    return None if a is None else to_torch(a)


CASES = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "int8"), ("f32", "int8")]


@pytest.mark.parametrize("src,kv", CASES)
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("hkv", [1, 8])
def test_append_bit_exact(src, kv, d, hkv):
    rng = np.random.default_rng(1000 + 7 * d + hkv)
    nb, T = 9, 45
    k, v = _rows(rng, T, hkv, d, src), _rows(rng, T, hkv, d, src)
    slots = rng.permutation(nb * BS)[:T].astype(np.int64)
    slots[[5, 17]] = -1                       # skipped tokens
    bad = slots.copy()
    bad[30] = nb * BS + 3                     # outside the pool: never written
    slots[30] = -1
    kp, vp, ks, vs = _empty_pools(nb, hkv, d, kv)
    dk, dv, dks, dvs = _dev(kp), _dev(vp), _dev(ks), _dev(vs)
    _log(f"append {src}->{kv} D={d} Hkv={hkv} T={T}")
    pa.cache_write(_dev(k), _dev(v), _dev(bad), dk, dv, dks, dvs)
    torch.cuda.synchronize()
    oracle.cache_write(k, v, slots, kp, vp, ks, vs)
    for got, exp in ((dk, kp), (dv, vp), (dks, ks), (dvs, vs)):
        if exp is not None:
            assert _host(got).tobytes() == exp.tobytes()


@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_append_aliased_pool(kv):
    # v_pool is k_pool (and v_new is k_new): the rows land once; the result is a one-pool append.
    rng = np.random.default_rng(55)
    nb, hkv, d, T = 5, 2, 128, 33
    src = "bf16"
    k = _rows(rng, T, hkv, d, src)
    slots = rng.permutation(nb * BS)[:T].astype(np.int64)
    kp, vp, ks, vs = _empty_pools(nb, hkv, d, kv)
    dk, dks = _dev(kp), _dev(ks)
    dkn = _dev(k)
    pa.cache_write(dkn, dkn, _dev(slots), dk, dk, dks, dks)
    torch.cuda.synchronize()
    oracle.cache_write(k, k.copy(), slots, kp, vp, ks, vs)
    assert _host(dk).tobytes() == kp.tobytes()
    if ks is not None:
        assert _host(dks).tobytes() == ks.tobytes()


def test_append_zero_tokens_is_a_no_op():
    kp, vp, ks, vs = _empty_pools(2, 1, 64, "int8")
    dk, dv, dks, dvs = _dev(kp), _dev(vp), _dev(ks), _dev(vs)
    e = torch.empty((0, 1, 64), dtype=torch.float32, device="cuda")
    pa.cache_write(e, e, torch.empty((0,), dtype=torch.int64, device="cuda"), dk, dv, dks, dvs)
    torch.cuda.synchronize()
    assert _host(dk).tobytes() == kp.tobytes() and _host(dvs).tobytes() == vs.tobytes()


def _step_slots(x, positions_per_seq):
    """Global slot ids of the given logical positions, sequence by sequence."""
    out = []
    for b in range(x.batch):
        for pos in positions_per_seq(int(x.seq_lens[b])):
            out.append(int(x.block_table[b, pos // BS]) * BS + pos % BS)
    return np.asarray(out, dtype=np.int64)


def _append_then_attend(x, src, rng):
    """Append each sequence's last q_len tokens on both sides, then compare pools and attention."""
    T = x.batch * x.q_len
    slots = _step_slots(x, lambda L: range(L - x.q_len, L))
    k = _rows(rng, T, x.num_kv_heads, x.head_dim, src, edge=False)
    v = k if x.v_pool is x.k_pool else _rows(rng, T, x.num_kv_heads, x.head_dim, src, edge=False)
    dev = Dev(x)
    dk = _dev(k)
    dvn = dk if v is k else _dev(v)
    pa.cache_write(dk, dvn, _dev(slots), dev.k, dev.v, dev.ks, dev.vs)
    torch.cuda.synchronize()
    oracle.cache_write(k, v if v is not k else k.copy(), slots, x.k_pool, x.v_pool, x.k_scale, x.v_scale)
    pairs = [(dev.k, x.k_pool), (dev.v, x.v_pool), (dev.ks, x.k_scale), (dev.vs, x.v_scale)]
    for got, exp in pairs:
        if exp is not None:
            assert _host(got).tobytes() == exp.tobytes()
    got = dev.run_f64()
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    assert not np.isnan(got).any()
    return max_err(got, ref)


@pytest.mark.parametrize("kv,src,q_len,alias", [
    ("int8", "f32", 1, False), ("int8", "bf16", 1, False), ("bf16", "bf16", 1, False),
    ("bf16", "bf16", 5, False), ("bf16", "bf16", 1, True), ("f32", "f32", 1, False),
])
def test_append_then_attend(kv, src, q_len, alias):
    lens = [37, 70, 129, 300, 16, 17, 512]
    q_dtype = "f32" if kv == "f32" else "bf16"
    x = make_inputs(lens, q_len=q_len, num_q_heads=8, num_kv_heads=2, head_dim=128, q_dtype=q_dtype,
                    kv_dtype=kv, window=0, seed=77, alias_v=alias, poison=True, name="append-step")
    err = _append_then_attend(x, src, np.random.default_rng(78))
    _log(f"append+attend {kv}<-{src} q_len={q_len} alias={alias}: max|err| = {err:.3e}")
    assert err <= TOL[kv]


@pytest.mark.parametrize("idx,src", [(2, "bf16"), (4, "f32"), (4, "bf16"), (5, "bf16")])
def test_append_full_size_step(idx, src):
    # One decode / verify step of a full-size workload: every sequence's newest tokens go in,
    # every other pool row must keep its bytes, the written rows must match the oracle's.
    x = make_config(idx, poison=False)
    rng = np.random.default_rng(500 + idx)
    T = x.batch * x.q_len
    slots = _step_slots(x, lambda L: range(L - x.q_len, L))
    k = _rows(rng, T, x.num_kv_heads, x.head_dim, src)
    v = k if x.v_pool is x.k_pool else _rows(rng, T, x.num_kv_heads, x.head_dim, src)
    dev = Dev(x)
    before = {n: t.clone() for n, t in (("k", dev.k), ("v", dev.v), ("ks", dev.ks), ("vs", dev.vs)) if t is not None}
    _log(f"full-size append {x.name}: T={T} Hkv={x.num_kv_heads} D={x.head_dim} {src}->{x.kv_dtype}")
    dk = _dev(k)
    pa.cache_write(dk, dk if v is k else _dev(v), _dev(slots), dev.k, dev.v, dev.ks, dev.vs)
    torch.cuda.synchronize()
    oracle.cache_write(k, v if v is not k else k.copy(), slots, x.k_pool, x.v_pool, x.k_scale, x.v_scale)
    ds = torch.from_numpy(slots).cuda()
    for name, exp in (("k", x.k_pool), ("v", x.v_pool)):
        t = dev.k if name == "k" else dev.v
        flat = t.view(-1, x.num_kv_heads, x.head_dim)
        got = _host(flat[ds])
        assert got.tobytes() == exp.reshape(-1, x.num_kv_heads, x.head_dim)[slots].tobytes()
        changed = (flat.view(torch.uint8 if t.element_size() == 1 else torch.int16) !=
                   before[name].view(-1, x.num_kv_heads, x.head_dim).view(
                       torch.uint8 if t.element_size() == 1 else torch.int16)).flatten(1).any(1)
        outside = changed.clone()
        outside[ds] = False
        assert not bool(outside.any()), f"{name} rows outside the step's slots changed"
    if x.kv_dtype == "int8":
        for name, t, exp in (("ks", dev.ks, x.k_scale), ("vs", dev.vs, x.v_scale)):
            assert _host(t).tobytes() == exp.tobytes()
