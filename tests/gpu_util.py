"""Helpers for the GPU tests: upload seeded inputs, run an entry point, compare."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_94_amd as pa

TOL = {"f32": 1e-5, "bf16": 1e-2, "int8": 1e-2}


def to_torch(a: np.ndarray, device="cuda"):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class Dev:
    """Device copies of a PagedInputs problem (the same tensor for K and V when shared)."""

    def __init__(self, x, device="cuda"):
        self.x = x
        self.q = to_torch(x.q, device)
        self.k = to_torch(x.k_pool, device)
        self.v = self.k if x.v_pool is x.k_pool else to_torch(x.v_pool, device)
        self.ks = None if x.k_scale is None else to_torch(x.k_scale, device)
        self.vs = None if x.v_scale is None else (self.ks if x.v_scale is x.k_scale else to_torch(x.v_scale, device))
        self.table = to_torch(x.block_table, device)
        self.lens = to_torch(x.seq_lens, device)

    def run(self, entry=None, **kw):
        x = self.x
        out = torch.full_like(self.q, float("nan"))
        kw.setdefault("window", x.window)
        kw.setdefault("scale", x.scale)
        kw.setdefault("max_seq_len", x.max_seq_len)
        kw.setdefault("ring_blocks", getattr(x, "ring_blocks", 0))
        if entry is None:
            entry = "verify" if x.q_len > 1 else ("decode_int8" if x.kv_dtype == "int8" else "decode")
        if entry == "decode_int8":
            pa.decode_int8(out, self.q, self.k, self.v, self.table, self.lens, self.ks, self.vs, **kw)
        elif entry == "verify":
            pa.verify(out, self.q, self.k, self.v, self.table, self.lens, k_scale=self.ks, v_scale=self.vs, **kw)
        else:
            pa.decode(out, self.q, self.k, self.v, self.table, self.lens, **kw)
        torch.cuda.synchronize()
        return out

    def plan(self, **kw) -> dict:
        x = self.x
        kw.setdefault("window", x.window)
        kw.setdefault("scale", x.scale)
        kw.setdefault("max_seq_len", x.max_seq_len)
        kw.setdefault("ring_blocks", getattr(x, "ring_blocks", 0))
        return pa.plan(self.q, self.k, self.v, self.table, self.lens, k_scale=self.ks, v_scale=self.vs, **kw)

    def run_f64(self, **kw) -> np.ndarray:
        return self.run(**kw).float().cpu().numpy().astype(np.float64)


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
