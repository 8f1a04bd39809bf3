"""The split merge when many units are merged: parity with the fp64 oracle.

With 1024 or more merged units the combine launches one workgroup per unit,
and a wavefront whose unit has more than four query rows merges several of
them, the next row's loads in flight while the current one is merged. These
cases reach that instance for every head size and output type (a partial
row is D floats, so one load instruction covers 256/D splits), with units of
a few splits, of more than the 8 a first batch holds, and of more than the
64 one (m, l) load covers. Forced context splits (aligned) give
B * Hkv = 1024 merged units in each case.
"""

from __future__ import annotations

import zlib

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, Dev, max_err
from workloads import make_inputs

pytestmark = pytest.mark.gpu

# (q_len, Hq, Hkv, D, q_dtype, kv_dtype, B, splits, lens lo, lens hi)
CASES = [
    (2, 16, 4, 256, "bf16", "bf16", 256, 3, 40, 300),      # matrix-core kernel, 8 rows, D 256
    (4, 64, 8, 64, "bf16", "bf16", 128, 2, 40, 300),       # 32 rows (8 per wavefront), D 64
    (1, 32, 4, 64, "f32", "f32", 256, 2, 40, 300),         # vector kernel, fp32 output, 8 rows
    (1, 64, 8, 128, "bf16", "int8", 128, 3, 40, 300),      # int8 cache, 8 rows
    (5, 32, 8, 128, "bf16", "bf16", 128, 12, 150, 400),    # 20 rows, units of up to 9 splits (> 8)
    (2, 16, 4, 128, "bf16", "bf16", 256, 80, 1030, 1100),  # one block per split: up to 69 (> 64)
]


def _ids(c):
    q_len, hq, hkv, d, qd, kd, b, splits, lo, hi = c
    return f"q{q_len}_g{hq // hkv}_d{d}_{kd}_b{b}_s{splits}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_many_units_merged(case):
    q_len, hq, hkv, d, qd, kd, b, splits, lo, hi = case
    seed = zlib.crc32(repr(case).encode())
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, b).tolist()
    x = make_inputs(lens, q_len=q_len, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_dtype=qd, kv_dtype=kd,
                    poison=True, seed=seed)
    print(f"combine {_ids(case)}: lens {min(lens)}..{max(lens)}", flush=True)
    dev = Dev(x)
    plan = dev.plan(num_splits=splits)
    rows = hq // hkv * q_len
    assert plan["splits"] > 1 and plan["balanced"] == 0 and rows > 4 and b * hkv >= 1024
    assert plan["splits"] > {12: 8, 80: 64}.get(splits, 1)
    got = dev.run_f64(num_splits=splits)
    ref = oracle.attention(oracle.Problem.from_inputs(x))
    assert not np.isnan(got).any()
    err = max_err(got, ref)
    print(f"  plan splits {plan['splits']}, max|err| = {err:.3e}", flush=True)
    assert err <= TOL[kd]
