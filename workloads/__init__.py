"""Seeded synthetic inputs for one paged decode-attention step.

This package is shared by the tests, the benchmark and the smoke check. It
draws random numbers and lays them out in the paged-cache format; it holds no
attention arithmetic and imports neither the HIP library nor the oracle.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    PREFILL_CONFIGS,
    PagedInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_config,
    make_inputs,
    make_prefill_config,
)
