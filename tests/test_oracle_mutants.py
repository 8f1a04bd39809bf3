"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is oracle.c rebuilt with ``-DORC_MUTANT=n`` (a wrong GQA head
map, a window one key too wide, verify rows all placed at the last position,
slot and head swapped in the pool address, the score scale dropped, the
softmax left unnormalised, the key scale used for values, one dimension left
out of the dot product; in the KV append, an int8 scale of max/128, codes
truncated instead of rounded, the scale stored [block][slot][head]; a ring
slot taken modulo the window instead of the ring; head 0's per-head scale
used for every head, in attention and in the append). The pins of
test_oracle_pins.py, test_oracle_append.py and test_oracle_ring.py run
against it; the mutant survives only if every pin still passes.
"""

from __future__ import annotations

import os
import tempfile

import pytest

import oracle
from tests import test_oracle_append as append_pins
from tests import test_oracle_pins as pins
from tests import test_oracle_prefill as prefill_pins
from tests import test_oracle_ring as ring_pins

MUTANTS = {
    1: "GQA head map h % Hkv",
    2: "window admits W+1 keys",
    3: "every verify row placed at the last position",
    4: "slot and head swapped in the pool address",
    5: "score scale dropped",
    6: "softmax not normalised",
    7: "key scale applied to values",
    8: "first dimension left out of the dot product",
    9: "append: int8 scale max over 128",
    10: "append: int8 codes truncated",
    11: "append: scale stored block-slot-head",
    12: "ring slot taken modulo the window instead of the ring",
    13: "per-head scale of head 0 for every head",
    14: "per-head append quantizes with head 0's scale",
}

PIN_CALLS = [
    lambda: [pins.test_matches_torch_sdpa(c) for c in pins.SDPA_CASES],
    pins.test_single_key_returns_value,
    pins.test_window_one_returns_own_value,
    pins.test_equal_keys_give_mean_value,
    pins.test_unit_values_give_ones,
    pins.test_verify_rows_equal_sequential_decode,
    pins.test_gqa_equals_expanded_heads,
    pins.test_visited_blocks_closed_form,
    pins.test_gather_matches_fancy_indexing,
    lambda: [pins.test_golden_closed_forms(p) for p in
             sorted(os.path.join(pins.GOLDEN, f) for f in os.listdir(pins.GOLDEN)
                    if f.endswith(".json") and "k_tokens" in open(os.path.join(pins.GOLDEN, f)).read())],
    lambda: [append_pins.test_float_append_is_a_copy(k) for k in ("f32", "bf16")],
    append_pins.test_int8_codes_in_range_with_the_peak_at_127,
    append_pins.test_int8_zero_row_has_unit_scale_and_zero_codes,
    append_pins.test_int8_exact_multiples_come_back_exactly,
    append_pins.test_int8_dequantized_row_is_within_half_a_step,
    append_pins.test_int8_negation_negates_codes,
    append_pins.test_int8_scale_of_head_g_lands_at_block_head_slot,
    lambda: [ring_pins.test_ring_equals_linear(i) for i in range(len(ring_pins.RING_CASES))],
    lambda: [ring_pins.test_ring_visits_closed_form(i) for i in range(len(ring_pins.RING_CASES))],
    lambda: [ring_pins.test_per_head_scales_equal_repeated_per_token_scales(w, q) for w, q in ((0, 1), (20, 1))],
    ring_pins.test_per_head_append_codes,
    lambda: [prefill_pins.test_prefill_matches_torch_sdpa(i) for i in range(len(prefill_pins.CASES))],
]


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as d:
        path = oracle.build(extra_flags=[f"-DORC_MUTANT={mutant}"], out=os.path.join(d, "mut.so"))
        caught = []
        with oracle.use_variant(path):
            for call in PIN_CALLS:
                try:
                    call()
                except (AssertionError, oracle.OracleError):
                    caught.append(call)
        assert caught, f"no pin caught mutant {mutant}: {MUTANTS[mutant]}"
