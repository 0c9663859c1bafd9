"""Seeded synthetic inputs for the vocabulary-sharded cross-entropy and embedding path.

This package only draws random numbers and lays them out as arrays (token IDs,
targets, hidden rows, table rows, permutations). It holds none of the method's
arithmetic: no logits, no softmax, no owner tests, no reductions over the
vocabulary. Both the float64 oracle side (through the tests) and the GPU side
(through the tests and the bench) take their inputs from here, so the two see
the same bits.
"""

from .gen import (  # noqa: F401
    bf16_bits_from_f32,
    zipf_ids,
    CEInputs,
    make_ce_inputs,
    make_tied_inputs,
    make_oth_inputs,
    make_sampled_inputs,
    make_layout,
    make_row_map,
)
from .configs import CONFIGS, config_inputs  # noqa: F401
