"""Float64 CPU oracle for the vocabulary-sharded LM-head cross-entropy and the
masked embedding lookup over one tied table.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check of the graft entry point
and the bench's CPU-baseline leg may import this package; the library, its HIP
kernels and its Python binding never do, and this package imports nothing from
them. It computes the plain definitions of what the GPU path computes, in
float64 with numpy (OpenBLAS for the matrix products), slowly and obviously.

Sources (page titles):
  [VS]  "Vocabulary shards: look up locally and normalize globally"
  [SP]  "Sequence-parallel normalization: shard tokens, retain their hidden features"
  [PAD] "Training collapses when token embeddings are not padded to a multiple of 64"
  [SS]  "Sampled Softmax with Over-Tokenized Transformer"
  [TP]  "Tensor Parallelism (TP)" (vLLM on Neuron design notes)

Each function says which passage it follows and which pinned test in
tests/test_oracle_pins.py holds it to something other than itself.
"""

from .bits import decode  # noqa: F401
from .geometry import shard_size, shard_bounds, owner_and_local, remap  # noqa: F401
from .embedding import gather_direct, gather_masked_shards, scatter_add  # noqa: F401
from .ce import (  # noqa: F401
    target_status, logits, lse_rows, shard_stats, merge_shard_stats, lse_two_phase,
    ce_forward, ce_backward, grad_scale, cross_entropy,
)
from .sampled import candidates, sampled_step  # noqa: F401
from .argmax import shard_argmax, merge_shard_argmax, greedy_argmax  # noqa: F401
from .tied import tied_step  # noqa: F401
from .oth import OT_H_WEIGHT, ot_h_step  # noqa: F401
from .ngram import mix64, ngram_backward, ngram_embed, ngram_ids  # noqa: F401
from . import parallel  # noqa: F401
