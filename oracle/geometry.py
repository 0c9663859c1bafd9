"""Shard geometry: contiguous, equal row ranges of the padded table.

[VS] paragraph 1: for an even split every shard owns a contiguous subset of
the table's rows; a shard tests whether a global ID falls in its subset and
turns owned IDs into local row indices. [TP] "Embedding
(VocabDimShardedEmbedding)": shard k holds rows [k*V/n, (k+1)*V/n).
[VS] paragraph 4: padded rows (at or past V_real) are not classes, so no shard
owns them.

Pinned by tests/test_oracle_pins.py::test_geometry_* (hand-written boundary
cases and exhaustive one-owner reconstruction).
"""

import numpy as np


def shard_size(V_pad: int, num_shards: int) -> int:
    if num_shards < 1 or V_pad % num_shards:
        raise ValueError("V_pad must be a positive multiple of num_shards")
    return V_pad // num_shards


def owner_and_local(ids, V_real: int, V_pad: int, num_shards: int):
    """Return (owner, local) int64 arrays: owner = -1 and local = 0 where no shard owns the ID.

    Each shard applies its own membership test, and the local index is formed
    only for IDs that passed it (the global ID is never used as an index).
    """
    ids = np.asarray(ids, dtype=np.int64)
    S = shard_size(V_pad, num_shards)
    owner = np.full(ids.shape, -1, dtype=np.int64)
    local = np.zeros(ids.shape, dtype=np.int64)
    for k in range(num_shards):
        lo, hi = k * S, min((k + 1) * S, V_real)
        mine = (ids >= lo) & (ids < hi)
        owner[mine] = k
        local[mine] = ids[mine] - lo
    return owner, local
