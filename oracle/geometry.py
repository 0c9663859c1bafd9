"""Shard geometry: contiguous, equal row ranges of the padded table.

[VS] paragraph 1: for an even split every shard owns a contiguous subset of
the table's rows; a shard tests whether a global ID falls in its subset and
turns owned IDs into local row indices. [TP] "Embedding
(VocabDimShardedEmbedding)": shard k holds rows [k*V/n, (k+1)*V/n).
[VS] paragraph 4: padded rows (at or past V_real) are not classes, so no shard
owns them.

[VS] paragraph 1 says this form is for an even split; [SP] paragraph 5 says
uneven layouts need explicit support. Explicit layouts: `shard_rows` lists
num_shards + 1 nondecreasing row offsets (0 first, V_pad last); shard k owns
rows [shard_rows[k], shard_rows[k+1]) (empty shards allowed). Explicitly
mapped ownership: classes are placed at physical rows by a permutation
row_of of [0, V_real) (the table is stored in physical order, shard by
shard); `remap` applies such a map to IDs and targets.

Pinned by tests/test_oracle_pins.py::test_geometry_* (hand-written boundary
cases and exhaustive one-owner reconstruction) and test_uneven_* / test_mapped_*.
"""

import numpy as np


def shard_size(V_pad: int, num_shards: int) -> int:
    if num_shards < 1 or V_pad % num_shards:
        raise ValueError("V_pad must be a positive multiple of num_shards")
    return V_pad // num_shards


def shard_bounds(V_pad: int, num_shards: int, shard_rows=None):
    """[(lo, hi)] physical row range of every shard: equal shards of
    V_pad / num_shards rows, or the ranges an explicit offset list gives."""
    if shard_rows is None:
        S = shard_size(V_pad, num_shards)
        return [(k * S, (k + 1) * S) for k in range(num_shards)]
    r = [int(x) for x in shard_rows]
    if len(r) != num_shards + 1 or r[0] != 0 or r[-1] != V_pad or \
            any(b < a for a, b in zip(r, r[1:])):
        raise ValueError("shard_rows must be num_shards + 1 nondecreasing offsets from 0 to V_pad")
    return list(zip(r[:-1], r[1:]))


def remap(ids, row_of, V_real: int):
    """IDs in [0, V_real) replaced by their physical row row_of[id]; any other
    value (ignore_index, out-of-range IDs) passes through unchanged."""
    ids = np.asarray(ids, dtype=np.int64)
    row_of = np.asarray(row_of, dtype=np.int64)
    ok = (ids >= 0) & (ids < V_real)
    out = ids.copy()
    out[ok] = row_of[ids[ok]]
    return out


def owner_and_local(ids, V_real: int, V_pad: int, num_shards: int, shard_rows=None):
    """Return (owner, local) int64 arrays: owner = -1 and local = 0 where no shard owns the ID.

    Each shard applies its own membership test, and the local index is formed
    only for IDs that passed it (the global ID is never used as an index).
    """
    ids = np.asarray(ids, dtype=np.int64)
    bounds = shard_bounds(V_pad, num_shards, shard_rows)
    owner = np.full(ids.shape, -1, dtype=np.int64)
    local = np.zeros(ids.shape, dtype=np.int64)
    for k, (lo, hi) in enumerate(bounds):
        hi = min(hi, V_real)
        mine = (ids >= lo) & (ids < hi)
        owner[mine] = k
        local[mine] = ids[mine] - lo
    return owner, local
