"""Greedy decoding over a vocabulary-sharded LM head: the global argmax of the
logits, found without gathering them, in float64.

Definition followed: [TP] "LM Head (ColumnParallelLinear)": every rank
computes the logits of its own vocabulary shard ([T, V/n]); with on-device
sampling the sampler finds the global argmax across the shards without
rebuilding the full [T, V] logits. [VS] paragraph 4: padded rows are not
classes, so they are never chosen.

Readings where the page is silent: greedy sampling is the argmax over the
real rows (no temperature or top-k is on the page); on equal maxima the
lowest vocabulary index wins, inside a shard and across shards (what an
unsharded argmax that returns the first maximum gives); every shard reports
(largest logit over the real rows it owns, lowest index holding it), a shard
that owns no real row reports (-inf, -1), and the shard reports are merged by
larger value, then lower index.

Pinned by tests/test_oracle_pins.py::test_argmax_* (pure-Python brute force
on tiny vocabularies with NaN padding, constructed ties, one-hot hidden rows,
sharded == unsharded).
"""

from __future__ import annotations

import numpy as np

from .ce import logits
from .geometry import shard_bounds


def shard_argmax(z, V_real: int, V_pad: int, num_shards: int, shard_rows=None):
    """Per shard k over the real columns it owns: (value, index) of the largest
    logit, the lowest index on ties; (-inf, -1) for a shard without real rows.
    z holds the real columns [0, V_real) only."""
    T = z.shape[0]
    val = np.full((num_shards, T), -np.inf)
    idx = np.full((num_shards, T), -1, dtype=np.int64)
    for k, (lo, hi) in enumerate(shard_bounds(V_pad, num_shards, shard_rows)):
        hi = min(hi, V_real)
        if hi <= lo:
            continue
        zk = z[:, lo:hi]
        j = np.argmax(zk, axis=1)          # first maximum: the lowest index
        val[k] = zk[np.arange(T), j]
        idx[k] = lo + j
    return val, idx


def merge_shard_argmax(val, idx):
    """Merge shard reports in shard order: a later shard replaces the best so
    far only with a strictly larger value, or an equal value at a lower index."""
    best_v = val[0].copy()
    best_i = idx[0].copy()
    for k in range(1, val.shape[0]):
        take = (val[k] > best_v) | ((val[k] == best_v) & (idx[k] >= 0) &
                                    ((best_i < 0) | (idx[k] < best_i)))
        best_v = np.where(take, val[k], best_v)
        best_i = np.where(take, idx[k], best_i)
    return best_v, best_i


def greedy_argmax(h, W, V_real: int, V_pad: int, num_shards: int, chunk: int = 256,
                  shard_rows=None) -> dict:
    """index [T] and value [T] of the global argmax over the real rows, plus the
    per-shard reports (shard_value, shard_index [num_shards, T]). h [T, H] and
    W [V_pad, H] are float64; rows of W at or past V_real are never read."""
    T = h.shape[0]
    sv = np.full((num_shards, T), -np.inf)
    si = np.full((num_shards, T), -1, dtype=np.int64)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        z = logits(h[t0:t1], W, V_real)
        sv[:, t0:t1], si[:, t0:t1] = shard_argmax(z, V_real, V_pad, num_shards, shard_rows)
    value, index = merge_shard_argmax(sv, si)
    return dict(index=index, value=value, shard_value=sv, shard_index=si)
