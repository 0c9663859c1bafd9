"""Masked embedding lookup and its scatter-add backward, in float64.

[VS] paragraph 1: non-owning shards contribute a zero vector, and adding the
masked contributions of all shards rebuilds the embedding because a valid ID
has exactly one owner. [VS] paragraph 2: the table is never indexed with an
unmasked global ID; repeated occurrences of a token add their gradients into
the one owned row; out-of-range and padded IDs need an explicit rule. Rule
adopted: an ID outside [0, V_real) yields a zero row and no gradient.
"""

import numpy as np

from .geometry import owner_and_local, shard_bounds


def gather_direct(ids, W, V_real: int) -> np.ndarray:
    """out[t] = W[ids[t]] if 0 <= ids[t] < V_real, else a zero row.

    Pinned by test_gather_masked_sum_equals_direct and test_gather_edge_ids.
    """
    ids = np.asarray(ids, dtype=np.int64)
    ok = (ids >= 0) & (ids < V_real)
    out = np.zeros((ids.shape[0], W.shape[1]), dtype=W.dtype)
    out[ok] = W[ids[ok]]
    return out


def gather_masked_shards(ids, W, V_real: int, V_pad: int, num_shards: int,
                         shard_rows=None) -> np.ndarray:
    """The sharded form: every shard looks up only IDs it owns, at their local
    index in its own slice of the table, contributes zeros elsewhere, and the
    contributions are summed over shards. Pinned against gather_direct."""
    ids = np.asarray(ids, dtype=np.int64)
    owner, local = owner_and_local(ids, V_real, V_pad, num_shards, shard_rows)
    out = np.zeros((ids.shape[0], W.shape[1]), dtype=np.float64)
    for k, (lo, hi) in enumerate(shard_bounds(V_pad, num_shards, shard_rows)):
        Wk = W[lo:hi]
        mine = owner == k
        contrib = np.zeros_like(out)
        contrib[mine] = Wk[local[mine]]
        out += contrib
    return out


def scatter_add(ids, dout, V_real: int, V_pad: int):
    """dW[v] = sum of dout[t] over the t with ids[t] == v (float64), for real
    rows v; rows no valid ID touches stay zero. Also returns the per-row count.

    Pinned by test_scatter_add_bruteforce (pure-Python loop) and the tied-step
    finite difference.
    """
    ids = np.asarray(ids, dtype=np.int64)
    dout = np.asarray(dout, dtype=np.float64)
    ok = (ids >= 0) & (ids < V_real)
    dW = np.zeros((V_pad, dout.shape[1]), dtype=np.float64)
    np.add.at(dW, ids[ok], dout[ok])
    count = np.bincount(ids[ok], minlength=V_pad).astype(np.int64)
    return dW, count
