"""Sampled-softmax cross-entropy over a candidate subset of the table.

[SS] Setup (the simplified loss listing): the candidates are the unique
targets of the batch followed by random negatives, P rows in all; logits are
h times the candidate rows' transpose; the cross-entropy target of each token
is its target's position among the candidates. No sampling correction is
applied, as in that listing.

Readings where the listing is loose: '+' joins the two lists (it cannot be an
element-wise sum); the unique targets are sorted ascending and exclude
ignored/out-of-range targets; the negatives are the first P - |U| entries of a
uniformly random permutation of [0, V) that are not in U, so they are drawn
uniformly without replacement from the rest of the vocabulary and every
candidate is distinct; if |U| > P the candidates are U alone. A target that is
not valid keeps its value as its position (so it stays ignored or bad).
Pinned by test_sampled_full_candidate_set_equals_full_ce and
test_candidates_bruteforce.
"""

import numpy as np

from .ce import MEAN, ce_backward, ce_forward, grad_scale


def candidates(targets, V: int, ignore_index: int, perm, P: int):
    """Return (cand int64 [max(P, |U|)], pos int64 [T], n_unique)."""
    y = np.asarray(targets, dtype=np.int64)
    valid = (y >= 0) & (y < V)
    U = np.unique(y[valid])
    in_u = np.zeros(V, dtype=bool)
    in_u[U] = True
    perm = np.asarray(perm, dtype=np.int64)
    need = max(P - U.shape[0], 0)
    neg = perm[~in_u[perm]][:need]
    cand = np.concatenate([U, neg])
    pos = y.copy()
    pos[valid] = np.searchsorted(U, y[valid])
    return cand, pos, int(U.shape[0])


def sampled_step(h, W, targets, perm, P: int, ignore_index: int = -100,
                 grad_loss: float = 1.0, reduction: int = MEAN, chunk: int = 256) -> dict:
    """Candidates, the candidate rows' gather, cross-entropy forward and
    backward over them (every candidate row is a real class, one shard), and
    the candidate-row gradients added back into a full-table dW."""
    V = W.shape[0]
    cand, pos, n_u = candidates(targets, V, ignore_index, perm, P)
    Pe = cand.shape[0]
    Wc = np.asarray(W, dtype=np.float64)[cand]
    f = ce_forward(h, Wc, pos, Pe, Pe, 1, ignore_index, chunk)
    scale = grad_scale(grad_loss, f["n_valid"], reduction)
    dh, dWc = ce_backward(h, Wc, pos, f["lse"], Pe, Pe, scale, ignore_index, chunk)
    dW = np.zeros((V, W.shape[1]))
    np.add.at(dW, cand, dWc)
    f.update(cand=cand, pos=pos, n_unique=n_u, scale=scale, dh=dh, dWc=dWc, dW=dW)
    return f
