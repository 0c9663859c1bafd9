"""The OT-H step: the tied embedding + LM-head step plus a second, untied head
that predicts the token two positions ahead, added to the loss at weight 0.1.

Definition followed: [SS] "Setup" and its loss listing: OT-H adds a second
head on the hidden rows but the last, scored against the tokens two positions
ahead, and adds 0.1 times its cross-entropy to the loss. With a token stream
tokens[0..T+1]: the input IDs are tokens[0..T-1]; the first head scores rows
0..T-1 against tokens[1..T]; the second head scores rows 0..T-2 against
tokens[2..T].

Readings where the page is silent: both cross-entropies are means over their
own valid targets (ignore_index and out-of-range targets as for the main
loss); the second head has its own table W2 [V_pad, H] of the same geometry
(vocabulary shards included); the hidden rows are the lookup of the input IDs
in the tied table, as in tied_step, so
  loss(W, W2) = CE(h W^T, y1) + 0.1 CE(h[:-1] W2^T, y2),  h = gather(ids, W)
and dloss/dh = dh1 + 0.1 dh2 (dh2 padded with a zero last row), dloss/dW =
(first head's gradient) + scatter-add of dloss/dh into the rows the IDs
picked, dloss/dW2 = the second head's gradient. Pinned by
test_ot_h_step_finite_difference.
"""

import numpy as np

from .ce import MEAN, ce_backward, ce_forward, grad_scale
from .embedding import gather_direct, scatter_add

OT_H_WEIGHT = 0.1


def ot_h_step(ids, targets1, targets2, W, W2, V_real: int, V_pad: int, num_shards: int,
              ignore_index: int = -100, weight: float = OT_H_WEIGHT, chunk: int = 256) -> dict:
    """ids [T], targets1 [T], targets2 [T - 1]; W, W2 [V_pad, H] float64."""
    T = len(ids)
    h = gather_direct(ids, W, V_real)
    f1 = ce_forward(h, W, targets1, V_real, V_pad, num_shards, ignore_index, chunk)
    f2 = ce_forward(h[:T - 1], W2, targets2, V_real, V_pad, num_shards, ignore_index, chunk)
    s1 = grad_scale(1.0, f1["n_valid"], MEAN)
    s2 = grad_scale(weight, f2["n_valid"], MEAN)
    dh1, dW1 = ce_backward(h, W, targets1, f1["lse"], V_real, V_pad, s1, ignore_index, chunk)
    dh2, dW2 = ce_backward(h[:T - 1], W2, targets2, f2["lse"], V_real, V_pad, s2,
                           ignore_index, chunk)
    dh = dh1.copy()
    dh[:T - 1] += dh2
    dW_emb, count = scatter_add(ids, dh, V_real, V_pad)
    loss1 = f1["loss_sum"] / f1["n_valid"] if f1["n_valid"] else 0.0
    loss2 = f2["loss_sum"] / f2["n_valid"] if f2["n_valid"] else 0.0
    return dict(h=h, f1=f1, f2=f2, loss=loss1 + weight * loss2, loss1=loss1, loss2=loss2,
                dh=dh, dW=dW1 + dW_emb, dW2=dW2, count=count)
