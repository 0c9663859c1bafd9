"""One tied embedding + LM-head step over a single table W.

[VS] paragraph 2: when the input embedding and the output projection share one
parameter, the tie is kept and every gradient contribution lands in that one
tensor. Reading adopted for the step (the pages fix no model between the two):
the hidden input of the loss is the embedding of the input IDs itself, so
  loss(W) = CE(gather(ids, W) W^T, targets)
and dloss/dW = (CE gradient w.r.t. the output rows) + scatter-add of dh into
the rows the IDs picked. Pinned by test_tied_step_finite_difference.
"""

from .ce import MEAN, ce_backward, ce_forward, grad_scale
from .embedding import gather_direct, scatter_add


def tied_step(ids, targets, W, V_real: int, V_pad: int, num_shards: int,
              ignore_index: int = -100, grad_loss: float = 1.0,
              reduction: int = MEAN, chunk: int = 256) -> dict:
    h = gather_direct(ids, W, V_real)
    f = ce_forward(h, W, targets, V_real, V_pad, num_shards, ignore_index, chunk)
    scale = grad_scale(grad_loss, f["n_valid"], reduction)
    dh, dW_ce = ce_backward(h, W, targets, f["lse"], V_real, V_pad, scale, ignore_index, chunk)
    dW_emb, count = scatter_add(ids, dh, V_real, V_pad)
    f.update(h=h, scale=scale, dh=dh, dW_ce=dW_ce, dW_emb=dW_emb, count=count,
             dW=dW_ce + dW_emb)
    return f
