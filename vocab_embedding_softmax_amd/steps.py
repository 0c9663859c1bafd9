"""Whole steps of the path as sequences of library calls (no arithmetic here).

ce_step       cross-entropy forward + backward on (h, W, targets)
tied_step     lookup -> cross-entropy forward/backward -> scatter-add of dh
              into the same dW ("Vocabulary shards: look up locally and
              normalize globally", ¶2: one tied table, all contributions)
sampled_step  candidates -> lookup of the candidate rows -> cross-entropy over
              them -> scatter of their gradients into the full table
              ("Sampled Softmax with Over-Tokenized Transformer", Setup)
ngram_bwd     backward of vngram_fwd: the scatter-add of dx into the unigram
              table and, by the rows vngram_fwd reported, into the two n-gram
              tables (same page, OT input side)
ot_h_step     tied_step plus a second, untied head on the hidden rows but the
              last, scored two tokens ahead and weighted 0.1 (same page, OT-H);
              its dh is added into the first head's before the scatter
"""

from __future__ import annotations

from collections import namedtuple
from typing import Optional

import numpy as np
import torch

from . import _lib as L

StepOut = namedtuple("StepOut", "fwd dh dW extra")


def from_bits(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host array -> GPU tensor holding the same bits (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    raise ValueError(dtype)


class Workspaces:
    """Device workspaces sized once for a step shape and reused by every call."""

    def __init__(self, device, **sizes):
        self.buf = {k: torch.empty(max(int(v), 16), dtype=torch.uint8, device=device)
                    for k, v in sizes.items()}

    def __getitem__(self, k):
        return self.buf[k]


def ce_step(h, W, targets, V_real, num_shards, ignore_index=-100, *, grad_loss=None,
            reduction=L.REDUCE_MEAN, ws: Optional[Workspaces] = None, dh=None, dW=None,
            shard_stats=False, allow_bad=False, stream=None) -> StepOut:
    dev = h.device
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
    f = L.vce_fwd(h, W, targets, V_real, num_shards, ignore_index, shard_stats=shard_stats,
                  ws=None if ws is None else ws["fwd"], allow_bad=allow_bad, stream=stream)
    b = L.vce_bwd(h, W, targets, f.lse, grad_loss, f.n_valid, V_real, num_shards, ignore_index,
                  reduction, dh=dh, dW=dW, ws=None if ws is None else ws["bwd"], stream=stream)
    return StepOut(f, b.dh, b.dW, None)


def tied_step(ids, targets, W, V_real, num_shards, ignore_index=-100, *, grad_loss=None,
              reduction=L.REDUCE_MEAN, ws: Optional[Workspaces] = None, h=None, dh=None,
              dW=None, allow_bad=False, stream=None) -> StepOut:
    dev = W.device
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
    h, n_bad_id = L.vemb_fwd(ids, W, V_real, num_shards, out=h, stream=stream)
    f = L.vce_fwd(h, W, targets, V_real, num_shards, ignore_index,
                  ws=None if ws is None else ws["fwd"], allow_bad=allow_bad, stream=stream)
    b = L.vce_bwd(h, W, targets, f.lse, grad_loss, f.n_valid, V_real, num_shards, ignore_index,
                  reduction, dh=dh, dW=dW, accumulate_dW=False,
                  ws=None if ws is None else ws["bwd"], stream=stream)
    L.vemb_bwd(ids, b.dh, V_real, W.shape[0], num_shards, dW=b.dW, accumulate=True,
               ws=None if ws is None else ws["emb"], stream=stream)
    return StepOut(f, b.dh, b.dW, dict(h=h, n_bad_id=n_bad_id))


def sampled_step(h, W, targets, perm, P, ignore_index=-100, *, grad_loss=None,
                 reduction=L.REDUCE_MEAN, ws: Optional[Workspaces] = None, dW=None,
                 prev_rows=None, n_cand: Optional[int] = None, allow_bad=False,
                 stream=None) -> StepOut:
    """The composite is sized by the number of candidates, n_cand = max(P, |U|)
    (U = the batch's distinct valid targets): with more distinct targets than
    P the candidates are U alone and every one of them takes part.

    n_cand=None (default) reads that count from the device after the
    candidate kernel (a stream synchronisation). A caller that must not
    synchronise (graph capture) passes n_cand itself; it must equal the
    device's count (P whenever |U| <= P). A smaller value would leave the
    targets ranked past it out of the candidates: they are then counted as
    bad targets (fwd.n_bad), which raises unless allow_bad=True. The
    workspaces in `ws` are sized for P candidates and are replaced by larger
    ones when n_cand exceeds P.

    dW [V, H] receives the table gradient: zero except the candidate rows.
    With prev_rows (int32, possibly empty) the caller keeps dW from step to
    step: it must be zero except at prev_rows, the previous step's
    extra["rows"] (empty for a zeroed table), and only those rows are cleared
    (vss_scatter_replace) instead of the whole table."""
    dev = h.device
    V, H = W.shape
    if grad_loss is None:
        grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
    c = L.vss_candidates(targets, V, perm, P, ignore_index,
                         ws=None if ws is None else ws["cand"], stream=stream)
    Pe = L.read_scalar(c.n_cand, stream) if n_cand is None else int(n_cand)
    if Pe < 1 or Pe > c.cand.shape[0]:
        raise ValueError(f"n_cand = {Pe} outside [1, {c.cand.shape[0]}]")
    fit = ws is not None and Pe <= P
    cand = c.cand[:Pe]
    Wc, _ = L.vemb_fwd(cand, W, V, 1, count_bad=False, stream=stream)
    f = L.vce_fwd(h, Wc, c.pos, Pe, 1, ignore_index, ws=ws["fwd"] if fit else None,
                  allow_bad=allow_bad, stream=stream)
    b = L.vce_bwd(h, Wc, c.pos, f.lse, grad_loss, f.n_valid, Pe, 1, ignore_index, reduction,
                  ws=ws["bwd"] if fit else None, stream=stream)
    if prev_rows is None:
        dW = L.vss_scatter(cand, b.dW, V, dW=dW, accumulate=False, stream=stream)
    else:
        if dW is None:
            raise ValueError("prev_rows needs the caller's dW table")
        dW = L.vss_scatter_replace(prev_rows, cand, b.dW, dW, stream=stream)
    return StepOut(f, b.dh, dW, dict(cand=c.cand, pos=c.pos, n_unique=c.n_unique,
                                     n_cand=c.n_cand, Wc=Wc, dWc=b.dW, rows=cand))


def ot_h_step(ids, targets1, targets2, W, W2, V_real, num_shards, ignore_index=-100, *,
              weight=0.1, ws: Optional[Workspaces] = None, ws2: Optional[Workspaces] = None,
              h=None, dh=None, dW=None, dW2=None, allow_bad=False, stream=None) -> StepOut:
    """ids, targets1 [T]; targets2 [T - 1] (the tokens two positions ahead of
    rows 0..T-2); W the tied table, W2 the second head's table (same shape).
    ws2 sizes the second head's calls (T - 1 rows)."""
    dev = W.device
    T = ids.shape[0]
    one = torch.ones(1, dtype=torch.float32, device=dev)
    wgt = torch.full((1,), float(weight), dtype=torch.float32, device=dev)
    h, n_bad_id = L.vemb_fwd(ids, W, V_real, num_shards, out=h, stream=stream)
    f1 = L.vce_fwd(h, W, targets1, V_real, num_shards, ignore_index,
                   ws=None if ws is None else ws["fwd"], allow_bad=allow_bad, stream=stream)
    h2 = h[:T - 1]
    f2 = L.vce_fwd(h2, W2, targets2, V_real, num_shards, ignore_index,
                   ws=None if ws2 is None else ws2["fwd"], allow_bad=allow_bad, stream=stream)
    b1 = L.vce_bwd(h, W, targets1, f1.lse, one, f1.n_valid, V_real, num_shards, ignore_index,
                   L.REDUCE_MEAN, dh=dh, dW=dW, ws=None if ws is None else ws["bwd"],
                   stream=stream)
    b2 = L.vce_bwd(h2, W2, targets2, f2.lse, wgt, f2.n_valid, V_real, num_shards, ignore_index,
                   L.REDUCE_MEAN, dh=b1.dh[:T - 1], dW=dW2, accumulate_dh=True,
                   ws=None if ws2 is None else ws2["bwd"], stream=stream)
    L.vemb_bwd(ids, b1.dh, V_real, W.shape[0], num_shards, dW=b1.dW, accumulate=True,
               ws=None if ws is None else ws["emb"], stream=stream)
    return StepOut(f1, b1.dh, b1.dW, dict(h=h, n_bad_id=n_bad_id, fwd2=f2, dW2=b2.dW))


_SIDE = {}


def _side_streams(device, n):
    """n extra streams of this device (default priority), made once."""
    key = (torch.device(device).index, n)
    if key not in _SIDE:
        _SIDE[key] = [torch.cuda.Stream(device=device) for _ in range(n)]
    return _SIDE[key]


def ngram_bwd(ids, fwd_out, dx, V_real, V_pad, num_shards, *, dE=None, dE2=None, dE3=None,
              rows2=None, rows3=None, accumulate=False, ws: Optional[Workspaces] = None,
              stream=None):
    """dE [V_pad,H], dE2 [rows2,H], dE3 [rows3,H] (float32) from dx [T,H]; the
    n-gram rows are the ones vngram_fwd returned (fwd_out.ids2 / ids3).

    The three scatters are independent: the n-gram tables' run on two side
    streams that fork from and join back into the caller's stream, so one
    table's single-workgroup sort overlaps another's row sums. Every buffer is
    allocated on the caller's stream before the fork and the join is enqueued
    before return, so later work on that stream is ordered after all three."""
    dev = dx.device
    T, H = dx.shape
    main = torch.cuda.current_stream(dev) if stream is None else stream
    rows2 = dE2.shape[0] if rows2 is None else rows2
    rows3 = dE3.shape[0] if rows3 is None else rows3
    f32 = dict(dtype=torch.float32, device=dev)
    if dE is None:
        dE = torch.empty(V_pad, H, **f32)
    if dE2 is None:
        dE2 = torch.empty(rows2, H, **f32)
    if dE3 is None:
        dE3 = torch.empty(rows3, H, **f32)
    if ws is None:
        ws = Workspaces(dev, emb=L.vemb_bwd_workspace_bytes(T, H, V_real, V_pad),
                        emb2=L.vemb_bwd_workspace_bytes(T, H, rows2, rows2),
                        emb3=L.vemb_bwd_workspace_bytes(T, H, rows3, rows3))
    s2, s3 = _side_streams(dev, 2)
    fork = torch.cuda.Event()
    fork.record(main)
    s2.wait_event(fork)
    s3.wait_event(fork)
    L.vemb_bwd(fwd_out.ids2, dx, rows2, rows2, num_shards, dW=dE2, accumulate=accumulate,
               ws=ws["emb2"], stream=s2)
    L.vemb_bwd(fwd_out.ids3, dx, rows3, rows3, num_shards, dW=dE3, accumulate=accumulate,
               ws=ws["emb3"], stream=s3)
    L.vemb_bwd(ids, dx, V_real, V_pad, num_shards, dW=dE, accumulate=accumulate, ws=ws["emb"],
               stream=main)
    for s in (s2, s3):
        j = torch.cuda.Event()
        j.record(s)
        main.wait_event(j)
    return dE, dE2, dE3
