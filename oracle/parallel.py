"""The oracle's cross-entropy and tied step at full workload sizes, spread
over the host's cores.

TEST INFRASTRUCTURE ONLY (like the rest of this package). Same definitions as
oracle.ce / oracle.tied ([VS] paragraphs 3-4: one global log-normaliser per
token over the real rows, loss = lse - target logit for valid targets, the
gradient of a logit = scale * (probability - target indicator), zero for
ignored or bad tokens and padded rows; [VS] paragraph 2 for the tied table),
evaluated in float64 with numpy, only scheduled for many cores:

  1. token chunks (in parallel): logits of the chunk's tokens over the real
     rows, lse, the target logit, loss, and dh = G W for those tokens. The
     scale grad_loss / n_valid depends only on the targets, so G is known as
     soon as the chunk's lse is;
  2. vocabulary chunks (in parallel): the logits of every token over the
     chunk's rows again, G for those rows, and dW rows = G^T h.

Every row of dh and of dW is one product of whole float64 operands, so the
results equal oracle.cross_entropy up to float64 rounding order (pinned by
tests/test_oracle_pins.py::test_parallel_schedule_matches_sequential).
Threads are used, not processes: numpy releases the interpreter lock inside
its matrix products and elementwise loops, and the operands are shared
without copies. BLAS runs one thread per worker while this runs.
"""

from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .ce import MEAN, grad_scale, logits, lse_rows, target_status
from .embedding import gather_direct, scatter_add
from .geometry import owner_and_local, shard_bounds


def default_workers(cap: int = 16) -> int:
    """Cores this process may run on, at most `cap`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ('unknown' if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1, user_api="blas")
    except Exception:  # pragma: no cover
        class _Null:
            def __enter__(self):
                return self

            def __exit__(self, *a):
                return False
        return _Null()


def cross_entropy(h, W, targets, V_real: int, V_pad: int, num_shards: int,
                  ignore_index: int = -100, grad_loss: float = 1.0, reduction: int = MEAN,
                  workers: int | None = None, tok_chunk: int = 256,
                  voc_chunk: int = 2048, progress=None) -> dict:
    """lse, loss, zt [T]; loss_sum, n_valid, n_bad, valid; dh [T, H] and
    dW [V_pad, H] (rows at or past V_real exactly 0), all float64.
    h [T, H] and W [V_pad, H] float64; rows of W past V_real are never read."""
    h = np.ascontiguousarray(h, dtype=np.float64)
    T, H = h.shape
    Wr = np.ascontiguousarray(W[:V_real], dtype=np.float64)
    y = np.asarray(targets, dtype=np.int64)
    valid, _, bad = target_status(y, V_real, ignore_index)
    n_valid = int(valid.sum())
    scale = grad_scale(grad_loss, n_valid, reduction)
    bounds = shard_bounds(V_pad, num_shards)
    owner, local = owner_and_local(y, V_real, V_pad, num_shards)
    workers = default_workers() if workers is None else workers

    lse = np.zeros(T)
    zt = np.zeros(T)
    dh = np.zeros((T, H))
    dW = np.zeros((V_pad, H))
    done = [0]
    lock = threading.Lock()

    def tick(what, total, offset):
        if progress is None:
            return
        with lock:
            done[0] += 1
            k = done[0] - offset
            if k % max(1, total // 8) == 0 or k == total:
                progress(f"oracle {what}: {k}/{total}")

    def tok_task(t0):
        t1 = min(T, t0 + tok_chunk)
        z = logits(h[t0:t1], Wr, V_real)
        l = lse_rows(z)
        lse[t0:t1] = l
        v = valid[t0:t1]
        rows = np.nonzero(v)[0]
        for i in rows:
            t = t0 + i
            # the owning shard's column at its local index
            zt[t] = z[i, bounds[owner[t]][0] + local[t]]
        G = np.exp(z - l[:, None])
        G[rows, y[t0:t1][rows]] -= 1.0
        G[~v] = 0.0
        G *= scale
        dh[t0:t1] = G @ Wr
        tick("token chunks", n_tok, 0)

    def voc_task(v0):
        v1 = min(V_real, v0 + voc_chunk)
        z = h @ Wr[v0:v1].T
        G = np.exp(z - lse[:, None])
        hit = np.nonzero(valid & (y >= v0) & (y < v1))[0]
        G[hit, y[hit] - v0] -= 1.0
        G[~valid] = 0.0
        G *= scale
        dW[v0:v1] = G.T @ h
        tick("vocabulary chunks", n_voc, n_tok)

    n_tok = (T + tok_chunk - 1) // tok_chunk
    n_voc = (V_real + voc_chunk - 1) // voc_chunk
    with _blas_one_thread(), ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(tok_task, range(0, T, tok_chunk)))
        list(ex.map(voc_task, range(0, V_real, voc_chunk)))
    loss = np.where(valid, lse - zt, 0.0)
    return dict(lse=lse, loss=loss, zt=zt, loss_sum=float(loss.sum()), n_valid=n_valid,
                n_bad=int(bad.sum()), valid=valid, scale=scale, dh=dh, dW=dW)


def tied_step(ids, targets, W, V_real: int, V_pad: int, num_shards: int,
              ignore_index: int = -100, grad_loss: float = 1.0, reduction: int = MEAN,
              workers: int | None = None, progress=None) -> dict:
    """oracle.tied_step's quantities (without dW_ce): h = lookup of ids; the
    cross-entropy of h W^T; dW = its output-row gradient + dW_emb, the
    scatter-add of dh by ID."""
    W = np.asarray(W, dtype=np.float64)
    h = gather_direct(ids, W, V_real)
    f = cross_entropy(h, W, targets, V_real, V_pad, num_shards, ignore_index, grad_loss,
                      reduction, workers=workers, progress=progress)
    dW_emb, count = scatter_add(ids, f["dh"], V_real, V_pad)
    f["dW"] += dW_emb  # the output-row gradient is not kept on its own (memory)
    f.update(h=h, dW_emb=dW_emb, count=count)
    return f
