"""Cross-entropy over a vocabulary-sharded LM head, in float64.

Definitions followed:
  [VS] paragraph 3: the log-normaliser of one token uses the maximum over the
    valid vocabulary entries, every shard sums exp(logit - max) over the rows it
    owns, and the sums are combined; the target logit comes from the one shard
    that owns the target; the loss uses that one global normaliser.
  [VS] paragraph 4: subtracting the maximum does not change probabilities;
    padded rows are not classes and add nothing to the normaliser; ignored
    targets follow the loss's mask; the gradient of a valid logit is its global
    probability minus the target indicator, times the loss scaling.
  [PAD] section 5 (fix, layer 1): logits of padded rows are set to -inf before
    a cross-entropy with ignore_index = -100 and mean reduction.
  [SP] paragraph 3: the loss average is taken once, over the valid tokens.

Readings where the pages are silent: a target outside [0, V_real) that is not
ignore_index is "bad": it is treated as ignored and counted; with no valid
token the mean loss and the gradients are 0 (no division by zero).
"""

from __future__ import annotations

import numpy as np

from .geometry import owner_and_local, shard_bounds

MEAN, SUM = 0, 1


def target_status(targets, V_real: int, ignore_index: int):
    """(valid, ignored, bad) boolean masks. valid: 0 <= y < V_real.
    Pinned by test_target_status_cases."""
    y = np.asarray(targets, dtype=np.int64)
    valid = (y >= 0) & (y < V_real)
    ignored = (~valid) & (y == ignore_index)
    bad = (~valid) & (~ignored)
    return valid, ignored, bad


def logits(h, W, V_real: int) -> np.ndarray:
    """z[t, v] = sum_j h[t, j] W[v, j] for the real rows v < V_real only
    (the padded rows never enter). Pinned by the brute-force tests."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(W[:V_real], dtype=np.float64).T


def lse_rows(z) -> np.ndarray:
    """log sum_v exp(z[t, v]) with the row maximum subtracted first.
    Pinned by test_lse_closed_forms and test_bruteforce_tiny."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def shard_stats(z, V_real: int, V_pad: int, num_shards: int, shard_rows=None):
    """Per shard k: m_k = max of the logits of the real rows k owns, and
    s_k = sum of exp(z - m_k) over them; a shard owning no real row gives
    (-inf, 0). z holds the real columns [0, V_real) only.
    Pinned by test_sharded_lse_equals_unsharded."""
    T = z.shape[0]
    m = np.full((num_shards, T), -np.inf)
    s = np.zeros((num_shards, T))
    for k, (lo, hi) in enumerate(shard_bounds(V_pad, num_shards, shard_rows)):
        hi = min(hi, V_real)
        if hi <= lo:
            continue
        zk = z[:, lo:hi]
        m[k] = zk.max(axis=1)
        s[k] = np.exp(zk - m[k][:, None]).sum(axis=1)
    return m, s


def merge_shard_stats(m, s) -> np.ndarray:
    """Combine per-shard (m_k, s_k) into the global log-normaliser:
    M = max_k m_k, total = sum over shards with s_k > 0 of s_k exp(m_k - M),
    lse = M + log(total). Pinned by test_sharded_lse_equals_unsharded."""
    M = m.max(axis=0)
    total = np.zeros_like(M)
    for k in range(m.shape[0]):
        live = s[k] > 0
        total[live] += s[k][live] * np.exp(m[k][live] - M[live])
    return M + np.log(total)


def lse_two_phase(z, V_real: int, V_pad: int, num_shards: int, shard_rows=None) -> np.ndarray:
    """The schedule as [VS] paragraph 3 orders it: first the global maximum
    over valid entries (the maximum of the shards' own maxima), then each
    shard's sum of exp(z - global max) over its owned real rows, then the
    global sum. Pinned by test_sharded_lse_equals_unsharded."""
    T = z.shape[0]
    parts = [(lo, min(hi, V_real)) for lo, hi in shard_bounds(V_pad, num_shards, shard_rows)]
    local_max = np.full((num_shards, T), -np.inf)
    for k, (lo, hi) in enumerate(parts):
        if hi > lo:
            local_max[k] = z[:, lo:hi].max(axis=1)
    gmax = local_max.max(axis=0)
    total = np.zeros(T)
    for lo, hi in parts:
        if hi > lo:
            total += np.exp(z[:, lo:hi] - gmax[:, None]).sum(axis=1)
    return gmax + np.log(total)


def grad_scale(grad_loss: float, n_valid: int, reduction: int) -> float:
    """Loss scaling of the gradient: grad_loss / max(n_valid, 1) for the mean
    over valid tokens, grad_loss for the sum."""
    if reduction == MEAN:
        return float(grad_loss) / max(int(n_valid), 1)
    if reduction == SUM:
        return float(grad_loss)
    raise ValueError("reduction must be 0 (mean) or 1 (sum)")


def ce_forward(h, W, targets, V_real: int, V_pad: int, num_shards: int,
               ignore_index: int = -100, chunk: int = 256, shard_rows=None) -> dict:
    """Per-token lse, loss and target logit; loss_sum, n_valid, n_bad; and the
    per-shard (m_k, s_k). h [T, H] and W [V_pad, H] are float64; rows of W at
    or past V_real are never read. Ignored and bad tokens still get lse but
    loss 0. Pinned by test_bruteforce_tiny, test_binomial_page_numbers,
    test_lse_closed_forms and test_padded_rows_do_not_matter."""
    T = h.shape[0]
    bounds = shard_bounds(V_pad, num_shards, shard_rows)
    valid, ignored, bad = target_status(targets, V_real, ignore_index)
    y = np.asarray(targets, dtype=np.int64)
    owner, local = owner_and_local(y, V_real, V_pad, num_shards, shard_rows)
    lse = np.zeros(T)
    zt = np.zeros(T)
    sm = np.full((num_shards, T), -np.inf)
    ss = np.zeros((num_shards, T))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        z = logits(h[t0:t1], W, V_real)
        lse[t0:t1] = lse_rows(z)
        m, s = shard_stats(z, V_real, V_pad, num_shards, shard_rows)
        sm[:, t0:t1], ss[:, t0:t1] = m, s
        for i in range(t1 - t0):
            t = t0 + i
            if valid[t]:
                # the owning shard reads its own column at the local index
                zt[t] = z[i, bounds[owner[t]][0] + local[t]]
    loss = np.where(valid, lse - zt, 0.0)
    return dict(lse=lse, loss=loss, zt=zt, loss_sum=float(loss.sum()),
                n_valid=int(valid.sum()), n_bad=int(bad.sum()), valid=valid,
                shard_m=sm, shard_s=ss)


def ce_backward(h, W, targets, lse, V_real: int, V_pad: int, scale: float,
                ignore_index: int = -100, chunk: int = 256):
    """dh = G W and dW = G^T h with G[t, v] = scale * (exp(z[t, v] - lse[t]) - [v == y_t])
    for valid tokens and real rows; G is 0 for ignored/bad tokens and padded
    rows, so dW rows at or past V_real are exactly 0. Pinned by
    test_gradient_finite_difference and test_gradient_rows_sum_to_zero."""
    T, H = h.shape
    valid, _, _ = target_status(targets, V_real, ignore_index)
    y = np.asarray(targets, dtype=np.int64)
    dh = np.zeros((T, H))
    dW = np.zeros((V_pad, H))
    Wr = np.asarray(W[:V_real], dtype=np.float64)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        z = logits(h[t0:t1], W, V_real)
        G = np.exp(z - lse[t0:t1, None])
        rows = np.nonzero(valid[t0:t1])[0]
        G[rows, y[t0:t1][rows]] -= 1.0
        G[~valid[t0:t1]] = 0.0
        G *= scale
        dh[t0:t1] = G @ Wr
        dW[:V_real] += G.T @ h[t0:t1]
    return dh, dW


def cross_entropy(h, W, targets, V_real: int, V_pad: int, num_shards: int,
                  ignore_index: int = -100, grad_loss: float = 1.0,
                  reduction: int = MEAN, chunk: int = 256, shard_rows=None) -> dict:
    """Forward, then backward with the loss scaling of ``reduction``.
    Adds loss (the reduced value), scale, dh and dW to the forward's dict."""
    f = ce_forward(h, W, targets, V_real, V_pad, num_shards, ignore_index, chunk, shard_rows)
    scale = grad_scale(grad_loss, f["n_valid"], reduction)
    dh, dW = ce_backward(h, W, targets, f["lse"], V_real, V_pad, scale, ignore_index, chunk)
    if reduction == MEAN:
        f["loss_reduced"] = f["loss_sum"] / f["n_valid"] if f["n_valid"] else 0.0
    else:
        f["loss_reduced"] = f["loss_sum"]
    f.update(scale=scale, dh=dh, dW=dW)
    return f
