"""Comparison helpers and GPU-run wrappers shared by the GPU parity tests.

Tolerances:
  bf16 inputs, fp32 accumulation: |d loss_sum| / |loss_sum| <= 2e-3,
    max_t |d lse_t| <= 1e-2, rel-L2 <= 1e-2 on dh and dW (and on every
    embedding-gradient tensor), and on every 256-row block of dW on its own
    (tile_rel_l2);
  fp32 inputs: 1e-5 relative on loss, lse (per element) and the gradients (rel-L2).
  Integer and byte results (gathers, counts, candidate lists): bit-exact.

Argmax (floating point decides the index): the kernel's logits carry float32
accumulation error, bounded for a row v by
    e(t, v) = gamma * sum_j |h[t, j] W[v, j]|,  gamma = (K + 2) u / (1 - (K + 2) u),
u = 2^-24 (products of bf16 inputs are exact in float32; float32 inputs add
one rounding per product). When the oracle's best row beats every other row
by more than the two rows' bounds, the kernel must return exactly that index;
otherwise (a near tie) the kernel's row must be within those bounds of the
maximum. The returned value must lie within the chosen row's bound of that
row's exact logit.
"""

import numpy as np

import oracle
from oracle.ce import MEAN

TOL = {
    "bf16": dict(loss=2e-3, lse_abs=1e-2, lse_rel=None, grad=1e-2),
    "f32": dict(loss=1e-5, lse_abs=None, lse_rel=1e-5, grad=1e-5),
}


def rel_l2(a, b, block=1 << 16):
    """||a - b|| / ||b|| (||a|| when b is 0), in float64, a row block at a time
    so that full-size tables need no float64 copy of the whole tensor."""
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        raise ValueError(f"shapes differ: {a.shape} vs {b.shape}")
    if a.ndim < 2:
        a = a.reshape(-1, 1)
        b = b.reshape(-1, 1)
    dd = bb = aa = 0.0
    for r0 in range(0, a.shape[0], block):
        x = a[r0:r0 + block].astype(np.float64)
        y = b[r0:r0 + block].astype(np.float64)
        dd += float(np.square(x - y).sum())
        bb += float(np.square(y).sum())
        aa += float(np.square(x).sum())
    if bb == 0:
        return float(np.sqrt(aa))
    return float(np.sqrt(dd / bb))


def tile_rel_l2(got, ref, rows=256, floor_frac=1e-6):
    """Relative L2 error of each block of `rows` consecutive rows (one GEMM
    tile of dW): ||got_j - ref_j|| / max(||ref_j||, floor), with the floor
    floor_frac * ||ref|| / sqrt(number of blocks) so that a block whose
    reference is (nearly) zero is held to an absolute bound. Returns the
    per-block errors. A whole-tensor rel-L2 is dominated by the few rows of
    frequent targets; this is not."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    n = (ref.shape[0] + rows - 1) // rows
    dn = np.zeros(n)
    rn = np.zeros(n)
    for j in range(n):
        x = got[j * rows:(j + 1) * rows].astype(np.float64)
        y = ref[j * rows:(j + 1) * rows].astype(np.float64)
        dn[j] = np.sqrt(np.square(x - y).sum())
        rn[j] = np.sqrt(np.square(y).sum())
    floor = floor_frac * np.sqrt(np.square(rn).sum()) / np.sqrt(max(n, 1))
    return dn / np.maximum(rn, max(floor, 1e-300))


def check_dw_tiles(got, ref, dtype, what="dW", rows=256):
    e = tile_rel_l2(got, ref, rows)
    j = int(np.argmax(e)) if e.size else 0
    assert e.size == 0 or e[j] <= TOL[dtype]["grad"], \
        f"{what}: rows [{j * rows}, {(j + 1) * rows}) rel-L2 {e[j]}"
    return float(e.max()) if e.size else 0.0


def check_ce(gpu: dict, ref: dict, dtype: str, V_real: int, check_grads: bool = True):
    tol = TOL[dtype]
    assert gpu["n_valid"] == ref["n_valid"], (gpu["n_valid"], ref["n_valid"])
    assert gpu["n_bad"] == ref["n_bad"], (gpu["n_bad"], ref["n_bad"])
    if ref["loss_sum"] != 0.0:
        dl = abs(gpu["loss_sum"] - ref["loss_sum"]) / abs(ref["loss_sum"])
        assert dl <= tol["loss"], f"loss rel err {dl}"
    else:  # e.g. a single real class: every loss is exactly 0
        assert abs(gpu["loss_sum"]) <= 1e-6
    lse_err = np.abs(gpu["lse"].astype(np.float64) - ref["lse"])
    if tol["lse_abs"] is not None:
        assert lse_err.max() <= tol["lse_abs"], f"lse abs err {lse_err.max()}"
    else:
        rel = (lse_err / np.maximum(np.abs(ref["lse"]), 1e-30)).max()
        assert rel <= tol["lse_rel"], f"lse rel err {rel}"
    valid = ref["valid"]
    assert not gpu["loss"][~valid].any()
    if check_grads:
        e_dh = rel_l2(gpu["dh"], ref["dh"])
        e_dw = rel_l2(gpu["dW"], ref["dW"])
        assert e_dh <= tol["grad"], f"dh rel-L2 {e_dh}"
        assert e_dw <= tol["grad"], f"dW rel-L2 {e_dw}"
        check_dw_tiles(gpu["dW"][:V_real], ref["dW"][:V_real], dtype)
        assert not gpu["dW"][V_real:].any(), "padded dW rows must be exactly 0"
        assert not gpu["dh"][~valid].any(), "ignored tokens must get dh = 0"


def oracle_ce(inp, grad_loss=1.0, reduction=MEAN, num_shards=None):
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    n = inp.num_shards if num_shards is None else num_shards
    return oracle.cross_entropy(h, W, inp.targets, inp.V_real, inp.V_pad, n,
                                inp.ignore_index, grad_loss, reduction)


U = 2.0 ** -24


def _bound(h64, W64, K):
    g = (K + 2) * U / (1 - (K + 2) * U)
    return g * (np.abs(h64) @ np.abs(W64).T)          # [T, V_real]


def check_argmax(idx, val, h64, W64, V_real, what):
    """idx, val: kernel results for the rows of h64; W64 holds the real rows."""
    z = h64 @ W64[:V_real].T
    e = _bound(h64, W64[:V_real], h64.shape[1])
    T = z.shape[0]
    o = np.argmax(z, axis=1)
    zmax = z[np.arange(T), o]
    # a row can overtake the oracle's best only if its upper bound reaches the
    # best row's lower bound
    reach = (z + e) >= (zmax - e[np.arange(T), o])[:, None]
    reach[np.arange(T), o] = False
    clear = ~reach.any(axis=1)
    assert (idx >= 0).all() and (idx < V_real).all(), what
    assert np.array_equal(idx[clear], o[clear]), (what, np.nonzero(idx[clear] != o[clear]))
    amb = ~clear
    zi = z[np.arange(T), idx]
    ei = e[np.arange(T), idx]
    assert (zi[amb] + ei[amb] >= zmax[amb] - e[np.arange(T), o][amb]).all(), what
    assert (np.abs(val - zi) <= ei + 1e-30).all(), (what, np.abs(val - zi).max())
    return int(clear.sum())
