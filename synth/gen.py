"""Seeded generators: random hidden rows, table rows, targets and token IDs.

Every tensor draws from its own child stream of
``numpy.random.SeedSequence(seed).spawn(8)`` so that changing one tensor's
recipe never shifts the bits of another. bf16 tensors are produced by rounding
float32 draws to nearest-even once, and are handed out as their raw uint16 bit
patterns: both sides of every comparison decode the same bits.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

INT32_MIN = -(2**31)
INT32_MAX = 2**31 - 1

# child-stream slots of SeedSequence(seed).spawn(8)
_S_H, _S_W, _S_TGT, _S_IGN, _S_IDS, _S_IDX, _S_PERM, _S_SPARE = range(8)


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(8)]


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits.

    NaN inputs become a quiet NaN with the same sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
         >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def zipf_ids(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """Draw ``n`` IDs from a Zipf law truncated to ``[0, V)``: P(id = k-1) ~ k**-s.

    No permutation is applied, so ID 0 is the most frequent. Sampling is by
    inverse CDF on a float64 cumulative sum.
    """
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-float(s))
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int64)


def _normal_rows(rng, rows: int, cols: int, std: float, chunk: int = 8192):
    """float32 N(0, std^2) of shape [rows, cols], drawn in row chunks."""
    out = np.empty((rows, cols), dtype=np.float32)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        blk = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r1] = blk
    return out


def _rms_rows(x: np.ndarray) -> np.ndarray:
    """Scale each row to unit root-mean-square (no epsilon, no weight).

    Only shapes the synthetic hidden input; it is not part of the path.
    """
    ms = np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True)
    return (x / np.sqrt(ms)).astype(np.float32)


def _encode(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x_f32)
    raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")


def _table(rng, V_real: int, V_pad: int, H: int, std: float, dtype: str,
           pad_fill: Optional[float]) -> np.ndarray:
    """Table [V_pad, H]. Real rows N(0, std^2); padded rows N(0, std^2) too,
    unless ``pad_fill`` gives a constant (e.g. +8.0 or NaN) for every padded element."""
    chunk = 16384
    if dtype == "f32":
        W = np.empty((V_pad, H), dtype=np.float32)
    else:
        W = np.empty((V_pad, H), dtype=np.uint16)
    for r0 in range(0, V_pad, chunk):
        r1 = min(V_pad, r0 + chunk)
        blk = rng.standard_normal((r1 - r0, H), dtype=np.float32)
        blk *= np.float32(std)
        if pad_fill is not None and r1 > V_real:
            blk[max(0, V_real - r0):] = np.float32(pad_fill)
        W[r0:r1] = _encode(blk, dtype)
    return W


def _choose_positions(rng, T: int, count: int, avoid: Sequence[int] = ()) -> np.ndarray:
    """``count`` distinct positions in [0, T), none in ``avoid``, in increasing order."""
    avoid_set = set(int(a) for a in avoid)
    order = rng.permutation(T)
    pos = [int(p) for p in order if int(p) not in avoid_set][:count]
    if len(pos) < count:
        raise ValueError("not enough positions")
    return np.array(sorted(pos), dtype=np.int64)


def _oob_values(count: int, V: int) -> np.ndarray:
    """Out-of-range IDs: alternately negative values and values >= V."""
    neg = [-1, -100, INT32_MIN, -2, -V]
    big = [V, V + 12345, INT32_MAX, V + 1]
    vals = []
    for i in range(count):
        if i % 2 == 0:
            vals.append(neg[(i // 2) % len(neg)])
        else:
            vals.append(big[(i // 2) % len(big)])
    return np.array(vals, dtype=np.int64)


@dataclasses.dataclass
class CEInputs:
    """One workload's arrays. ``h``/``W`` are float32 (dtype 'f32') or uint16 bf16 bits."""
    T: int
    H: int
    V_real: int
    V_pad: int
    num_shards: int
    dtype: str
    ignore_index: int
    h: Optional[np.ndarray]          # [T, H]; None for the tied workload (h is gathered)
    W: np.ndarray                    # [V_pad, H]
    targets: np.ndarray              # [T] int32
    ids: Optional[np.ndarray] = None  # [T] int32 embedding input IDs
    perm: Optional[np.ndarray] = None  # [V_real] int32 random permutation (sampled softmax)
    P: int = 0                       # sampled-softmax candidate count
    forced_positions: Optional[np.ndarray] = None
    name: str = ""

    @property
    def S(self) -> int:
        return self.V_pad // self.num_shards


def make_ce_inputs(T: int, H: int, V_real: int, V_pad: int, num_shards: int,
                   dtype: str = "bf16", seed: int = 0, *,
                   target_dist: str = "uniform", zipf_s: float = 1.1,
                   ignore_frac: float = 0.0, ignore_index: int = -100,
                   forced_targets: Sequence[int] = (),
                   h_dist: str = "normal", w_std: float = 0.02,
                   pad_fill: Optional[float] = None,
                   id_dist: Optional[str] = None, id_repeat_frac: float = 0.0,
                   id_extra: Sequence[int] = (), name: str = "") -> CEInputs:
    """Inputs for the cross-entropy (and optionally embedding) path.

    target_dist: 'uniform' over [0, V_real) or 'zipf' (truncated, exponent zipf_s).
    ignore_frac: round(frac*T) positions (never a forced one) get ignore_index.
    forced_targets: values written at the first seeded positions.
    h_dist: 'normal' = N(0,1); 'rms' = N(0,1) rows scaled to unit RMS.
    pad_fill: constant for every element of the padded rows (None = random like real rows).
    id_dist: None (no IDs), 'uniform' or 'zipf'; id_repeat_frac of positions copy an
      earlier position's ID; id_extra values are written at seeded positions.
    """
    rs = _streams(seed)
    if h_dist == "normal":
        hf = _normal_rows(rs[_S_H], T, H, 1.0)
    elif h_dist == "rms":
        hf = _rms_rows(_normal_rows(rs[_S_H], T, H, 1.0))
    else:
        raise ValueError(h_dist)
    h = _encode(hf, dtype)
    W = _table(rs[_S_W], V_real, V_pad, H, w_std, dtype, pad_fill)

    if target_dist == "uniform":
        tgt = rs[_S_TGT].integers(0, V_real, size=T).astype(np.int64)
    elif target_dist == "zipf":
        tgt = zipf_ids(rs[_S_TGT], T, V_real, zipf_s)
    else:
        raise ValueError(target_dist)
    forced = np.array(list(forced_targets), dtype=np.int64)
    fpos = _choose_positions(rs[_S_IGN], T, len(forced)) if len(forced) else np.zeros(0, np.int64)
    tgt[fpos] = forced
    n_ign = int(round(ignore_frac * T))
    if n_ign:
        ipos = _choose_positions(rs[_S_IGN], T, n_ign, avoid=fpos)
        tgt[ipos] = ignore_index

    ids = None
    if id_dist is not None:
        if id_dist == "uniform":
            ids = rs[_S_IDS].integers(0, V_real, size=T).astype(np.int64)
        elif id_dist == "zipf":
            ids = zipf_ids(rs[_S_IDS], T, V_real, zipf_s)
        else:
            raise ValueError(id_dist)
        n_rep = int(round(id_repeat_frac * T))
        if n_rep and T > 1:
            rpos = _choose_positions(rs[_S_IDX], T - 1, n_rep) + 1
            for p in rpos:
                ids[p] = ids[int(rs[_S_IDX].integers(0, p))]
        if len(id_extra):
            epos = _choose_positions(rs[_S_IDX], T, len(id_extra))
            ids[epos] = np.array(list(id_extra), dtype=np.int64)
        ids = ids.astype(np.int32)

    return CEInputs(T=T, H=H, V_real=V_real, V_pad=V_pad, num_shards=num_shards,
                    dtype=dtype, ignore_index=ignore_index, h=h, W=W,
                    targets=tgt.astype(np.int32), ids=ids, forced_positions=fpos,
                    name=name)


def make_tied_inputs(T: int, H: int, V_real: int, V_pad: int, num_shards: int,
                     dtype: str = "bf16", seed: int = 0, *, zipf_s: float = 1.1,
                     oob_frac: float = 0.01, ignore_frac: float = 0.02,
                     ignore_index: int = -100, w_std: float = 0.02,
                     pad_fill: Optional[float] = None, name: str = "") -> CEInputs:
    """Tied embedding + LM-head step: a Zipf token stream of T+1 tokens;
    input IDs are tokens[:-1] with round(oob_frac*T) replaced by out-of-range
    values, targets are tokens[1:] with round(ignore_frac*T) set to ignore_index.
    The hidden input is not drawn: it is the embedding of the IDs."""
    rs = _streams(seed)
    W = _table(rs[_S_W], V_real, V_pad, H, w_std, dtype, pad_fill)
    tokens = zipf_ids(rs[_S_TGT], T + 1, V_real, zipf_s)
    ids = tokens[:-1].copy()
    tgt = tokens[1:].copy()
    n_oob = int(round(oob_frac * T))
    if n_oob:
        opos = _choose_positions(rs[_S_IDX], T, n_oob)
        ids[opos] = _oob_values(n_oob, V_real)
    n_ign = int(round(ignore_frac * T))
    if n_ign:
        ipos = _choose_positions(rs[_S_IGN], T, n_ign)
        tgt[ipos] = ignore_index
    return CEInputs(T=T, H=H, V_real=V_real, V_pad=V_pad, num_shards=num_shards,
                    dtype=dtype, ignore_index=ignore_index, h=None, W=W,
                    targets=tgt.astype(np.int32), ids=ids.astype(np.int32), name=name)


def make_oth_inputs(T: int, H: int, V_real: int, V_pad: int, num_shards: int,
                    dtype: str = "bf16", seed: int = 0, **kw):
    """The tied-step inputs (make_tied_inputs, same arguments and draws) plus,
    for the second head of the OT-H step, its table W2 (same distribution and
    geometry, its own stream) and its targets: the tokens two positions ahead
    of rows 0..T-2, i.e. targets[1:] of the tied step.
    Returns (CEInputs, W2, targets2)."""
    inp = make_tied_inputs(T, H, V_real, V_pad, num_shards, dtype, seed, **kw)
    rs = _streams(seed)
    W2 = _table(rs[_S_SPARE], V_real, V_pad, H, kw.get("w_std", 0.02), dtype, kw.get("pad_fill"))
    return inp, W2, inp.targets[1:].copy()


def make_sampled_inputs(T: int, H: int, V: int, P: int, dtype: str = "bf16",
                        seed: int = 0, *, zipf_s: float = 1.1, ignore_frac: float = 0.0,
                        ignore_index: int = -100, w_std: float = 0.02,
                        h_dist: str = "rms", name: str = "") -> CEInputs:
    """Sampled-softmax inputs: hidden rows, table [V, H], Zipf targets and a
    uniformly random permutation of [0, V) that supplies the negatives."""
    rs = _streams(seed)
    if h_dist == "rms":
        hf = _rms_rows(_normal_rows(rs[_S_H], T, H, 1.0))
    else:
        hf = _normal_rows(rs[_S_H], T, H, 1.0)
    h = _encode(hf, dtype)
    W = _table(rs[_S_W], V, V, H, w_std, dtype, None)
    tgt = zipf_ids(rs[_S_TGT], T, V, zipf_s)
    n_ign = int(round(ignore_frac * T))
    if n_ign:
        ipos = _choose_positions(rs[_S_IGN], T, n_ign)
        tgt[ipos] = ignore_index
    perm = rs[_S_PERM].permutation(V).astype(np.int32)
    return CEInputs(T=T, H=H, V_real=V, V_pad=V, num_shards=1, dtype=dtype,
                    ignore_index=ignore_index, h=h, W=W, targets=tgt.astype(np.int32),
                    perm=perm, P=P, name=name)


def make_layout(V_pad: int, num_shards: int, seed: int, n_empty: int = 0,
                n_single: int = 0) -> np.ndarray:
    """A seeded uneven shard layout: num_shards + 1 int64 row offsets from 0 to
    V_pad, nondecreasing. n_empty shards own no row and n_single shards own one
    row (chosen at seeded positions); the rest split the remaining rows at
    uniformly drawn cut points."""
    rng = np.random.default_rng(seed)
    kinds = np.zeros(num_shards, dtype=np.int64)          # 0 free, 1 empty, 2 one row
    pick = rng.permutation(num_shards)
    kinds[pick[:n_empty]] = 1
    kinds[pick[n_empty:n_empty + n_single]] = 2
    free = int((kinds == 0).sum())
    rest = V_pad - n_single
    if free == 0 and rest != 0:
        raise ValueError("no shard left for the remaining rows")
    cuts = np.sort(rng.integers(0, rest + 1, size=max(free - 1, 0)))
    sizes_free = np.diff(np.concatenate([[0], cuts, [rest]]))
    sizes = np.zeros(num_shards, dtype=np.int64)
    sizes[kinds == 2] = 1
    sizes[kinds == 0] = sizes_free
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def make_row_map(V_real: int, seed: int) -> np.ndarray:
    """A seeded permutation of [0, V_real) (class -> physical row), int32."""
    return np.random.default_rng(seed).permutation(V_real).astype(np.int32)
