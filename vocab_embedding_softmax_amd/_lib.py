"""ctypes binding of libvce (include/vce.h).

Argument marshalling only: every function here takes torch tensors that live
on the GPU, checks their dtype/shape/contiguity, allocates outputs and
workspaces with torch when the caller did not pass them, and calls the C entry
point of the same name on the current torch stream. All arithmetic happens in
the library's HIP kernels. Importing this module fails loudly when the library
has not been built.
"""

from __future__ import annotations

import ctypes
import os
from collections import namedtuple
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvce.so")

VCE_F32, VCE_BF16 = 0, 1
REDUCE_MEAN, REDUCE_SUM = 0, 1
ACC_DW, ACC_DH = 1, 2   # flags of vce_bwd's accumulate argument

STATUS = {0: "VCE_OK", 1: "VCE_ERR_NULL", 2: "VCE_ERR_SHAPE", 3: "VCE_ERR_SHARD",
          4: "VCE_ERR_DTYPE", 5: "VCE_ERR_ALIGN", 6: "VCE_ERR_WORKSPACE", 7: "VCE_ERR_HIP"}

# every symbol include/vce.h declares, with its C signature
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
SIGNATURES = {
    "vce_abi_version": (_I32, []),
    "vce_strerror": (ctypes.c_char_p, [_I32]),
    "vce_fwd_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32, _I32]),
    "vce_fwd": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _I32,
                       _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "vce_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32, _I32]),
    "vce_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _I32, _I32, _I32,
                       _P, _P, _I32, _P, _SZ, _P]),
    "vce_bwd_event_count": (_I64, [_I64, _I64, _I64, _I64, _I32, _I32]),
    "vce_bwd_timed": (_I32, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _I32, _I32,
                             _I32, _P, _P, _I32, _P, _SZ, _P, _P, _I64]),
    "vemb_fwd": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _P, _P, _P]),
    "vemb_bwd_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "vemb_bwd": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _I64, _I32, _P, _I32, _P, _SZ, _P]),
    "vce_argmax_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I32, _I32]),
    "vce_argmax": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _SZ,
                          _P]),
    "vce_argmax_noalloc": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _P, _P, _P, _P,
                                  _P]),
    "vngram_fwd": (_I32, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I32, _I32, _P, _P,
                          _P, _P, _P]),
    "vce_fwd_workspace_bytes_ex": (_SZ, [_I64, _I64, _I64, _I64, _I32, _P, _I32]),
    "vce_fwd_ex": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P, _I32, _I32,
                          _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "vce_argmax_workspace_bytes_ex": (_SZ, [_I64, _I64, _I64, _I64, _I32, _P, _I32]),
    "vce_argmax_ex": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _P, _I32, _P, _P, _P, _P, _P,
                             _SZ, _P]),
    "vemb_fwd_ex": (_I32, [_P, _P, _I64, _I64, _I64, _I64, _I32, _P, _I32, _P, _P, _P]),
    "vce_remap": (_I32, [_P, _I64, _P, _I64, _P, _P]),
    "vss_candidates_workspace_bytes": (_SZ, [_I64, _I64]),
    "vss_candidates": (_I32, [_P, _I64, _I64, _I32, _P, _I64, _P, _I64, _P, _P, _P, _P, _SZ, _P]),
    "vss_scatter": (_I32, [_P, _I64, _P, _I64, _I64, _P, _I32, _P]),
    "vss_scatter_replace": (_I32, [_P, _I64, _P, _I64, _P, _I64, _I64, _P, _P]),
}


class VceError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {strerror(status)}")


class BadTargetError(ValueError):
    """Targets outside [0, V_real) other than ignore_index reached the loss.
    The library treats them as ignored and counts them (n_bad_target); the
    binding refuses them unless the caller passes allow_bad=True, as
    PyTorch's cross-entropy refuses an out-of-range class."""

    def __init__(self, n_bad: int):
        self.n_bad = n_bad
        super().__init__(f"{n_bad} target(s) outside [0, V_real) that are not ignore_index "
                         f"(pass allow_bad=True to treat them as ignored)")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"`python vocab_embedding_softmax_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.vce_strerror(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise VceError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return VCE_BF16
    if t.dtype == torch.float32:
        return VCE_F32
    raise TypeError(f"element type must be bfloat16 or float32, got {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _layout(shard_rows, num_shards: int):
    """Host int64 array of an explicit shard layout (num_shards + 1 offsets), or None."""
    if shard_rows is None:
        return None
    rows = [int(x) for x in shard_rows]
    if len(rows) != num_shards + 1:
        raise ValueError(f"shard_rows must hold num_shards + 1 = {num_shards + 1} offsets")
    return (ctypes.c_int64 * len(rows))(*rows)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def read_scalar(t: torch.Tensor, stream=None) -> int:
    """A one-element device tensor's value on the host, after the work queued
    on `stream` (default: the current stream) has finished. Synchronises."""
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    s.synchronize()
    return int(t.cpu().item())


# ------------------------------------------------------------------ sizes

def vce_fwd_workspace_bytes(T, H, V_real, V_pad, num_shards, dtype=VCE_BF16,
                            shard_rows=None) -> int:
    rows = _layout(shard_rows, num_shards)
    if rows is not None:
        return int(lib.vce_fwd_workspace_bytes_ex(T, H, V_real, V_pad, num_shards, rows, dtype))
    return int(lib.vce_fwd_workspace_bytes(T, H, V_real, V_pad, num_shards, dtype))


def vce_bwd_workspace_bytes(T, H, V_real, V_pad, num_shards, dtype=VCE_BF16) -> int:
    return int(lib.vce_bwd_workspace_bytes(T, H, V_real, V_pad, num_shards, dtype))


def vce_bwd_event_count(T, H, V_real, V_pad, num_shards, dt) -> int:
    return int(lib.vce_bwd_event_count(T, H, V_real, V_pad, num_shards, dt))


def vce_argmax_workspace_bytes(T, H, V_real, V_pad, num_shards, dtype=VCE_BF16,
                               shard_rows=None) -> int:
    rows = _layout(shard_rows, num_shards)
    if rows is not None:
        return int(lib.vce_argmax_workspace_bytes_ex(T, H, V_real, V_pad, num_shards, rows,
                                                     dtype))
    return int(lib.vce_argmax_workspace_bytes(T, H, V_real, V_pad, num_shards, dtype))


def vemb_bwd_workspace_bytes(T, H, V_real, V_pad) -> int:
    return int(lib.vemb_bwd_workspace_bytes(T, H, V_real, V_pad))


def vss_candidates_workspace_bytes(T, V) -> int:
    return int(lib.vss_candidates_workspace_bytes(T, V))


# ------------------------------------------------------------------ entry points

FwdOut = namedtuple("FwdOut", "lse loss loss_sum n_valid n_bad shard_stats")


def vce_fwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, V_real: int,
            num_shards: int, ignore_index: int = -100, *, shard_stats: bool = False,
            shard_rows=None, out: Optional[FwdOut] = None, ws: Optional[torch.Tensor] = None,
            allow_bad: bool = False, stream=None) -> FwdOut:
    """Cross-entropy forward. h [T,H], W [V_pad,H] (same dtype), targets [T] int32.
    shard_rows (optional): num_shards + 1 row offsets of an explicit layout
    (calls vce_fwd_ex).

    Bad targets (outside [0, V_real), not ignore_index): the library counts
    them in n_bad and treats them as ignored. With allow_bad=False (default)
    this call then waits for the forward (a stream synchronisation) and raises
    BadTargetError if any was counted; allow_bad=True skips that check (no
    synchronisation: use it under graph capture or where the caller reads
    n_bad itself)."""
    T, H = h.shape
    V_pad = W.shape[0]
    dt = _dt(h)
    _need(h, "h")
    _need(W, "W", h.dtype, (V_pad, H))
    _need(targets, "targets", torch.int32, (T,))
    dev = h.device
    if out is None:
        f = dict(dtype=torch.float32, device=dev)
        i = dict(dtype=torch.int32, device=dev)
        out = FwdOut(torch.empty(T, **f), torch.empty(T, **f), torch.empty(1, **f),
                     torch.empty(1, **i), torch.empty(1, **i),
                     torch.empty(2, num_shards, T, **f) if shard_stats else None)
    rows = _layout(shard_rows, num_shards)
    need = vce_fwd_workspace_bytes(T, H, V_real, V_pad, num_shards, dt, shard_rows)
    ws = _workspace(need, dev, ws)
    outs = (_ptr(out.lse), _ptr(out.loss), _ptr(out.loss_sum), _ptr(out.n_valid),
            _ptr(out.n_bad), _ptr(out.shard_stats), _ptr(ws), ws.numel(), _stream(stream, dev))
    if rows is None:
        st = lib.vce_fwd(_ptr(h), _ptr(W), _ptr(targets), T, H, V_real, V_pad, num_shards,
                         ignore_index, dt, *outs)
        _check("vce_fwd", st)
    else:
        st = lib.vce_fwd_ex(_ptr(h), _ptr(W), _ptr(targets), T, H, V_real, V_pad, num_shards,
                            rows, ignore_index, dt, *outs)
        _check("vce_fwd_ex", st)
    if not allow_bad:
        nb = read_scalar(out.n_bad, stream)
        if nb:
            raise BadTargetError(nb)
    return out


BwdOut = namedtuple("BwdOut", "dh dW")


def vce_bwd(h: torch.Tensor, W: torch.Tensor, targets: torch.Tensor, lse: torch.Tensor,
            grad_loss: torch.Tensor, n_valid: torch.Tensor, V_real: int, num_shards: int,
            ignore_index: int = -100, reduction: int = REDUCE_MEAN, *,
            dh: Optional[torch.Tensor] = None, dW: Optional[torch.Tensor] = None,
            accumulate_dW: bool = False, accumulate_dh: bool = False,
            ws: Optional[torch.Tensor] = None, stream=None, events=None) -> BwdOut:
    """Cross-entropy backward: dh [T,H] and dW [V_pad,H] (float32), overwritten
    or (accumulate_dW / accumulate_dh) added into. `events`
    (optional): vce_bwd_event_count(...) torch.cuda.Event objects, recorded
    before the first kernel and after each vocabulary chunk's G, dh and dW
    kernels (calls vce_bwd_timed)."""
    T, H = h.shape
    V_pad = W.shape[0]
    dt = _dt(h)
    _need(h, "h")
    _need(W, "W", h.dtype, (V_pad, H))
    _need(targets, "targets", torch.int32, (T,))
    _need(lse, "lse", torch.float32, (T,))
    _need(grad_loss, "grad_loss", torch.float32)
    _need(n_valid, "n_valid", torch.int32)
    dev = h.device
    if (accumulate_dh and dh is None) or (accumulate_dW and dW is None):
        raise ValueError("accumulating needs the tensor to add into")
    if dh is None:
        dh = torch.empty(T, H, dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty(V_pad, H, dtype=torch.float32, device=dev)
    _need(dh, "dh", torch.float32, (T, H))
    _need(dW, "dW", torch.float32, (V_pad, H))
    need = vce_bwd_workspace_bytes(T, H, V_real, V_pad, num_shards, dt)
    ws = _workspace(need, dev, ws)
    args = (_ptr(h), _ptr(W), _ptr(targets), _ptr(lse), _ptr(grad_loss), _ptr(n_valid),
            reduction, T, H, V_real, V_pad, num_shards, ignore_index, dt, _ptr(dh), _ptr(dW),
            (ACC_DW if accumulate_dW else 0) | (ACC_DH if accumulate_dh else 0), _ptr(ws),
            ws.numel(), _stream(stream, dev))
    if events is None:
        _check("vce_bwd", lib.vce_bwd(*args))
    else:
        n_ev = vce_bwd_event_count(T, H, V_real, V_pad, num_shards, dt)
        if len(events) != n_ev:
            raise ValueError(f"events must hold {n_ev} torch.cuda.Event objects")
        for e in events:
            if e.cuda_event == 0:   # created lazily by torch: force creation on this device
                e.record(torch.cuda.current_stream(dev))
        arr = (ctypes.c_void_p * n_ev)(*[e.cuda_event for e in events])
        _check("vce_bwd_timed", lib.vce_bwd_timed(*args, arr, n_ev))
    return BwdOut(dh, dW)


ArgOut = namedtuple("ArgOut", "index value shard_value shard_index")


def vce_argmax(h: torch.Tensor, W: torch.Tensor, V_real: int, num_shards: int, *,
               shard_reports: bool = False, shard_rows=None, out: Optional[ArgOut] = None,
               ws: Optional[torch.Tensor] = None, stream=None) -> ArgOut:
    """Greedy argmax over the real rows: index [T] int32, value [T] float32, and
    (shard_reports=True) each shard's (value, index) [num_shards, T].
    shard_rows (optional): an explicit layout (calls vce_argmax_ex)."""
    T, H = h.shape
    V_pad = W.shape[0]
    dt = _dt(h)
    _need(h, "h")
    _need(W, "W", h.dtype, (V_pad, H))
    dev = h.device
    if out is None:
        f = dict(dtype=torch.float32, device=dev)
        i = dict(dtype=torch.int32, device=dev)
        out = ArgOut(torch.empty(T, **i), torch.empty(T, **f),
                     torch.empty(num_shards, T, **f) if shard_reports else None,
                     torch.empty(num_shards, T, **i) if shard_reports else None)
    rows = _layout(shard_rows, num_shards)
    need = vce_argmax_workspace_bytes(T, H, V_real, V_pad, num_shards, dt, shard_rows)
    ws = _workspace(need, dev, ws)
    outs = (_ptr(out.index), _ptr(out.value), _ptr(out.shard_value), _ptr(out.shard_index),
            _ptr(ws), ws.numel(), _stream(stream, dev))
    if rows is None:
        st = lib.vce_argmax(_ptr(h), _ptr(W), T, H, V_real, V_pad, num_shards, dt, *outs)
        _check("vce_argmax", st)
    else:
        st = lib.vce_argmax_ex(_ptr(h), _ptr(W), T, H, V_real, V_pad, num_shards, rows, dt,
                               *outs)
        _check("vce_argmax_ex", st)
    return out


def vce_argmax_noalloc(h: torch.Tensor, W: torch.Tensor, V_real: int, num_shards: int, *,
                       shard_reports: bool = False, out: Optional[ArgOut] = None,
                       stream=None) -> ArgOut:
    """vce_argmax with the library's static scratch instead of a workspace
    (nothing is allocated when `out` is given)."""
    T, H = h.shape
    V_pad = W.shape[0]
    dt = _dt(h)
    _need(h, "h")
    _need(W, "W", h.dtype, (V_pad, H))
    dev = h.device
    if out is None:
        f = dict(dtype=torch.float32, device=dev)
        i = dict(dtype=torch.int32, device=dev)
        out = ArgOut(torch.empty(T, **i), torch.empty(T, **f),
                     torch.empty(num_shards, T, **f) if shard_reports else None,
                     torch.empty(num_shards, T, **i) if shard_reports else None)
    st = lib.vce_argmax_noalloc(_ptr(h), _ptr(W), T, H, V_real, V_pad, num_shards, dt,
                                _ptr(out.index), _ptr(out.value), _ptr(out.shard_value),
                                _ptr(out.shard_index), _stream(stream, dev))
    _check("vce_argmax_noalloc", st)
    return out


def vemb_fwd(ids: torch.Tensor, W: torch.Tensor, V_real: int, num_shards: int, *,
             out: Optional[torch.Tensor] = None, n_bad: Optional[torch.Tensor] = None,
             count_bad: bool = True, shard_rows=None, stream=None):
    """Masked lookup: returns (out [T,H] in W's dtype, n_bad [1] int32 or None).
    shard_rows (optional): an explicit layout (calls vemb_fwd_ex)."""
    T = ids.shape[0]
    V_pad, H = W.shape
    dt = _dt(W)
    _need(ids, "ids", torch.int32, (T,))
    _need(W, "W")
    dev = W.device
    if out is None:
        out = torch.empty(T, H, dtype=W.dtype, device=dev)
    _need(out, "out", W.dtype, (T, H))
    if count_bad and n_bad is None:
        n_bad = torch.empty(1, dtype=torch.int32, device=dev)
    rows = _layout(shard_rows, num_shards)
    tail = (_ptr(out), _ptr(n_bad) if count_bad else None, _stream(stream, dev))
    if rows is None:
        st = lib.vemb_fwd(_ptr(ids), _ptr(W), T, H, V_real, V_pad, num_shards, dt, *tail)
        _check("vemb_fwd", st)
    else:
        st = lib.vemb_fwd_ex(_ptr(ids), _ptr(W), T, H, V_real, V_pad, num_shards, rows, dt,
                             *tail)
        _check("vemb_fwd_ex", st)
    return out, n_bad


def vce_remap(ids: torch.Tensor, row_of: torch.Tensor, *, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """Mapped ownership: out[t] = row_of[ids[t]] for IDs in [0, V_real), else
    ids[t] (V_real = row_of's length). out may be ids itself."""
    T = ids.shape[0]
    V_real = row_of.shape[0]
    _need(ids, "ids", torch.int32, (T,))
    _need(row_of, "row_of", torch.int32, (V_real,))
    dev = ids.device
    if out is None:
        out = torch.empty(T, dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, (T,))
    _check("vce_remap", lib.vce_remap(_ptr(ids), T, _ptr(row_of), V_real, _ptr(out),
                                      _stream(stream, dev)))
    return out


NgramOut = namedtuple("NgramOut", "out ids2 ids3 n_bad")


def vngram_fwd(ids: torch.Tensor, E: torch.Tensor, E2: torch.Tensor, E3: torch.Tensor,
               V_real: int, num_shards: int, *, out: Optional[NgramOut] = None,
               stream=None) -> NgramOut:
    """Hashed n-gram input embedding: out [T,H] (E's dtype) = unigram + 2-gram +
    3-gram rows; ids2 / ids3 [T] int32 table rows (-1: missing); n_bad [1]."""
    T = ids.shape[0]
    V_pad, H = E.shape
    dt = _dt(E)
    _need(ids, "ids", torch.int32, (T,))
    _need(E, "E")
    _need(E2, "E2", E.dtype)
    _need(E3, "E3", E.dtype)
    if E2.shape[1] != H or E3.shape[1] != H:
        raise ValueError("E, E2 and E3 must have the same row width")
    dev = E.device
    if out is None:
        i = dict(dtype=torch.int32, device=dev)
        out = NgramOut(torch.empty(T, H, dtype=E.dtype, device=dev), torch.empty(T, **i),
                       torch.empty(T, **i), torch.empty(1, **i))
    st = lib.vngram_fwd(_ptr(ids), _ptr(E), _ptr(E2), _ptr(E3), T, H, V_real, V_pad,
                        E2.shape[0], E3.shape[0], num_shards, dt, _ptr(out.out), _ptr(out.ids2),
                        _ptr(out.ids3), _ptr(out.n_bad), _stream(stream, dev))
    _check("vngram_fwd", st)
    return out


def vemb_bwd(ids: torch.Tensor, dout: torch.Tensor, V_real: int, V_pad: int, num_shards: int,
             *, dW: Optional[torch.Tensor] = None, accumulate: bool = False,
             ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Scatter-add of dout rows into dW [V_pad, H] (float32) by ID."""
    T, H = dout.shape
    dt = _dt(dout)
    _need(ids, "ids", torch.int32, (T,))
    _need(dout, "dout")
    dev = dout.device
    if dW is None:
        if accumulate:
            raise ValueError("accumulate=True needs dW")
        dW = torch.empty(V_pad, H, dtype=torch.float32, device=dev)
    _need(dW, "dW", torch.float32, (V_pad, H))
    need = vemb_bwd_workspace_bytes(T, H, V_real, V_pad)
    ws = _workspace(need, dev, ws)
    st = lib.vemb_bwd(_ptr(ids), _ptr(dout), dt, T, H, V_real, V_pad, num_shards, _ptr(dW),
                      1 if accumulate else 0, _ptr(ws), ws.numel(), _stream(stream, dev))
    _check("vemb_bwd", st)
    return dW


CandOut = namedtuple("CandOut", "cand pos n_unique n_cand")


def vss_candidates(targets: torch.Tensor, V: int, perm: torch.Tensor, P: int,
                   ignore_index: int = -100, *, out: Optional[CandOut] = None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> CandOut:
    """Sampled-softmax candidates: cand [cap], pos [T], n_unique [1], n_cand [1] (int32)."""
    T = targets.shape[0]
    _need(targets, "targets", torch.int32, (T,))
    _need(perm, "perm", torch.int32, (V,))
    dev = targets.device
    cap = max(P, min(T, V))
    if out is None:
        i = dict(dtype=torch.int32, device=dev)
        out = CandOut(torch.empty(cap, **i), torch.empty(T, **i), torch.empty(1, **i),
                      torch.empty(1, **i))
    need = vss_candidates_workspace_bytes(T, V)
    ws = _workspace(need, dev, ws)
    st = lib.vss_candidates(_ptr(targets), T, V, ignore_index, _ptr(perm), P, _ptr(out.cand),
                            out.cand.numel(), _ptr(out.pos), _ptr(out.n_unique), _ptr(out.n_cand),
                            _ptr(ws), ws.numel(), _stream(stream, dev))
    _check("vss_candidates", st)
    return out


def vss_scatter(cand: torch.Tensor, dWc: torch.Tensor, V: int, *,
                dW: Optional[torch.Tensor] = None, accumulate: bool = False,
                stream=None) -> torch.Tensor:
    """Candidate rows' gradient back to the table: dW[cand[i]] (+)= dWc[i] for
    cand entries in [0, V), which must be distinct. cand [P] int32, dWc [P, H]
    float32; dW [V, H] float32 (every other row zeroed unless accumulate)."""
    P, H = dWc.shape
    _need(cand, "cand", torch.int32, (P,))
    _need(dWc, "dWc", torch.float32, (P, H))
    dev = dWc.device
    if dW is None:
        dW = torch.empty(V, H, dtype=torch.float32, device=dev)
    _need(dW, "dW", torch.float32, (V, H))
    st = lib.vss_scatter(_ptr(cand), P, _ptr(dWc), H, V, _ptr(dW), 1 if accumulate else 0,
                         _stream(stream, dev))
    _check("vss_scatter", st)
    return dW


def vss_scatter_replace(prev: Optional[torch.Tensor], cand: torch.Tensor, dWc: torch.Tensor,
                        dW: torch.Tensor, *, stream=None) -> torch.Tensor:
    """dW [V, H] float32 holds nonzero values only in the rows listed in prev
    (the previous call's candidates; None or empty for a zero table): those
    rows are cleared, then dW[cand[i]] = dWc[i]. Same table as
    vss_scatter(cand, dWc, V, dW=dW) with accumulate=False."""
    P, H = dWc.shape
    _need(cand, "cand", torch.int32, (P,))
    _need(dWc, "dWc", torch.float32, (P, H))
    V = dW.shape[0]
    _need(dW, "dW", torch.float32, (V, H))
    n_prev = 0 if prev is None else prev.shape[0]
    if n_prev:
        _need(prev, "prev", torch.int32, (n_prev,))
    st = lib.vss_scatter_replace(_ptr(prev) if n_prev else None, n_prev, _ptr(cand), P,
                                 _ptr(dWc), H, V, _ptr(dW), _stream(stream, dWc.device))
    _check("vss_scatter_replace", st)
    return dW
