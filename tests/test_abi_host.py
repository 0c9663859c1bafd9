"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (so these run
without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vce.h")

vce = pytest.importorskip("vocab_embedding_softmax_amd._lib",
                          reason="libvce.so not built (python vocab_embedding_softmax_amd/build.py)")
lib = vce.lib

OK, NULL, SHAPE, SHARD, DTYPE, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5, 6

# fake, never dereferenced device addresses (16-byte aligned unless stated)
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10008)  # 8-byte aligned only
NUL = None


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"defined"})


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(lib, n), n
        assert n in vce.SIGNATURES, n


def test_version_and_strerror():
    assert lib.vce_abi_version() == 1
    for s in range(8):
        assert vce.strerror(s)
    assert vce.strerror(99) == "unknown status"


def _fwd(T=4, H=64, V_real=1000, V_pad=1024, n=4, ign=-100, dt=1, h=A, W=B, tg=C, lse=A,
         loss=B, ls=C, nv=A, nb=B, ss=NUL, ws=A, wsb=1 << 40):
    return lib.vce_fwd(h, W, tg, T, H, V_real, V_pad, n, ign, dt, lse, loss, ls, nv, nb, ss, ws,
                       wsb, None)


def test_fwd_argument_errors():
    assert _fwd(n=3) == SHARD
    assert _fwd(n=0) == SHARD
    assert _fwd(V_real=0) == SHAPE
    assert _fwd(V_real=1025) == SHAPE
    assert _fwd(T=-1) == SHAPE
    assert _fwd(H=0) == SHAPE
    assert _fwd(ign=5) == SHAPE          # ignore_index must not be a real class
    assert _fwd(dt=7) == DTYPE
    assert _fwd(h=NUL) == NULL
    assert _fwd(ls=NUL) == NULL
    assert _fwd(H=60) == ALIGN
    assert _fwd(W=MIS) == ALIGN
    assert _fwd(ws=NUL) == WORKSPACE
    need = lib.vce_fwd_workspace_bytes(4, 64, 1000, 1024, 4, 1)
    assert need > 0
    assert _fwd(wsb=need - 1) == WORKSPACE


def _bwd(T=4, H=64, V_real=1000, V_pad=1024, n=4, ign=-100, dt=1, red=0, dh=A, dW=B, gl=C,
         nv=A, ws=A, wsb=1 << 40, h=A):
    return lib.vce_bwd(h, B, C, A, gl, nv, red, T, H, V_real, V_pad, n, ign, dt, dh, dW, 0, ws,
                       wsb, None)


def test_bwd_argument_errors():
    assert _bwd(n=5) == SHARD
    assert _bwd(red=2) == DTYPE
    assert _bwd(dW=NUL) == NULL
    assert _bwd(gl=NUL) == NULL
    assert _bwd(nv=NUL) == NULL            # needed for the mean
    assert _bwd(h=NUL) == NULL
    assert _bwd(dh=MIS) == ALIGN
    need = lib.vce_bwd_workspace_bytes(4, 64, 1000, 1024, 4, 1)
    assert need > 0
    assert _bwd(wsb=need - 1) == WORKSPACE
    assert _bwd(ign=0) == SHAPE


def test_emb_argument_errors():
    assert lib.vemb_fwd(A, B, 4, 64, 1000, 1024, 3, 1, C, NUL, None) == SHARD
    assert lib.vemb_fwd(A, B, 4, 64, 1000, 1024, 4, 9, C, NUL, None) == DTYPE
    assert lib.vemb_fwd(NUL, B, 4, 64, 1000, 1024, 4, 1, C, NUL, None) == NULL
    assert lib.vemb_fwd(A, B, 4, 12, 1000, 1024, 4, 1, C, NUL, None) == ALIGN
    assert lib.vemb_fwd(A, MIS, 4, 64, 1000, 1024, 4, 1, C, NUL, None) == ALIGN
    need = lib.vemb_bwd_workspace_bytes(4, 64, 1000, 1024)
    assert need > 0
    assert lib.vemb_bwd(A, B, 0, 4, 64, 1000, 1024, 4, C, 1, A, need - 1, None) == WORKSPACE
    assert lib.vemb_bwd(A, B, 0, 4, 64, 1000, 1024, 4, NUL, 1, A, need, None) == NULL
    assert lib.vemb_bwd(A, B, 0, 4, 64, 1001, 1000, 4, C, 1, A, need, None) == SHAPE


def test_argmax_argument_errors():
    need = lib.vce_argmax_workspace_bytes(4, 64, 1000, 1024, 4, 1)
    assert need > 0
    args = lambda T=4, H=64, Vr=1000, Vp=1024, n=4, dt=1, h=A, W=B, idx=C, val=A, ws=A, \
        wsb=need: lib.vce_argmax(h, W, T, H, Vr, Vp, n, dt, idx, val, NUL, NUL, ws, wsb, None)
    assert args(n=3) == SHARD
    assert args(dt=7) == DTYPE
    assert args(Vr=1025) == SHAPE
    assert args(h=NUL) == NULL
    assert args(idx=NUL) == NULL
    assert args(H=12) == ALIGN
    assert args(W=MIS) == ALIGN
    assert args(wsb=need - 1) == WORKSPACE
    assert args(ws=NUL) == WORKSPACE
    assert args(T=0, h=NUL, W=NUL, idx=NUL, val=NUL, ws=NUL, wsb=0) == OK  # nothing to do
    assert lib.vce_argmax_workspace_bytes(8, 64, 100, 101, 2, 1) == 0     # 101 % 2 != 0


def _rows(*r):
    return (ctypes.c_int64 * len(r))(*r)


def test_uneven_layout_argument_errors():
    good = _rows(0, 100, 100, 601, 1000)            # one empty shard, V_pad not a multiple of 4
    need = lib.vce_fwd_workspace_bytes_ex(4, 64, 990, 1000, 4, good, 1)
    assert need > 0
    assert lib.vce_fwd_workspace_bytes_ex(4, 64, 990, 1000, 4, _rows(0, 600, 500, 900, 1000),
                                          1) == 0     # decreasing
    assert lib.vce_fwd_workspace_bytes_ex(4, 64, 990, 1000, 4, NUL, 1) == 0

    def fwd(rows=good, n=4, Vr=990, Vp=1000, h=A, ws=A, wsb=need):
        return lib.vce_fwd_ex(h, B, C, 4, 64, Vr, Vp, n, rows, -100, 1, A, B, C, A, B, NUL, ws,
                              wsb, None)
    assert fwd(rows=NUL) == NULL
    assert fwd(rows=_rows(0, 100, 100, 601, 999)) == SHARD    # does not end at V_pad
    assert fwd(rows=_rows(1, 100, 100, 601, 1000)) == SHARD   # does not start at 0
    assert fwd(rows=_rows(0, 700, 600, 900, 1000)) == SHARD   # decreasing
    assert fwd(n=129, rows=_rows(*[min(7 * i, 1000) for i in range(129)], 1000)) == SHARD
    assert fwd(Vr=1001) == SHAPE
    assert fwd(h=NUL) == NULL
    assert fwd(wsb=need - 1) == WORKSPACE

    aneed = lib.vce_argmax_workspace_bytes_ex(4, 64, 990, 1000, 4, good, 1)
    assert aneed > 0
    assert lib.vce_argmax_ex(A, B, 4, 64, 990, 1000, 4, NUL, 1, C, A, NUL, NUL, A, aneed,
                             None) == NULL
    assert lib.vce_argmax_ex(A, B, 4, 64, 990, 1000, 4, _rows(0, 1, 2, 3, 4), 1, C, A, NUL, NUL,
                             A, aneed, None) == SHARD
    assert lib.vce_argmax_ex(A, B, 4, 64, 990, 1000, 4, good, 1, C, A, NUL, NUL, A, aneed - 1,
                             None) == WORKSPACE
    assert lib.vemb_fwd_ex(A, B, 4, 64, 990, 1000, 4, NUL, 1, C, NUL, None) == NULL
    assert lib.vemb_fwd_ex(A, B, 4, 64, 990, 1000, 4, _rows(0, 5, 4, 6, 1000), 1, C, NUL,
                           None) == SHARD
    assert lib.vemb_fwd_ex(A, MIS, 4, 64, 990, 1000, 4, good, 1, C, NUL, None) == ALIGN
    assert lib.vemb_fwd_ex(A, B, 0, 64, 990, 1000, 4, good, 1, NUL, NUL, None) == OK
    # the even layout written out is accepted wherever the even call is
    even = _rows(0, 256, 512, 768, 1024)
    assert lib.vce_fwd_workspace_bytes_ex(4, 64, 1000, 1024, 4, even, 1) > 0


def test_remap_argument_errors():
    assert lib.vce_remap(A, 4, B, 0, C, None) == SHAPE
    assert lib.vce_remap(A, -1, B, 10, C, None) == SHAPE
    assert lib.vce_remap(NUL, 4, B, 10, C, None) == NULL
    assert lib.vce_remap(A, 4, NUL, 10, C, None) == NULL
    assert lib.vce_remap(ctypes.c_void_p(0x10002), 4, B, 10, C, None) == ALIGN
    assert lib.vce_remap(NUL, 0, NUL, 10, NUL, None) == OK     # nothing to do


def test_ngram_argument_errors():
    def call(T=4, H=64, Vr=1000, Vp=1024, r2=4096, r3=8192, n=4, dt=1, ids=A, E=B, E2=C, E3=A,
             out=B, i2=C, i3=A):
        return lib.vngram_fwd(ids, E, E2, E3, T, H, Vr, Vp, r2, r3, n, dt, out, i2, i3, NUL,
                              None)
    assert call(r2=0) == SHAPE
    assert call(r3=(1 << 31)) == SHAPE
    assert call(r2=4098) == SHARD            # not a multiple of num_shards
    assert call(n=3) == SHARD
    assert call(dt=5) == DTYPE
    assert call(E2=NUL) == NULL
    assert call(i3=NUL) == NULL
    assert call(H=20) == ALIGN
    assert call(E3=MIS) == ALIGN


def test_candidates_argument_errors():
    need = lib.vss_candidates_workspace_bytes(8, 100)
    assert need > 0
    args = lambda P=10, cap=10, ws=A, wsb=need, ign=-100: lib.vss_candidates(
        A, 8, 100, ign, B, P, C, cap, A, B, C, ws, wsb, None)
    assert args(P=0) == SHAPE
    assert args(cap=9) == SHAPE          # capacity below max(P, min(T, V))
    assert args(P=101, cap=101) == SHAPE  # more candidates than rows: they cannot be distinct
    assert args(ign=3) == SHAPE
    assert args(wsb=need - 1) == WORKSPACE
    assert args(ws=NUL) == WORKSPACE


def test_scatter_argument_errors():
    args = lambda cand=A, P=10, src=B, H=64, V=100, dW=C, acc=0: lib.vss_scatter(
        cand, P, src, H, V, dW, acc, None)
    assert args(P=-1) == SHAPE
    assert args(V=0) == SHAPE
    assert args(H=0) == SHAPE
    assert args(acc=2) == DTYPE
    assert args(dW=NUL) == NULL
    assert args(cand=NUL) == NULL
    assert args(src=NUL) == NULL
    assert args(H=60) == ALIGN
    assert args(dW=MIS) == ALIGN
    assert args(src=MIS) == ALIGN


def test_scatter_replace_argument_errors():
    args = lambda prev=A, Pp=5, cand=A, P=10, src=B, H=64, V=100, dW=C: lib.vss_scatter_replace(
        prev, Pp, cand, P, src, H, V, dW, None)
    assert args(Pp=-1) == SHAPE
    assert args(P=-1) == SHAPE
    assert args(V=0) == SHAPE
    assert args(H=0) == SHAPE
    assert args(prev=NUL) == NULL
    assert args(dW=NUL) == NULL
    assert args(cand=NUL) == NULL
    assert args(src=NUL) == NULL
    assert args(H=60) == ALIGN
    assert args(dW=MIS) == ALIGN
    assert args(src=MIS) == ALIGN


def test_workspace_queries_are_deterministic_and_reject_bad_shapes():
    a = lib.vce_bwd_workspace_bytes(8192, 3072, 201088, 201088, 8, 1)
    b = lib.vce_bwd_workspace_bytes(8192, 3072, 201088, 201088, 8, 1)
    # one chunk of G (four shards: 100544 columns) is staged, never [T, V]; the dh
    # GEMM's 32 x 12 tiles fill 1.5 rounds of 256 CUs, so its K is split in two
    # and one float32 partial plane [T, H] is kept; the dW GEMM's 393 x 12 tiles
    # fill 18 rounds and 108 tiles: rows past 384 tiles (2240 of them) run as a
    # second launch with K split in two, and one plane of those rows is kept
    assert a == b == 8192 * 100544 * 2 + 8192 * 3072 * 4 + 2240 * 3072 * 4
    # one shard of 201088 rows: two tile-aligned pieces of 100608 rows (393
    # tiles, a tail of 2304 rows)
    assert lib.vce_bwd_workspace_bytes(8192, 3072, 201088, 201088, 1, 1) == \
        8192 * 100608 * 2 + 8192 * 3072 * 4 + 2304 * 3072 * 4
    # one shard's rows alone (25136): two pieces of 12800 rows; dW's 50 x 12
    # tiles: the first 42 tile rows fill two rounds, the last 8 (2048 rows)
    # run with K split in two
    assert lib.vce_bwd_workspace_bytes(8192, 3072, 25136, 25136, 1, 1) == \
        8192 * 12800 * 2 + 8192 * 3072 * 4 + 2048 * 3072 * 4
    # 16384 tokens: 64 x 12 dh tiles are three full rounds, no split; G and the
    # dW tail's plane
    assert lib.vce_bwd_workspace_bytes(16384, 3072, 201088, 201088, 8, 1) == \
        16384 * 100544 * 2 + 2240 * 3072 * 4
    # sampled-softmax shape (P = 16384 rows, H = 1536): chunks of 8192 rows; dh
    # (64 x 6 tiles) split in two; dW (32 x 6 tiles, K = 16384) not split: one
    # round of long tiles costs about what four short rounds plus three planes do
    assert lib.vce_bwd_workspace_bytes(16384, 1536, 16384, 16384, 1, 1) == \
        16384 * 8192 * 2 + 1 * 16384 * 1536 * 4
    # a table of two tiles or more is never staged whole
    for T, H, Vr, Vp, n in ((64, 64, 1000, 1024, 4), (2048, 1024, 50000, 50016, 8),
                            (300, 72, 1001, 1002, 1)):
        assert lib.vce_bwd_workspace_bytes(T, H, Vr, Vp, n, 1) < T * Vp * 2
    assert lib.vce_fwd_workspace_bytes(8, 64, 100, 101, 2, 1) == 0  # 101 % 2 != 0
    assert lib.vce_bwd_workspace_bytes(8, 64, 100, 128, 4, 3) == 0  # bad dtype


def test_bwd_event_count_and_timed_checks():
    # 8 shards of 25136 rows: two chunks of four shards
    assert lib.vce_bwd_event_count(16384, 3072, 201088, 201088, 8, 1) == 1 + 3 * 2
    # one shard of 201088 rows: two pieces
    assert lib.vce_bwd_event_count(16384, 3072, 201088, 201088, 1, 1) == 1 + 3 * 2
    # a table narrower than two tiles: one chunk
    assert lib.vce_bwd_event_count(8, 64, 300, 300, 3, 1) == 1 + 3 * 1
    assert lib.vce_bwd_event_count(8, 64, 100, 101, 2, 1) == 0      # 101 % 2 != 0
    ev = (ctypes.c_void_p * 3)()
    args = (A, B, C, A, C, A, 0, 4, 64, 1000, 1024, 4, -100, 1, A, B, 0, A, 1 << 40, None)
    # wrong event count is rejected before any HIP call
    assert lib.vce_bwd_timed(*args, ev, 3) == SHAPE


def test_bwd_accumulate_flags_checked():
    def call(acc):
        return lib.vce_bwd(A, B, C, A, C, A, 0, 4, 64, 1000, 1024, 4, -100, 1, A, B, acc, A, 0,
                           None)
    # unknown flag bits are rejected; known ones pass the flag check and stop at the
    # (deliberately missing) workspace
    assert call(4) == DTYPE and call(-1) == DTYPE
    for acc in (0, 1, 2, 3):
        assert call(acc) == WORKSPACE


def test_argmax_noalloc_argument_errors():
    """Checked before any HIP call: bad arguments as for vce_argmax, and a
    call whose per-tile reports would not fit the static scratch."""
    call = lambda T=4, H=64, Vr=1000, Vp=1024, n=4, dt=1, h=A, W=B, idx=C, val=A: \
        lib.vce_argmax_noalloc(h, W, T, H, Vr, Vp, n, dt, idx, val, NUL, NUL, None)
    assert call(dt=7) == DTYPE
    assert call(Vr=0) == SHAPE
    assert call(n=3) == SHARD
    assert call(h=NUL) == NULL
    assert call(H=60) == ALIGN
    need = lib.vce_argmax_workspace_bytes(2648, 3072, 201088, 201088, 8, 1)
    assert need > 16 << 20 >= lib.vce_argmax_workspace_bytes(2647, 3072, 201088, 201088, 8, 1)
    assert call(T=2648, H=3072, Vr=201088, Vp=201088, n=8) == WORKSPACE
    assert call(T=0) == OK
