"""GPU parity of explicit (uneven) shard layouts and mapped class ownership
(vce_fwd_ex, vce_argmax_ex, vemb_fwd_ex, vce_remap through the C ABI) against
the float64 oracle on the same seeded inputs.

Layouts cover an empty shard, a one-row shard, a shard wholly inside the
padding, V_pad not a multiple of the shard count, 100 and 128 shards of
random sizes, and the even layout written out (which must give the even
entry points' bits). Mapped ownership stores class c at physical row
row_of[c]; after remapping targets and IDs the results by class must be those
of the unmapped table. Tolerances are those of the other parity tests.
"""

import sys

import numpy as np
import pytest

import oracle
from oracle.ce import MEAN
from synth import make_ce_inputs, make_layout, make_row_map
from tests._cmp import TOL, check_argmax, check_ce, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_embedding_softmax_amd as v
    return v


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


LAYOUTS = [
    # name, T, H, V_real, V_pad, rows (None: drawn by make_layout(V_pad, n, seed, empty, single)), dtype
    ("empty-shard", 300, 72, 990, 1000, [0, 100, 100, 601, 1000], "bf16"),
    ("one-row", 257, 64, 2500, 2560, [0, 1, 257, 1000, 2400, 2560], "f32"),
    ("pad-shard", 129, 64, 900, 1024, [0, 512, 900, 1024], "bf16"),
    ("n100", 513, 136, 5000, 5000, (100, 3, 10, 5), "bf16"),
    ("n128", 100, 64, 4000, 4096, (128, 4, 20, 20), "f32"),
    ("n1", 64, 64, 1000, 1024, [0, 1024], "bf16"),
]


def _layout(Vp, rows):
    if isinstance(rows, tuple):
        n, seed, empty, single = rows
        return make_layout(Vp, n, seed, empty, single)
    return np.asarray(rows, dtype=np.int64)


def _inputs(T, H, Vr, Vp, rows, dt, seed):
    inp = make_ce_inputs(T, H, Vr, Vp, 1, dt, seed=seed, ignore_frac=0.1,
                         pad_fill=float("nan"))
    # targets on every shard's first and last real row, and one bad target
    edge = []
    for lo, hi in zip(rows[:-1], rows[1:]):
        hi = min(hi, Vr)
        if hi > lo:
            edge += [lo, hi - 1]
    k = min(len(edge), T - 1)
    inp.targets[:k] = np.asarray(edge[:k], dtype=np.int32)
    inp.targets[T - 1] = Vr + 3
    return inp


def _gpu_ce(V, inp, rows, n_even=None, W_bits=None, targets=None):
    dev = "cuda"
    h = V.from_bits(inp.h, inp.dtype, dev)
    W = V.from_bits(inp.W if W_bits is None else W_bits, inp.dtype, dev)
    tg = torch.from_numpy(inp.targets if targets is None else targets).to(dev)
    if n_even is None:
        n = len(rows) - 1
        f = V.vce_fwd(h, W, tg, inp.V_real, n, inp.ignore_index, shard_stats=True, allow_bad=True,
                      shard_rows=[int(x) for x in rows])
    else:
        f = V.vce_fwd(h, W, tg, inp.V_real, n_even, inp.ignore_index, shard_stats=True,
                      allow_bad=True)
    gl = torch.ones(1, dtype=torch.float32, device=dev)
    b = V.vce_bwd(h, W, tg, f.lse, gl, f.n_valid, inp.V_real, 1, inp.ignore_index, MEAN)
    torch.cuda.synchronize()
    return dict(lse=f.lse.cpu().numpy(), loss=f.loss.cpu().numpy(),
                loss_sum=float(f.loss_sum.item()), n_valid=int(f.n_valid.item()),
                n_bad=int(f.n_bad.item()), shard=f.shard_stats.cpu().numpy(),
                dh=b.dh.cpu().numpy(), dW=b.dW.cpu().numpy())


@pytest.mark.parametrize("name,T,H,Vr,Vp,rows,dt", LAYOUTS, ids=[x[0] for x in LAYOUTS])
def test_uneven_ce_parity(V, name, T, H, Vr, Vp, rows, dt):
    rows = _layout(Vp, rows)
    say(f"case uneven ce {name} T={T} H={H} V={Vr}/{Vp} n={len(rows) - 1} {dt}")
    inp = _inputs(T, H, Vr, Vp, rows, dt, seed=T + 11 * H)
    g = _gpu_ce(V, inp, rows)
    h64 = oracle.decode(inp.h, dt)
    W64 = oracle.decode(inp.W, dt)
    ref = oracle.cross_entropy(h64, W64, inp.targets, Vr, Vp, len(rows) - 1, inp.ignore_index,
                               1.0, MEAN, shard_rows=rows)
    check_ce(g, ref, dt, Vr)
    m, s = g["shard"][0], g["shard"][1]
    empty = np.isneginf(ref["shard_m"])
    # a shard with no real row reports exactly (-inf, 0)
    assert np.isneginf(m[empty]).all() and not s[empty].any(), name
    m_tol = 1e-3 if dt == "bf16" else 1e-5
    s_tol = 2e-3 if dt == "bf16" else 1e-5
    assert np.abs(m[~empty] - ref["shard_m"][~empty]).max(initial=0.0) < m_tol, name
    assert np.allclose(s[~empty], ref["shard_s"][~empty], rtol=s_tol), name


def test_even_layout_written_out_is_bitwise_the_even_call(V):
    say("case even layout via _ex")
    T, H, Vr, Vp, n = 300, 64, 1000, 1024, 4
    rows = np.arange(n + 1, dtype=np.int64) * (Vp // n)
    inp = _inputs(T, H, Vr, Vp, rows, "bf16", seed=5)
    a = _gpu_ce(V, inp, rows)
    b = _gpu_ce(V, inp, rows, n_even=n)
    for k in ("lse", "loss", "shard", "dh", "dW"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    assert a["loss_sum"] == b["loss_sum"]


@pytest.mark.parametrize("name,T,H,Vr,Vp,rows,dt", LAYOUTS, ids=[x[0] for x in LAYOUTS])
def test_uneven_argmax_parity(V, name, T, H, Vr, Vp, rows, dt):
    rows = _layout(Vp, rows)
    n = len(rows) - 1
    say(f"case uneven argmax {name} n={n}")
    inp = _inputs(T, H, Vr, Vp, rows, dt, seed=T + 13 * H)
    dev = "cuda"
    h = V.from_bits(inp.h, dt, dev)
    W = V.from_bits(inp.W, dt, dev)
    r = V.vce_argmax(h, W, Vr, n, shard_reports=True, shard_rows=[int(x) for x in rows])
    one = V.vce_argmax(h, W, Vr, 1)
    torch.cuda.synchronize()
    idx = r.index.cpu().numpy().astype(np.int64)
    val = r.value.cpu().numpy().astype(np.float64)
    sv = r.shard_value.cpu().numpy().astype(np.float64)
    si = r.shard_index.cpu().numpy().astype(np.int64)
    h64 = oracle.decode(inp.h, dt)
    W64 = oracle.decode(inp.W, dt)
    check_argmax(idx, val, h64, W64, Vr, name)
    for k, (lo, hi) in enumerate(zip(rows[:-1], rows[1:])):
        hi = min(hi, Vr)
        if hi <= lo:
            assert (si[k] == -1).all() and np.isneginf(sv[k]).all(), (name, k)
            continue
        check_argmax(si[k] - lo, sv[k], h64, W64[lo:hi], hi - lo, f"{name} shard {k}")
    # every logit is computed the same way whatever the layout
    assert np.array_equal(idx, one.index.cpu().numpy()), name
    assert np.array_equal(r.value.cpu().numpy(), one.value.cpu().numpy()), name
    ref = oracle.greedy_argmax(h64, W64, Vr, Vp, n, shard_rows=rows)
    assert np.array_equal(np.isneginf(ref["shard_value"]), np.isneginf(sv)), name


@pytest.mark.parametrize("name,T,H,Vr,Vp,rows,dt", LAYOUTS, ids=[x[0] for x in LAYOUTS])
def test_uneven_gather_bit_exact(V, name, T, H, Vr, Vp, rows, dt):
    rows = _layout(Vp, rows)
    n = len(rows) - 1
    say(f"case uneven gather {name} n={n}")
    inp = make_ce_inputs(T, H, Vr, Vp, 1, dt, seed=T + 17, id_dist="uniform",
                         pad_fill=float("nan"))
    edge = [-1, Vr, Vp - 1, Vp, -(2**31), 2**31 - 1]
    for lo, hi in zip(rows[:-1], rows[1:]):
        edge += [lo, hi - 1, hi]
    ids = np.concatenate([inp.ids, np.asarray(edge, dtype=np.int64)])
    ids = np.clip(ids, -(2**31), 2**31 - 1).astype(np.int32)
    dev = "cuda"
    W = V.from_bits(inp.W, dt, dev)
    out, nbad = V.vemb_fwd(torch.from_numpy(ids).to(dev), W, Vr, n,
                           shard_rows=[int(x) for x in rows])
    torch.cuda.synchronize()
    a = out.cpu()
    got = (a.view(torch.int16) if dt == "bf16" else a.view(torch.int32)).numpy()
    Wb = inp.W.view(np.int16) if dt == "bf16" else inp.W.view(np.int32)
    ok = (ids >= 0) & (ids < Vr)
    want = np.zeros_like(got)
    want[ok] = Wb[ids[ok]]
    assert np.array_equal(got, want), name
    assert int(nbad.item()) == int((~ok).sum())
    ms = oracle.gather_masked_shards(ids, oracle.decode(inp.W, dt), Vr, Vp, n, shard_rows=rows)
    dec = oracle.decode(got.view(np.uint16) if dt == "bf16" else got.view(np.float32), dt)
    assert np.array_equal(dec, ms), name


def test_zero_tokens_uneven(V):
    dev = "cuda"
    rows = [0, 10, 10, 128]
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(128, 64, dtype=torch.bfloat16, device=dev)
    tg = torch.empty(0, dtype=torch.int32, device=dev)
    f = V.vce_fwd(h, W, tg, 100, 3, shard_rows=rows)
    r = V.vce_argmax(h, W, 100, 3, shard_rows=rows)
    o, nb = V.vemb_fwd(tg, W, 100, 3, shard_rows=rows)
    torch.cuda.synchronize()
    assert int(f.n_valid.item()) == 0 and float(f.loss_sum.item()) == 0.0
    assert r.index.numel() == 0 and o.numel() == 0 and int(nb.item()) == 0


# ------------------------------------------------------------------ mapped ownership

@pytest.mark.parametrize("dt,rows", [("bf16", None), ("f32", [0, 300, 300, 701, 1024])])
def test_mapped_ownership_is_a_relabelling(V, dt, rows):
    T, H, Vr, Vp = 300, 64, 1000, 1024
    say(f"case mapped ownership {dt} rows={rows}")
    inp = make_ce_inputs(T, H, Vr, Vp, 4, dt, seed=23, ignore_frac=0.1, id_dist="uniform")
    inp.targets[:3] = [Vr + 3, -7, Vr - 1]
    inp.ids[:3] = [Vr, -1, 0]
    row_of = make_row_map(Vr, seed=29)
    inv = np.empty(Vr, dtype=np.int64)
    inv[row_of] = np.arange(Vr)
    Wp = inp.W.copy()
    Wp[row_of] = inp.W[:Vr]                   # class c stored at physical row row_of[c]
    dev = "cuda"
    m = torch.from_numpy(row_of).to(dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    ids = torch.from_numpy(inp.ids).to(dev)
    tg_p = V.vce_remap(tg, m)
    ids_p = ids.clone()
    V.vce_remap(ids_p, m, out=ids_p)          # in place
    torch.cuda.synchronize()
    for src, got in ((inp.targets, tg_p), (inp.ids, ids_p)):
        assert np.array_equal(got.cpu().numpy(), oracle.remap(src, row_of, Vr)), dt
    tgp = tg_p.cpu().numpy()

    n = 4 if rows is None else len(rows) - 1
    lay = None if rows is None else np.asarray(rows, dtype=np.int64)
    if lay is None:
        g = _gpu_ce(V, inp, None, n_even=4, W_bits=Wp, targets=tgp)
    else:
        g = _gpu_ce(V, inp, lay, W_bits=Wp, targets=tgp)
    h64 = oracle.decode(inp.h, dt)
    ref = oracle.cross_entropy(h64, oracle.decode(inp.W, dt), inp.targets, Vr, Vp, 4,
                               inp.ignore_index, 1.0, MEAN)
    # per-token loss and lse by class; gradients of class c live at row row_of[c]
    g_cls = dict(g)
    dW_cls = g["dW"].copy()
    dW_cls[:Vr] = g["dW"][row_of]
    g_cls["dW"] = dW_cls
    check_ce(g_cls, ref, dt, Vr)
    tol = TOL[dt]["grad"]
    assert rel_l2(g["loss"], ref["loss"]) <= tol

    # argmax: the physical row maps back to the class
    hd = V.from_bits(inp.h, dt, dev)
    r = V.vce_argmax(hd, V.from_bits(Wp, dt, dev), Vr, n,
                     shard_rows=None if lay is None else [int(x) for x in lay])
    torch.cuda.synchronize()
    cls = inv[r.index.cpu().numpy().astype(np.int64)]
    check_argmax(cls, r.value.cpu().numpy().astype(np.float64), h64,
                 oracle.decode(inp.W, dt), Vr, "mapped argmax")

    # lookups: remapped IDs on the physical table give the unmapped rows' bits
    a, _ = V.vemb_fwd(ids_p, V.from_bits(Wp, dt, dev), Vr, n,
                      shard_rows=None if lay is None else [int(x) for x in lay])
    b, _ = V.vemb_fwd(ids, V.from_bits(inp.W, dt, dev), Vr, 4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if dt == "bf16" else a.view(torch.int32),
                       b.view(torch.int16) if dt == "bf16" else b.view(torch.int32))
