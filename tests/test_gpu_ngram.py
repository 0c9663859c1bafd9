"""GPU parity of the hashed n-gram input embedding (vngram_fwd, and its backward
through vemb_bwd) against the float64 oracle on the same seeded inputs:
n-gram rows bit-exact; the summed rows equal to the exact sum rounded once to
the table type (a float32 intermediate may round first: at most one unit in
the last place apart, rarely); the backward within the bf16 gradient
tolerance, rows no n-gram touches exactly zero."""

import sys

import numpy as np
import pytest

import oracle
from synth import make_tied_inputs
from tests._cmp import rel_l2

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


def _round_bf16_bits(x64):
    """float64 -> bf16 bits, round to nearest-even (exact sums of three bf16
    values fit float64, so this is one rounding of the exact sum)."""
    f = x64.astype(np.float32)               # exact for these sums in practice
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _tables(rng, rows, H, dt):
    x = (rng.standard_normal((rows, H)) * 0.02).astype(np.float32)
    if dt == "bf16":
        from synth import bf16_bits_from_f32
        return bf16_bits_from_f32(x)
    return x


@pytest.mark.parametrize("dt,T,H,Vr,Vp,r2,r3,n", [
    ("bf16", 2048, 256, 8000, 8192, 40000, 60000, 8),
    ("f32", 300, 64, 1000, 1024, 4096, 8192, 4),
    ("bf16", 1, 8, 10, 16, 8, 8, 2),
])
def test_ngram_parity(V, dt, T, H, Vr, Vp, r2, r3, n):
    say(f"case ngram {dt} T={T} H={H} V={Vr}/{Vp} rows={r2},{r3} n={n}")
    inp = make_tied_inputs(T, H, Vr, Vp, n, dt, seed=T + r2)
    rng = np.random.default_rng(T)
    E2b, E3b = _tables(rng, r2, H, dt), _tables(rng, r3, H, dt)
    Wb = inp.W.copy()
    Wb[Vr:] = 0x7FC0 if dt == "bf16" else np.float32("nan")   # padded rows: NaN, never read
    dev = "cuda"
    ids = torch.from_numpy(inp.ids).to(dev)
    E, E2, E3 = (V.from_bits(a, dt, dev) for a in (Wb, E2b, E3b))
    r = V.vngram_fwd(ids, E, E2, E3, Vr, n)
    torch.cuda.synchronize()
    x64, i2, i3 = oracle.ngram_embed(inp.ids, oracle.decode(Wb, dt), oracle.decode(E2b, dt),
                                     oracle.decode(E3b, dt), Vr)
    assert np.array_equal(r.ids2.cpu().numpy(), i2.astype(np.int32))
    assert np.array_equal(r.ids3.cpu().numpy(), i3.astype(np.int32))
    assert int(r.n_bad.item()) == int(((inp.ids < 0) | (inp.ids >= Vr)).sum())
    got = r.out.cpu()
    if dt == "bf16":
        gb = got.view(torch.int16).numpy().view(np.uint16).astype(np.int64)
        wb = _round_bf16_bits(x64).astype(np.int64)
        ulp = np.abs(gb - wb)
        assert ulp.max() <= 1, ulp.max()
        assert (ulp > 0).mean() <= 1e-3
    else:
        g = got.numpy().astype(np.float64)
        assert np.abs(g - x64).max() <= 1e-6 * max(1.0, np.abs(x64).max())
    assert not np.isnan(got.float().numpy()).any()
    # backward: scatter of a seeded dx into the three tables
    dx = rng.standard_normal((T, H)).astype(np.float32)
    dE, dE2, dE3 = V.ngram_bwd(ids, r, torch.from_numpy(dx).to(dev), Vr, Vp, n, rows2=r2,
                               rows3=r3)
    rE, rE2, rE3 = oracle.ngram_backward(inp.ids, dx.astype(np.float64), Vr, Vp, r2, r3)
    for name, g, w in (("dE", dE, rE), ("dE2", dE2, rE2), ("dE3", dE3, rE3)):
        g = g.cpu().numpy()
        assert rel_l2(g, w) <= 1e-6, name
        assert not g[~w.any(axis=1)].any(), name


@pytest.mark.slow
def test_ngram_full_size(V):
    """At the tied-step shapes (T=16384 Zipf tokens with out-of-range IDs,
    H=3072, the 201088-row table, 8 shards) with two 65536-row n-gram tables:
    every n-gram row bit-exact, sampled output rows against the oracle, and
    sampled rows of the n-gram tables' gradients against direct sums."""
    from synth import config_inputs
    say("case ngram full size")
    inp = config_inputs("c4")
    T, H, Vr, n = inp.T, inp.H, inp.V_real, inp.num_shards
    r2 = r3 = 65536
    rng = np.random.default_rng(99)
    E2b, E3b = _tables(rng, r2, H, "bf16"), _tables(rng, r3, H, "bf16")
    dev = "cuda"
    ids = torch.from_numpy(inp.ids).to(dev)
    E, E2, E3 = (V.from_bits(a, "bf16", dev) for a in (inp.W, E2b, E3b))
    r = V.vngram_fwd(ids, E, E2, E3, Vr, n)
    torch.cuda.synchronize()
    i2, i3 = oracle.ngram_ids(inp.ids, Vr, r2, r3)
    assert np.array_equal(r.ids2.cpu().numpy(), i2.astype(np.int32))
    assert np.array_equal(r.ids3.cpu().numpy(), i3.astype(np.int32))
    sample = np.unique(np.concatenate([[0, 1, 2, T - 1], rng.choice(T, 60, replace=False)]))
    W64 = oracle.decode(inp.W, "bf16")
    x64 = oracle.gather_direct(inp.ids[sample], W64, Vr)
    x64 += oracle.gather_direct(i2[sample], oracle.decode(E2b, "bf16"), r2)
    x64 += oracle.gather_direct(i3[sample], oracle.decode(E3b, "bf16"), r3)
    gb = r.out[torch.from_numpy(sample).to(dev)].cpu().view(torch.int16).numpy()
    ulp = np.abs(gb.view(np.uint16).astype(np.int64) - _round_bf16_bits(x64).astype(np.int64))
    assert ulp.max() <= 1
    dx = torch.randn(T, H, device=dev, generator=torch.Generator(device=dev).manual_seed(5))
    dE, dE2, dE3 = V.ngram_bwd(ids, r, dx, Vr, inp.V_pad, n, rows2=r2, rows3=r3)
    torch.cuda.synchronize()
    dxh = dx.cpu().numpy().astype(np.float64)
    for rows_of, g in ((i2, dE2), (i3, dE3)):
        touched = np.unique(rows_of[rows_of >= 0])
        pick = rng.choice(touched, min(20, touched.size), replace=False)
        for row in pick:
            want = dxh[rows_of == row].sum(axis=0)
            got = g[int(row)].cpu().numpy().astype(np.float64)
            assert np.abs(got - want).max() <= 1e-4 * max(1.0, np.abs(want).max())
        untouched = np.setdiff1d(np.arange(rows_of.max() + 1), touched)[:50]
        assert not g[torch.from_numpy(untouched).to(dev)].any()
