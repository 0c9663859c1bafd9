"""GPU parity: libvce (through its C ABI) against the float64 oracle on the
same seeded inputs. Every test here needs an MI355X."""

import sys

import numpy as np
import pytest

import oracle
from oracle.ce import MEAN, SUM
from synth import config_inputs, make_ce_inputs, make_tied_inputs, make_sampled_inputs
from tests._cmp import TOL, check_ce, oracle_ce, rel_l2

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


def gpu_ce(V, inp, grad_loss=1.0, reduction=MEAN, num_shards=None, W_override=None):
    dev = "cuda"
    n = inp.num_shards if num_shards is None else num_shards
    h = V.from_bits(inp.h, inp.dtype, dev)
    W = V.from_bits(inp.W if W_override is None else W_override, inp.dtype, dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    gl = torch.tensor([grad_loss], dtype=torch.float32, device=dev)
    r = V.ce_step(h, W, tg, inp.V_real, n, inp.ignore_index, grad_loss=gl,
                  reduction=reduction, shard_stats=True, allow_bad=True)
    torch.cuda.synchronize()
    f = r.fwd
    return dict(lse=f.lse.cpu().numpy(), loss=f.loss.cpu().numpy(),
                loss_sum=float(f.loss_sum.item()), n_valid=int(f.n_valid.item()),
                n_bad=int(f.n_bad.item()), shard=f.shard_stats.cpu().numpy(),
                dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())


# ------------------------------------------------------------------ cross-entropy

def test_c1_ce_parity_fp32(V):
    say("case c1 fp32 ce")
    inp = config_inputs("c1")
    for red, gl in ((MEAN, 1.0), (SUM, 0.5)):
        g = gpu_ce(V, inp, gl, red)
        ref = oracle_ce(inp, gl, red)
        check_ce(g, ref, "f32", inp.V_real)
        # per-shard statistics: what each emulated rank holds before the merge
        m, s = g["shard"][0], g["shard"][1]
        assert np.allclose(m, ref["shard_m"], rtol=1e-5, atol=1e-6)
        assert np.allclose(s, ref["shard_s"], rtol=1e-5, atol=1e-6)


def test_c2_ce_parity_bf16_garbage_pad_rows(V):
    say("case c2 bf16 ce")
    inp = config_inputs("c2")
    g = gpu_ce(V, inp)
    ref = oracle_ce(inp)
    check_ce(g, ref, "bf16", inp.V_real)
    m, s = g["shard"][0], g["shard"][1]
    assert np.abs(m - ref["shard_m"]).max() < 1e-3
    assert np.allclose(s, ref["shard_s"], rtol=2e-3)


def test_c2_pad_rows_do_not_change_any_bit(V):
    say("case c2 pad rows +8 vs NaN vs 0")
    inp = config_inputs("c2", T=512)
    base = gpu_ce(V, inp)
    for fill in (0x7FC0, 0x0000, 0xFF80):  # NaN, +0, -inf
        W2 = inp.W.copy()
        W2[inp.V_real:] = fill
        g = gpu_ce(V, inp, W_override=W2)
        for k in ("lse", "loss", "dh", "dW", "shard"):
            assert np.array_equal(g[k].view(np.uint32), base[k].view(np.uint32)), k
        assert g["loss_sum"] == base["loss_sum"]


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_num_shards_invariance(V, n):
    say(f"case c2-recipe T=384 shards={n}")
    inp = config_inputs("c2", T=384)
    g = gpu_ce(V, inp, num_shards=n)
    ref = oracle_ce(inp, num_shards=n)
    check_ce(g, ref, "bf16", inp.V_real)
    assert np.abs(g["lse"] - ref["lse"]).max() < 1e-4


RAGGED = [
    # T, H, V_real, V_pad, n, dtype
    (1, 8, 1, 8, 8, "f32"),
    (5, 8, 13, 16, 4, "bf16"),
    (300, 72, 1001, 1002, 2, "bf16"),    # V_pad not a multiple of 8, H not of 64
    (257, 64, 777, 800, 5, "f32"),
    (513, 136, 2500, 2560, 10, "bf16"),
    (64, 64, 1000, 1024, 4, "bf16"),
    (40, 1024, 300, 300, 3, "f32"),
    # dh's K split in four in the first vocabulary chunk, not at all in the
    # second (few real classes): the second chunk's result lands in dh while
    # the first chunk's planes wait for the one addition after it
    (512, 256, 4200, 8192, 2, "bf16"),
    (300, 128, 6000, 8192, 2, "f32"),
    # several tiles and 64-K slices in every GEMM, each with a partial last
    # one: K tails of 8 (H) and 9 or 12 (T, dW's K) on the 16x16x32 blocks
    (777, 200, 3000, 3008, 4, "bf16"),
    (1100, 520, 9000, 9024, 3, "bf16"),
]


@pytest.mark.parametrize("T,H,Vr,Vp,n,dt", RAGGED)
def test_ragged_shapes(V, T, H, Vr, Vp, n, dt):
    say(f"case ragged T={T} H={H} V_real={Vr} V_pad={Vp} n={n} {dt}")
    inp = make_ce_inputs(T, H, Vr, Vp, n, dt, seed=T * 7 + H, ignore_frac=0.1,
                         pad_fill=float("nan"))
    inp.targets[0] = Vr - 1
    if T > 2:
        inp.targets[1] = Vr + 1 if Vr + 1 < 2**31 else -5   # a bad target
    g = gpu_ce(V, inp)
    ref = oracle_ce(inp)
    check_ce(g, ref, dt, Vr)


@pytest.mark.parametrize("T,H,Vr,Vp,tail0,dt", [
    # one shard of 33792 rows in two chunks of 16896 (66 x 4 dW tiles over
    # K = 2048 tokens: one round of 256 and 8 more): rows past 64 tiles run as
    # a second launch with K split in two; the second chunk's tail holds the
    # last 212 real classes and all 300 padding rows
    (2048, 1024, 33492, 33792, 16384, "bf16"),
    (2048, 1024, 33492, 33792, 16384, "f32"),
    # two chunks of 25600 rows (100 x 3 tiles over K = 4096): the first 85
    # tile rows fill one round but one CU, the last 15 (3840 rows) run with K
    # split in four; 200 padding rows at the end
    (4096, 768, 51000, 51200, 21760, "bf16"),
])
def test_dw_tail_split(V, T, H, Vr, Vp, tail0, dt):
    say(f"case dW tail split T={T} H={H} V_real={Vr} V_pad={Vp} {dt}")
    inp = make_ce_inputs(T, H, Vr, Vp, 1, dt, seed=4242 + H, ignore_frac=0.05,
                         pad_fill=float("nan"))
    inp.targets[:64] = np.arange(Vr - 64, Vr)            # targets in the padded tail
    inp.targets[64:128] = np.arange(tail0, tail0 + 64)   # and in the first chunk's tail
    g = gpu_ce(V, inp)
    ref = oracle_ce(inp)
    check_ce(g, ref, dt, Vr)
    # accumulating adds the same result (split 0 into dW, split 1 through its
    # plane) and leaves the padding rows alone
    dev = "cuda"
    h = V.from_bits(inp.h, inp.dtype, dev)
    W = V.from_bits(inp.W, inp.dtype, dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    gl = torch.ones(1, dtype=torch.float32, device=dev)
    f = V.vce_fwd(h, W, tg, Vr, 1, inp.ignore_index, allow_bad=True)
    dW = torch.from_numpy(g["dW"]).to(dev)
    dW[Vr:] = 7.0
    V.vce_bwd(h, W, tg, f.lse, gl, f.n_valid, Vr, 1, inp.ignore_index, V.REDUCE_MEAN, dW=dW,
              accumulate_dW=True)
    torch.cuda.synchronize()
    d2 = dW.cpu().numpy()
    assert rel_l2(d2[:Vr], 2.0 * g["dW"][:Vr].astype(np.float64)) <= 1e-6
    assert (d2[Vr:] == 7.0).all()


def test_zero_tokens(V):
    say("case T=0")
    inp = make_ce_inputs(0, 64, 100, 128, 2, "bf16", seed=1)
    dev = "cuda"
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    W = V.from_bits(inp.W, "bf16", dev)
    tg = torch.empty(0, dtype=torch.int32, device=dev)
    dW = torch.full((128, 64), 7.0, device=dev)
    r = V.ce_step(h, W, tg, 100, 2, dW=dW)
    torch.cuda.synchronize()
    assert r.fwd.loss_sum.item() == 0.0 and r.fwd.n_valid.item() == 0
    assert not r.dW.any()


def test_all_targets_ignored(V):
    say("case all ignored")
    inp = make_ce_inputs(70, 64, 500, 512, 4, "bf16", seed=3)
    inp.targets[:] = -100
    g = gpu_ce(V, inp)
    assert g["n_valid"] == 0 and g["loss_sum"] == 0.0
    assert not g["dh"].any() and not g["dW"].any()
    ref = oracle_ce(inp)
    assert np.abs(g["lse"] - ref["lse"]).max() < 1e-2


def test_rerun_is_bitwise_identical(V):
    say("case determinism c2 T=1024")
    inp = config_inputs("c2", T=1024)
    a = gpu_ce(V, inp)
    b = gpu_ce(V, inp)
    for k in ("lse", "loss", "dh", "dW"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    assert a["loss_sum"] == b["loss_sum"]


# ------------------------------------------------------------------ embedding

def _bits(t):
    a = t.cpu()
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16).numpy()
    return a.view(torch.int32).numpy()


@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_embedding_gather_bit_exact(V, cfg):
    say(f"case gather {cfg}")
    inp = config_inputs(cfg)
    dev = "cuda"
    edge = np.array([-1, inp.V_real, inp.V_pad - 1, inp.V_pad, -(2**31), 2**31 - 1, 0,
                     inp.V_real - 1, inp.S - 1, inp.S], dtype=np.int32)
    ids = np.concatenate([inp.ids, edge]).astype(np.int32)
    W = V.from_bits(inp.W, inp.dtype, dev)
    out, nbad = V.vemb_fwd(torch.from_numpy(ids).to(dev), W, inp.V_real, inp.num_shards)
    torch.cuda.synchronize()
    got = _bits(out)
    Wb = inp.W.view(np.int16) if inp.dtype == "bf16" else inp.W.view(np.int32)
    ok = (ids >= 0) & (ids < inp.V_real)
    want = np.zeros_like(got)
    want[ok] = Wb[ids[ok]]
    assert np.array_equal(got, want)
    assert int(nbad.item()) == int((~ok).sum())
    # and the masked per-shard sum (the sharded form) agrees in value
    Wf = oracle.decode(inp.W, inp.dtype)
    ms = oracle.gather_masked_shards(ids, Wf, inp.V_real, inp.V_pad, inp.num_shards)
    assert np.array_equal(oracle.decode(got.view(np.uint16) if inp.dtype == "bf16" else
                                        got.view(np.float32), inp.dtype), ms)


def _dout(T, H, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    if dtype == "bf16":
        from synth import bf16_bits_from_f32
        return bf16_bits_from_f32(x)
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_scatter_add_parity(V, cfg, dtype):
    say(f"case scatter {cfg} dout={dtype}")
    inp = config_inputs(cfg)
    dev = "cuda"
    T, H = inp.ids.shape[0], inp.H
    dout = _dout(T, H, 5, dtype)
    ids_t = torch.from_numpy(inp.ids).to(dev)
    d = V.from_bits(dout, dtype, dev)
    ref, count = oracle.scatter_add(inp.ids, oracle.decode(dout, dtype), inp.V_real, inp.V_pad)
    # overwrite mode
    got = V.vemb_bwd(ids_t, d, inp.V_real, inp.V_pad, inp.num_shards).cpu().numpy()
    torch.cuda.synchronize()
    assert rel_l2(got, ref) <= 1e-6
    assert not got[count == 0].any()
    once = count == 1
    assert np.array_equal(got[once], ref[once].astype(np.float32))
    # accumulate mode adds into the rows the IDs touch and leaves the others
    base = np.random.default_rng(1).standard_normal((inp.V_pad, H)).astype(np.float32)
    dW = torch.from_numpy(base).to(dev)
    V.vemb_bwd(ids_t, d, inp.V_real, inp.V_pad, inp.num_shards, dW=dW, accumulate=True)
    got2 = dW.cpu().numpy()
    assert np.array_equal(got2[count == 0], base[count == 0])
    assert rel_l2(got2 - base, ref) <= 1e-5


def test_scatter_add_heavy_repeats(V):
    say("case scatter heavy repeats")
    dev = "cuda"
    rng = np.random.default_rng(3)
    T, H, Vr = 5000, 264, 300
    ids = np.where(rng.random(T) < 0.6, 7, rng.integers(-5, Vr + 5, T)).astype(np.int32)
    dout = rng.standard_normal((T, H)).astype(np.float32)
    ref, count = oracle.scatter_add(ids, dout, Vr, Vr)
    got = V.vemb_bwd(torch.from_numpy(ids).to(dev), torch.from_numpy(dout).to(dev), Vr, Vr,
                     1).cpu().numpy()
    assert count[7] > 2500
    assert rel_l2(got, ref) <= 1e-6
    # fixed summation order: a second run gives the same bits
    got_b = V.vemb_bwd(torch.from_numpy(ids).to(dev), torch.from_numpy(dout).to(dev), Vr, Vr,
                       1).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), got_b.view(np.uint32))


@pytest.mark.parametrize("T,H,Vr,label", [
    (20000, 64, 3000, "20 sorted runs, the last one partial"),
    (4000, 72, (1 << 20) + 5, "IDs of 21 bits (four radix passes)"),
    (16384, 40, 262143, "16 runs, 18-bit IDs"),
    (32768, 16, 70000, "32 runs, the most the merge holds"),
    (40000, 16, 3000, "T above the sorted runs: block sorts and ID scans"),
    (1, 8, 10, "one token"),
    (777, 8, 5, "five IDs, long runs over many chunks"),
])
def test_scatter_add_sort_paths(V, T, H, Vr, label):
    """Both ways the library sorts tokens by ID (sorted runs + merge, or
    block-local sorts + ID scans) against the oracle, with repeats that cross
    chunk ends and runs."""
    say(f"case scatter sort path T={T} H={H} V={Vr}: {label}")
    dev = "cuda"
    rng = np.random.default_rng(T + H)
    ids = rng.integers(0, Vr, T)
    rep = rng.random(T) < 0.5
    ids[rep] = rng.integers(0, min(Vr, 4), rep.sum())        # heavy repeats of a few IDs
    ids[rng.random(T) < 0.03] = -1                            # out of range
    if T > 2:
        ids[-1] = Vr - 1                                      # the largest ID
    ids = ids.astype(np.int32)
    dout = rng.standard_normal((T, H)).astype(np.float32)
    ref, count = oracle.scatter_add(ids, dout, Vr, Vr)
    got = V.vemb_bwd(torch.from_numpy(ids).to(dev), torch.from_numpy(dout).to(dev), Vr, Vr,
                     1).cpu().numpy()
    assert rel_l2(got, ref) <= 1e-6
    assert not got[count == 0].any()
    once = count == 1
    assert np.array_equal(got[once], ref[once].astype(np.float32))
    base = rng.standard_normal((Vr, H)).astype(np.float32)
    dW = torch.from_numpy(base).to(dev)
    V.vemb_bwd(torch.from_numpy(ids).to(dev), torch.from_numpy(dout).to(dev), Vr, Vr, 1,
               dW=dW, accumulate=True)
    got2 = dW.cpu().numpy()
    assert np.array_equal(got2[count == 0], base[count == 0])
    assert rel_l2(got2 - base, ref) <= 1e-5


# ------------------------------------------------------------------ tied step

def test_tied_step_small(V):
    say("case tied step T=1024 H=256 V=8192")
    inp = make_tied_inputs(1024, 256, 8000, 8192, 8, "bf16", seed=44)
    dev = "cuda"
    W = V.from_bits(inp.W, "bf16", dev)
    r = V.tied_step(torch.from_numpy(inp.ids).to(dev), torch.from_numpy(inp.targets).to(dev),
                    W, inp.V_real, inp.num_shards, allow_bad=True)
    torch.cuda.synchronize()
    ref = oracle.tied_step(inp.ids, inp.targets, oracle.decode(inp.W, "bf16"), inp.V_real,
                           inp.V_pad, inp.num_shards)
    h_bits = _bits(r.extra["h"])
    ok = (inp.ids >= 0) & (inp.ids < inp.V_real)
    want = np.zeros_like(h_bits)
    want[ok] = inp.W.view(np.int16)[inp.ids[ok]]
    assert np.array_equal(h_bits, want)
    assert int(r.extra["n_bad_id"].item()) == int((~ok).sum())
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             loss_sum=float(r.fwd.loss_sum.item()), n_valid=int(r.fwd.n_valid.item()),
             n_bad=int(r.fwd.n_bad.item()), dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())
    check_ce(g, ref, "bf16", inp.V_real)


@pytest.mark.parametrize("dt,T,H,Vr,Vp,n", [("f32", 64, 64, 1000, 1024, 4),
                                              ("bf16", 1024, 256, 8000, 8192, 8)])
def test_ot_h_step(V, dt, T, H, Vr, Vp, n):
    """Tied step plus the untied second head (two tokens ahead, weight 0.1):
    both losses, the summed dh, dW (head 1 + scatter of the summed dh) and dW2."""
    from synth import make_oth_inputs
    say(f"case OT-H step {dt} T={T} H={H} V={Vr}/{Vp} n={n}")
    inp, W2b, y2 = make_oth_inputs(T, H, Vr, Vp, n, dt, seed=T + 7)
    dev = "cuda"
    W = V.from_bits(inp.W, dt, dev)
    W2 = V.from_bits(W2b, dt, dev)
    r = V.ot_h_step(torch.from_numpy(inp.ids).to(dev), torch.from_numpy(inp.targets).to(dev),
                    torch.from_numpy(y2).to(dev), W, W2, Vr, n, allow_bad=True)
    torch.cuda.synchronize()
    ref = oracle.ot_h_step(inp.ids, inp.targets, y2, oracle.decode(inp.W, dt),
                           oracle.decode(W2b, dt), Vr, Vp, n)
    tol = TOL[dt]
    f1, f2 = r.fwd, r.extra["fwd2"]
    for f, rf in ((f1, ref["f1"]), (f2, ref["f2"])):
        assert int(f.n_valid.item()) == rf["n_valid"] and int(f.n_bad.item()) == rf["n_bad"]
        dl = abs(float(f.loss_sum.item()) - rf["loss_sum"]) / abs(rf["loss_sum"])
        assert dl <= tol["loss"], dl
        lse = f.lse.cpu().numpy().astype(np.float64)
        if tol["lse_abs"] is not None:
            assert np.abs(lse - rf["lse"]).max() <= tol["lse_abs"]
        else:
            assert (np.abs(lse - rf["lse"]) / np.abs(rf["lse"])).max() <= tol["lse_rel"]
    for name, got, want in (("dh", r.dh, ref["dh"]), ("dW", r.dW, ref["dW"]),
                            ("dW2", r.extra["dW2"], ref["dW2"])):
        e = rel_l2(got.cpu().numpy(), want)
        assert e <= tol["grad"], (name, e)
    assert not r.extra["dW2"][Vr:].cpu().numpy().any()
    # the second head's share of dh alone: run the first head only and compare
    r1 = V.tied_step(torch.from_numpy(inp.ids).to(dev), torch.from_numpy(inp.targets).to(dev),
                     W, Vr, n, allow_bad=True)
    d2 = (r.dh - r1.dh).cpu().numpy()
    want2 = ref["dh"] - oracle.tied_step(inp.ids, inp.targets, oracle.decode(inp.W, dt), Vr, Vp,
                                         n)["dh"]
    assert rel_l2(d2[:T - 1], want2[:T - 1]) <= 5 * tol["grad"]
    assert not d2[T - 1].any()


# ------------------------------------------------------------------ sampled softmax

@pytest.mark.parametrize("T,Vc,P", [
    (3000, 20000, 2048),      # one workgroup, bit maps in LDS
    (3000, 20001, 2048),      # a partial last word of the bit maps
    (500, 1000, 1000),        # P = V: every non-target row is a negative
    (3000, 20000, 256),       # more distinct targets than P: the candidates are U alone
    (3000, 300000, 256),      # the same on the several-launch path
    (3000, 300000, 4096),     # past the LDS bit maps: flags, scans and emits in several launches
    (20000, 262144, 16384),   # the largest one-workgroup table; negatives from two read blocks
    (3000, 262145, 4096),     # one row past it: the several-launch path
])
def test_candidates_bit_exact(V, T, Vc, P):
    say(f"case candidates T={T} V={Vc} P={P}")
    dev = "cuda"
    inp = make_sampled_inputs(T, 64, Vc, P, "bf16", seed=9, ignore_frac=0.03)
    inp.targets[5] = Vc + 5000  # out of range: keeps its value as position
    c = V.vss_candidates(torch.from_numpy(inp.targets).to(dev), inp.V_real,
                         torch.from_numpy(inp.perm).to(dev), inp.P)
    torch.cuda.synchronize()
    cand, pos, nu = oracle.candidates(inp.targets, inp.V_real, -100, inp.perm, inp.P)
    assert int(c.n_unique.item()) == nu
    assert int(c.n_cand.item()) == max(inp.P, nu)
    # with P above V only V - |U| negatives exist: the list holds those
    assert np.array_equal(c.cand.cpu().numpy()[:cand.shape[0]], cand.astype(np.int32))
    assert np.array_equal(c.pos.cpu().numpy(), pos.astype(np.int32))


def test_candidates_reject_more_than_the_table(V):
    dev = "cuda"
    tg = torch.zeros(8, dtype=torch.int32, device=dev)
    perm = torch.arange(100, dtype=torch.int32, device=dev)
    with pytest.raises(V.VceError):
        V.vss_candidates(tg, 100, perm, 101)


def test_sampled_step_more_distinct_targets_than_P(V):
    """|U| > P: the composite is sized by n_cand = |U| (the candidates are the
    distinct targets alone, no negatives); every valid target keeps its
    class, nothing is dropped as a bad target."""
    say("case sampled step T=2048 H=128 V=8192 P=256 (|U| > P)")
    dev = "cuda"
    inp = make_sampled_inputs(2048, 128, 8192, 256, "bf16", seed=31, zipf_s=0.6,
                              ignore_frac=0.02)
    h = V.from_bits(inp.h, "bf16", dev)
    W = V.from_bits(inp.W, "bf16", dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    perm = torch.from_numpy(inp.perm).to(dev)
    ref = oracle.sampled_step(oracle.decode(inp.h, "bf16"), oracle.decode(inp.W, "bf16"),
                              inp.targets, inp.perm, inp.P)
    assert ref["n_unique"] > inp.P
    ws = V.Workspaces(dev, cand=V.vss_candidates_workspace_bytes(2048, 8192),
                      fwd=V.vce_fwd_workspace_bytes(2048, 128, 256, 256, 1),
                      bwd=V.vce_bwd_workspace_bytes(2048, 128, 256, 256, 1))
    r = V.sampled_step(h, W, tg, perm, inp.P, ws=ws)
    torch.cuda.synchronize()
    n_cand = int(r.extra["n_cand"].item())
    assert n_cand == ref["n_unique"] == ref["cand"].shape[0]
    assert np.array_equal(r.extra["cand"].cpu().numpy()[:n_cand], ref["cand"].astype(np.int32))
    assert np.array_equal(r.extra["pos"].cpu().numpy(), ref["pos"].astype(np.int32))
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             loss_sum=float(r.fwd.loss_sum.item()), n_valid=int(r.fwd.n_valid.item()),
             n_bad=int(r.fwd.n_bad.item()), dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())
    assert g["n_bad"] == 0
    check_ce(g, ref, "bf16", inp.V_real)
    # sizing by P instead would drop the targets ranked past P: refused as bad targets
    with pytest.raises(V.BadTargetError):
        V.sampled_step(h, W, tg, perm, inp.P, n_cand=inp.P)


def test_bad_target_policy(V):
    """A target outside [0, V_real) other than ignore_index: the library
    counts it and treats it as ignored; the binding raises unless the caller
    allows it."""
    say("case bad-target policy")
    dev = "cuda"
    inp = make_ce_inputs(64, 64, 1000, 1024, 4, "f32", seed=3)
    inp.targets[7] = 1010      # a padded class
    inp.targets[9] = -7        # negative, not ignore_index
    h = V.from_bits(inp.h, "f32", dev)
    W = V.from_bits(inp.W, "f32", dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    with pytest.raises(V.BadTargetError) as e:
        V.ce_step(h, W, tg, inp.V_real, inp.num_shards, inp.ignore_index)
    assert e.value.n_bad == 2
    r = V.ce_step(h, W, tg, inp.V_real, inp.num_shards, inp.ignore_index, allow_bad=True)
    torch.cuda.synchronize()
    ref = oracle_ce(inp)
    assert int(r.fwd.n_bad.item()) == 2 and ref["n_bad"] == 2
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             loss_sum=float(r.fwd.loss_sum.item()), n_valid=int(r.fwd.n_valid.item()),
             n_bad=int(r.fwd.n_bad.item()), dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())
    check_ce(g, ref, "f32", inp.V_real)


@pytest.mark.parametrize("P,H,Vt,acc", [(0, 64, 50, 0), (1, 8, 3, 1), (777, 264, 5000, 0),
                                         (2000, 2056, 3000, 1), (4096, 1536, 40000, 0)])
def test_sampled_scatter_exact(V, P, H, Vt, acc):
    """vss_scatter against the oracle's scatter-add on distinct rows (some
    outside [0, V), which are skipped): a single contribution per row, so the
    result is exact (plus the old row when accumulating)."""
    say(f"case sampled scatter P={P} H={H} V={Vt} accumulate={acc}")
    dev = "cuda"
    rng = np.random.default_rng(P * 7 + H)
    cand = rng.permutation(Vt + 40)[:P].astype(np.int32) - 20  # distinct; some < 0 or >= V
    dWc = rng.standard_normal((P, H)).astype(np.float32)
    dW0 = rng.standard_normal((Vt, H)).astype(np.float32)
    dW = torch.from_numpy(dW0).to(dev)
    out = V.vss_scatter(torch.from_numpy(cand).to(dev), torch.from_numpy(dWc).to(dev), Vt, dW=dW,
                        accumulate=bool(acc))
    torch.cuda.synchronize()
    ref, _ = oracle.scatter_add(cand, dWc.astype(np.float64), Vt, Vt)
    if acc:
        ref = dW0.astype(np.float64) + ref
    np.testing.assert_array_equal(out.cpu().numpy(), ref.astype(np.float32))


def test_sampled_scatter_replace_keeps_only_the_last_rows(V):
    """vss_scatter_replace over a run of calls on one table (zeroed once):
    after each call the table equals the oracle's scatter of that call's rows
    into zeros, whatever rows the earlier calls wrote (overlapping sets,
    repeated and out-of-range entries in the previous list)."""
    say("case sampled scatter replace, four calls")
    dev = "cuda"
    rng = np.random.default_rng(77)
    Vt, H = 3000, 264
    dW = torch.zeros(Vt, H, dtype=torch.float32, device=dev)
    prev = None
    for k, P in enumerate([500, 1200, 0, 800]):
        cand = rng.permutation(Vt + 40)[:P].astype(np.int32) - 20  # distinct; some outside
        dWc = rng.standard_normal((P, H)).astype(np.float32)
        cand_t = torch.from_numpy(cand).to(dev)
        if prev is not None and prev.numel():
            prev = torch.cat([prev, prev[:3]])  # repeats are harmless
        V.vss_scatter_replace(prev, cand_t, torch.from_numpy(dWc).to(dev), dW)
        torch.cuda.synchronize()
        ref, _ = oracle.scatter_add(cand, dWc.astype(np.float64), Vt, Vt)
        np.testing.assert_array_equal(dW.cpu().numpy(), ref.astype(np.float32), err_msg=f"call {k}")
        prev = cand_t


def test_sampled_step_replace_is_bitwise_the_full_fill(V):
    """Consecutive sampled steps with different batches: the table kept across
    steps (only the previous step's rows cleared) holds the same bits as the
    whole-table fill of every step."""
    say("case sampled step replace vs full fill, three steps")
    dev = "cuda"
    Vt = 16384
    dW_keep = torch.zeros(Vt, 128, dtype=torch.float32, device=dev)
    rows = torch.empty(0, dtype=torch.int32, device=dev)
    for seed in (21, 22, 23):
        inp = make_sampled_inputs(1024, 128, Vt, 2048, "bf16", seed=seed)
        h = V.from_bits(inp.h, "bf16", dev)
        W = V.from_bits(inp.W, "bf16", dev)
        tg = torch.from_numpy(inp.targets).to(dev)
        pm = torch.from_numpy(inp.perm).to(dev)
        full = V.sampled_step(h, W, tg, pm, inp.P)
        kept = V.sampled_step(h, W, tg, pm, inp.P, dW=dW_keep, prev_rows=rows)
        torch.cuda.synchronize()
        assert torch.equal(full.dW.view(torch.int32), kept.dW.view(torch.int32)), seed
        rows = kept.extra["rows"]


def test_sampled_step_small(V):
    say("case sampled step T=1024 H=128 V=16384 P=2048")
    dev = "cuda"
    inp = make_sampled_inputs(1024, 128, 16384, 2048, "bf16", seed=12)
    h = V.from_bits(inp.h, "bf16", dev)
    W = V.from_bits(inp.W, "bf16", dev)
    r = V.sampled_step(h, W, torch.from_numpy(inp.targets).to(dev),
                       torch.from_numpy(inp.perm).to(dev), inp.P)
    torch.cuda.synchronize()
    ref = oracle.sampled_step(oracle.decode(inp.h, "bf16"), oracle.decode(inp.W, "bf16"),
                              inp.targets, inp.perm, inp.P)
    assert int(r.extra["n_cand"].item()) == inp.P
    assert np.array_equal(r.extra["cand"].cpu().numpy()[:inp.P], ref["cand"].astype(np.int32))
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             loss_sum=float(r.fwd.loss_sum.item()), n_valid=int(r.fwd.n_valid.item()),
             n_bad=int(r.fwd.n_bad.item()), dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())
    check_ce(g, ref, "bf16", inp.V_real)
