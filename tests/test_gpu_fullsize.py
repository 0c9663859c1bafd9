"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times. The large-vocabulary CE (T=8192), the tied step (T=16384), the
scatter-add and the sampled-softmax step are checked in full against the
float64 oracle (spread over the host's cores by oracle.parallel; about a
minute each). Only the T=65536 stress case is checked on sampled tokens
(every quantity of a sampled token computed one by one from its own logit
row) plus properties that hold at any size."""

import sys

import numpy as np
import pytest

import oracle
from oracle.ce import MEAN
from synth import config_inputs
from tests._cmp import TOL, check_dw_tiles, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

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


def _sample_tokens(targets, V_real, k, seed):
    rng = np.random.default_rng(seed)
    T = targets.shape[0]
    pick = set(rng.choice(T, size=k, replace=False).tolist())
    bad = np.nonzero((targets < 0) | (targets >= V_real))[0]
    pick.update(bad[:3].tolist())
    pick.update([0, T - 1])
    return np.array(sorted(pick))


def _check_sampled(g, inp, h64_rows, W64, sample, n_valid_all):
    """lse, loss and dh rows of the sampled tokens against the oracle."""
    y = inp.targets[sample]
    f = oracle.ce_forward(h64_rows, W64, y, inp.V_real, inp.V_pad, inp.num_shards,
                          inp.ignore_index)
    scale = 1.0 / max(n_valid_all, 1)
    dh, _ = oracle.ce_backward(h64_rows, W64, y, f["lse"], inp.V_real, inp.V_pad, scale,
                               inp.ignore_index)
    lse_err = np.abs(g["lse"][sample] - f["lse"]).max()
    assert lse_err <= TOL["bf16"]["lse_abs"], lse_err
    valid = f["valid"]
    # per token: the lse bound plus a relative term for the target logit
    lo = np.abs(g["loss"][sample][valid] - f["loss"][valid])
    assert (lo <= TOL["bf16"]["lse_abs"] + 1e-3 * np.abs(f["loss"][valid])).all(), lo.max()
    assert not g["loss"][sample][~valid].any()
    e = rel_l2(g["dh"][sample], dh)
    assert e <= TOL["bf16"]["grad"], e
    assert not g["dh"][sample][~valid].any()
    return f


def _counts(inp):
    v, ign, bad = oracle.target_status(inp.targets, inp.V_real, inp.ignore_index)
    return int(v.sum()), int(bad.sum())


def _check_full(g, ref, V_real, what):
    """Every token and every table row against the float64 oracle, at the
    bf16 tolerances ([VS] paragraph 4: the gradient is the probability minus
    the target indicator, times the loss scaling)."""
    tol = TOL["bf16"]
    assert g["n_valid"] == ref["n_valid"] and g["n_bad"] == ref["n_bad"]
    dl = abs(g["loss_sum"] - ref["loss_sum"]) / abs(ref["loss_sum"])
    lse_err = float(np.abs(g["lse"].astype(np.float64) - ref["lse"]).max())
    valid = ref["valid"]
    lo = np.abs(g["loss"][valid].astype(np.float64) - ref["loss"][valid])
    e_dh = rel_l2(g["dh"], ref["dh"])
    e_dw = rel_l2(g["dW"], ref["dW"])
    e_tile = check_dw_tiles(g["dW"][:V_real], ref["dW"][:V_real], "bf16", f"{what} dW")
    say(f"{what}: loss_sum rel {dl:.2e}, max|dlse| {lse_err:.2e} over {len(g['lse'])} tokens, "
        f"dh rel-L2 {e_dh:.2e}, dW rel-L2 {e_dw:.2e}, worst 256-row dW block {e_tile:.2e}")
    assert dl <= tol["loss"], dl
    assert lse_err <= tol["lse_abs"], lse_err
    assert (lo <= tol["lse_abs"] + 1e-3 * np.abs(ref["loss"][valid])).all(), lo.max()
    assert not g["loss"][~valid].any()
    assert e_dh <= tol["grad"], e_dh
    assert e_dw <= tol["grad"], e_dw
    assert not g["dh"][~valid].any(), "ignored tokens must get dh = 0"
    assert not g["dW"][V_real:].any(), "padded rows must get dW = 0"


@pytest.mark.timeout(600)
def test_c3_full_size(V):
    """The large-vocabulary workload (T=8192, H=3072, V=201088, 8 shards) in
    full: every token's lse and loss, the loss sum, the whole dh and dW, and
    every 256-row block of dW, against the float64 oracle over all tokens."""
    say("case c3 full size: GPU step")
    inp = config_inputs("c3")
    dev = "cuda"
    h = V.from_bits(inp.h, "bf16", dev)
    W = V.from_bits(inp.W, "bf16", dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    r = V.ce_step(h, W, tg, inp.V_real, inp.num_shards, inp.ignore_index, shard_stats=True)
    torch.cuda.synchronize()
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             loss_sum=float(r.fwd.loss_sum.item()), n_valid=int(r.fwd.n_valid.item()),
             n_bad=int(r.fwd.n_bad.item()), dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())
    # the per-shard statistics merge to the reported lse
    ss = r.fwd.shard_stats.cpu().numpy().astype(np.float64)
    assert np.abs(oracle.merge_shard_stats(ss[0], ss[1]) - g["lse"]).max() < 1e-4
    del r, h, W, tg
    torch.cuda.empty_cache()
    say(f"case c3: float64 oracle over all {inp.T} tokens on "
        f"{oracle.parallel.default_workers()} threads")
    ref = oracle.parallel.cross_entropy(oracle.decode(inp.h, "bf16"),
                                        oracle.decode(inp.W, "bf16"), inp.targets, inp.V_real,
                                        inp.V_pad, inp.num_shards, inp.ignore_index,
                                        progress=say)
    _check_full(g, ref, inp.V_real, "c3")


def test_max_tokens_sampled(V):
    """Four times c3's tokens (T = 65536) on the same table: the staged G chunk
    holds T x 100544 = 6.6e9 elements and the per-tile statistics 51e6 pairs,
    so any 32-bit element index in the backward would wrap."""
    say("case T=65536 (c3 recipe) full size")
    inp = config_inputs("c3", T=65536)
    dev = "cuda"
    h = V.from_bits(inp.h, "bf16", dev)
    W = V.from_bits(inp.W, "bf16", dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    r = V.ce_step(h, W, tg, inp.V_real, inp.num_shards, inp.ignore_index)
    torch.cuda.synchronize()
    nv, nb = _counts(inp)
    assert int(r.fwd.n_valid.item()) == nv and int(r.fwd.n_bad.item()) == nb
    dW = r.dW
    colsum = dW.double().sum(dim=0).abs().max().item()
    scale = dW.double().abs().sum(dim=0).max().item()
    assert colsum <= 1e-3 * scale, (colsum, scale)
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             dh=r.dh.cpu().numpy())
    del r, dW, h
    torch.cuda.empty_cache()
    sample = _sample_tokens(inp.targets, inp.V_real, 24, 5)
    sample = np.union1d(sample, [16383, 16384, 32767, 32768, 65535])
    W64 = oracle.decode(inp.W, "bf16")
    h64 = oracle.decode(inp.h[sample], "bf16")
    _check_sampled(g, inp, h64, W64, sample, nv)


@pytest.mark.timeout(600)
def test_c4_full_size_tied_step(V):
    """The tied step (T=16384, H=3072, V=201088, 8 shards) in full: the
    lookup bit for bit, the counts, every token's lse and loss, the whole dh,
    and the whole tied dW (CE rows + scatter of dh) with every 256-row block,
    against the float64 oracle's tied step over all tokens."""
    say("case c4 full size: GPU tied step")
    inp = config_inputs("c4")
    dev = "cuda"
    W = V.from_bits(inp.W, "bf16", dev)
    ids = torch.from_numpy(inp.ids).to(dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    r = V.tied_step(ids, tg, W, inp.V_real, inp.num_shards, inp.ignore_index)
    torch.cuda.synchronize()
    # the lookup, bit for bit, and its count of out-of-range IDs
    hb = r.extra["h"].cpu().view(torch.int16).numpy()
    ok = (inp.ids >= 0) & (inp.ids < inp.V_real)
    want = np.zeros_like(hb)
    want[ok] = inp.W.view(np.int16)[inp.ids[ok]]
    assert np.array_equal(hb, want)
    assert int(r.extra["n_bad_id"].item()) == int((~ok).sum())
    g = dict(lse=r.fwd.lse.cpu().numpy(), loss=r.fwd.loss.cpu().numpy(),
             loss_sum=float(r.fwd.loss_sum.item()), n_valid=int(r.fwd.n_valid.item()),
             n_bad=int(r.fwd.n_bad.item()), dh=r.dh.cpu().numpy(), dW=r.dW.cpu().numpy())
    del r, W, ids, tg
    torch.cuda.empty_cache()
    say(f"case c4: float64 oracle tied step over all {inp.T} tokens on "
        f"{oracle.parallel.default_workers()} threads")
    ref = oracle.parallel.tied_step(inp.ids, inp.targets, oracle.decode(inp.W, "bf16"),
                                    inp.V_real, inp.V_pad, inp.num_shards, inp.ignore_index,
                                    progress=say)
    _check_full(g, ref, inp.V_real, "c4")


def test_c4_full_size_scatter(V):
    say("case c4 scatter full size")
    inp = config_inputs("c4")
    dev = "cuda"
    rng = np.random.default_rng(40)
    dout = rng.standard_normal((inp.T, inp.H)).astype(np.float32)
    got = V.vemb_bwd(torch.from_numpy(inp.ids).to(dev), torch.from_numpy(dout).to(dev),
                     inp.V_real, inp.V_pad, inp.num_shards).cpu().numpy()
    ref, count = oracle.scatter_add(inp.ids, dout, inp.V_real, inp.V_pad)
    assert rel_l2(got, ref) <= 1e-5   # float32 sums of up to thousands of rows
    once = count == 1
    assert np.array_equal(got[once], ref[once].astype(np.float32))
    assert not got[count == 0].any()


def test_c5_full_size_sampled_softmax(V):
    say("case c5 full size")
    inp = config_inputs("c5")
    dev = "cuda"
    h = V.from_bits(inp.h, "bf16", dev)
    W = V.from_bits(inp.W, "bf16", dev)
    r = V.sampled_step(h, W, torch.from_numpy(inp.targets).to(dev),
                       torch.from_numpy(inp.perm).to(dev), inp.P)
    torch.cuda.synchronize()
    ref = oracle.sampled_step(oracle.decode(inp.h, "bf16"), oracle.decode(inp.W, "bf16"),
                              inp.targets, inp.perm, inp.P, chunk=1024)
    assert int(r.extra["n_unique"].item()) == ref["n_unique"]
    assert int(r.extra["n_cand"].item()) == inp.P
    assert np.array_equal(r.extra["cand"].cpu().numpy()[:inp.P], ref["cand"].astype(np.int32))
    assert np.array_equal(r.extra["pos"].cpu().numpy(), ref["pos"].astype(np.int32))
    assert int(r.fwd.n_valid.item()) == ref["n_valid"]
    dl = abs(float(r.fwd.loss_sum.item()) - ref["loss_sum"]) / abs(ref["loss_sum"])
    assert dl <= TOL["bf16"]["loss"], dl
    assert np.abs(r.fwd.lse.cpu().numpy() - ref["lse"]).max() <= TOL["bf16"]["lse_abs"]
    assert rel_l2(r.dh.cpu().numpy(), ref["dh"]) <= TOL["bf16"]["grad"]
    dWc = r.extra["dWc"].cpu().numpy()
    dW = r.dW.cpu().numpy()
    assert rel_l2(dWc, ref["dWc"]) <= TOL["bf16"]["grad"]
    assert rel_l2(dW, ref["dW"]) <= TOL["bf16"]["grad"]
    check_dw_tiles(dWc, ref["dWc"], "bf16", "c5 dWc")
    check_dw_tiles(dW, ref["dW"], "bf16", "c5 dW")


def test_c3_full_size_argmax_sampled_tokens(V):
    """Greedy argmax at the large-vocabulary shape (T=8192, H=3072, V=201088,
    8 shards), in the launch configuration the bench times; sampled tokens
    against the oracle, every token against properties of the merge."""
    from tests._cmp import check_argmax
    say("case c3 full-size argmax")
    inp = config_inputs("c3")
    dev = "cuda"
    h = V.from_bits(inp.h, inp.dtype, dev)
    W = V.from_bits(inp.W, inp.dtype, dev)
    r = V.vce_argmax(h, W, inp.V_real, inp.num_shards, shard_reports=True)
    torch.cuda.synchronize()
    idx = r.index.cpu().numpy().astype(np.int64)
    val = r.value.cpu().numpy().astype(np.float64)
    sv = r.shard_value.cpu().numpy()
    si = r.shard_index.cpu().numpy()
    S = inp.V_pad // inp.num_shards
    # every token: the global result is the best shard report, and each shard
    # report lies inside its shard
    assert np.array_equal(r.value.cpu().numpy(), sv.max(axis=0))
    for k in range(inp.num_shards):
        assert ((si[k] >= k * S) & (si[k] < (k + 1) * S)).all()
    sample = _sample_tokens(inp.targets, inp.V_real, 40, 17)
    h64 = oracle.decode(inp.h[sample], inp.dtype)
    W64 = oracle.decode(inp.W, inp.dtype)
    nclear = check_argmax(idx[sample], val[sample], h64, W64, inp.V_real, "c3 sampled")
    say(f"c3 argmax: {nclear} of {len(sample)} sampled tokens without a near tie")


def test_c4_full_size_ot_h_step(V):
    """The OT-H step at the tied-step shapes (second table of the same size):
    counts exact; sampled rows of dh against the oracle's per-token values of
    both heads; padded-free dW2 finite; loss against the oracle on sampled
    tokens of both heads."""
    from synth import make_oth_inputs
    from synth.configs import CONFIGS
    say("case c4 full-size OT-H step")
    c = CONFIGS["c4"]
    inp, W2b, y2 = make_oth_inputs(c.T, c.H, c.V_real, c.V_pad, c.num_shards, c.dtype, c.seed,
                                   zipf_s=1.1, oob_frac=0.01, ignore_frac=0.02)
    dev = "cuda"
    W = V.from_bits(inp.W, inp.dtype, dev)
    W2 = V.from_bits(W2b, inp.dtype, dev)
    ids = torch.from_numpy(inp.ids).to(dev)
    r = V.ot_h_step(ids, torch.from_numpy(inp.targets).to(dev), torch.from_numpy(y2).to(dev),
                    W, W2, inp.V_real, inp.num_shards)
    torch.cuda.synchronize()
    T = inp.T
    f1, f2 = r.fwd, r.extra["fwd2"]
    v1 = (inp.targets >= 0) & (inp.targets < inp.V_real)
    v2 = (y2 >= 0) & (y2 < inp.V_real)
    assert int(f1.n_valid.item()) == int(v1.sum()) and int(f2.n_valid.item()) == int(v2.sum())
    sample = _sample_tokens(inp.targets, inp.V_real, 24, 23)
    sample = sample[sample < T - 1]
    W64 = oracle.decode(inp.W, inp.dtype)
    W2_64 = oracle.decode(W2b, inp.dtype)
    h64 = oracle.gather_direct(inp.ids[sample], W64, inp.V_real)
    g1 = oracle.ce_forward(h64, W64, inp.targets[sample], inp.V_real, inp.V_pad, inp.num_shards)
    g2 = oracle.ce_forward(h64, W2_64, y2[sample], inp.V_real, inp.V_pad, inp.num_shards)
    assert np.abs(f1.lse.cpu().numpy()[sample] - g1["lse"]).max() <= TOL["bf16"]["lse_abs"]
    assert np.abs(f2.lse.cpu().numpy()[sample] - g2["lse"]).max() <= TOL["bf16"]["lse_abs"]
    s1 = 1.0 / int(v1.sum())
    s2 = 0.1 / int(v2.sum())
    dh1, _ = oracle.ce_backward(h64, W64, inp.targets[sample], g1["lse"], inp.V_real, inp.V_pad, s1)
    dh2, _ = oracle.ce_backward(h64, W2_64, y2[sample], g2["lse"], inp.V_real, inp.V_pad, s2)
    e = rel_l2(r.dh.cpu().numpy()[sample], dh1 + dh2)
    assert e <= TOL["bf16"]["grad"], e
    assert torch.isfinite(r.extra["dW2"]).all()
