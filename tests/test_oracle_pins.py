"""Pins that hold the float64 oracle to things other than itself: values the
pages print, closed forms, invariants the pages state, pure-Python brute force
on tiny inputs and central finite differences. CPU only."""

import math
import os

import numpy as np
import pytest

import oracle
from oracle.ce import MEAN, SUM
from synth import bf16_bits_from_f32, make_ce_inputs, config_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(r) for r in rest]
    return vals


# ---------------------------------------------------------------- bits

def test_decode_bf16_exact():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0001, 0x7F80, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.25, 2.0 ** -133, math.inf, -0.0, 3.140625]
    got = oracle.decode(bits, "bf16")
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def test_generator_bf16_round_to_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 1 + 2 ** -8 + 2 ** -20,
                  np.nan], dtype=np.float32)
    b = bf16_bits_from_f32(x)
    assert list(b[:5]) == [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x3F81]
    assert (b[5] & 0x7F80) == 0x7F80 and (b[5] & 0x7F) != 0


# ---------------------------------------------------------------- geometry

def test_geometry_boundaries():
    ids = [0, 255, 256, 511, 512, 767, 768, 999, 1000, 1023, 1024, -1, -100]
    own, loc = oracle.owner_and_local(ids, 1000, 1024, 4)
    assert list(own) == [0, 0, 1, 1, 2, 2, 3, 3, -1, -1, -1, -1, -1]
    assert list(loc) == [0, 255, 0, 255, 0, 255, 0, 231, 0, 0, 0, 0, 0]


@pytest.mark.parametrize("V_real,V_pad,n", [(1000, 1024, 4), (50000, 50016, 8), (5, 8, 8),
                                             (7, 8, 2), (24, 24, 3)])
def test_geometry_exhaustive(V_real, V_pad, n):
    ids = np.arange(-5, V_pad + 5)
    own, loc = oracle.owner_and_local(ids, V_real, V_pad, n)
    S = V_pad // n
    for i, o, l in zip(ids, own, loc):
        owners = [k for k in range(n) if k * S <= i < min((k + 1) * S, V_real)]
        if 0 <= i < V_real:
            assert owners == [o] and o * S + l == i and 0 <= l < S
        else:
            assert owners == [] and o == -1


def test_geometry_rejects_uneven():
    with pytest.raises(ValueError):
        oracle.shard_size(1000, 3)


# ---------------------------------------------------------------- embedding

def test_gather_masked_sum_equals_direct():
    inp = config_inputs("c1")
    W = oracle.decode(inp.W, inp.dtype)
    ids = np.concatenate([inp.ids, np.array([-1, 1000, 1023, 1024, 255, 256, 0, 999])])
    a = oracle.gather_direct(ids, W, inp.V_real)
    b = oracle.gather_masked_shards(ids, W, inp.V_real, inp.V_pad, inp.num_shards)
    assert np.array_equal(a, b)
    # every valid ID reproduces its own row; invalid IDs give zero rows
    for t, i in enumerate(ids):
        if 0 <= i < inp.V_real:
            assert np.array_equal(a[t], W[i])
        else:
            assert not a[t].any()


def test_gather_edge_ids():
    W = np.arange(8 * 3, dtype=np.float64).reshape(8, 3) + 1.0
    ids = [-(2 ** 31), -1, 0, 4, 5, 7, 8, 2 ** 31 - 1]
    out = oracle.gather_direct(ids, W, 5)
    assert np.array_equal(out[2], W[0]) and np.array_equal(out[3], W[4])
    assert not out[[0, 1, 4, 5, 6, 7]].any()


def test_scatter_add_bruteforce():
    rng = np.random.default_rng(7)
    V_real, V_pad, H = 11, 12, 5
    ids = np.array([3, 3, 0, 10, 11, -1, 3, 12, 5, 0, 10, 7], dtype=np.int64)
    dout = rng.standard_normal((ids.shape[0], H))
    dW, count = oracle.scatter_add(ids, dout, V_real, V_pad)
    want = [[0.0] * H for _ in range(V_pad)]
    cnt = [0] * V_pad
    for t, i in enumerate(ids):
        if 0 <= i < V_real:
            cnt[i] += 1
            for j in range(H):
                want[i][j] += float(dout[t, j])
    assert list(count) == cnt
    assert np.allclose(dW, np.array(want), rtol=0, atol=1e-15)
    assert not dW[V_real:].any()


# ---------------------------------------------------------------- CE forward

def test_target_status_cases():
    v, i, b = oracle.target_status([-100, -1, 0, 4, 5, 7, 2 ** 31 - 1], 5, -100)
    assert list(v) == [False, False, True, True, False, False, False]
    assert list(i) == [True, False, False, False, False, False, False]
    assert list(b) == [False, True, False, False, True, True, True]


def _bruteforce_ce(h, W, y, V_real, ignore_index, grad_loss, reduction):
    """Pure-Python reference: math.fsum over explicit loops."""
    T, H = len(h), len(h[0])
    z = [[math.fsum(h[t][j] * W[v][j] for j in range(H)) for v in range(V_real)]
         for t in range(T)]
    lse = []
    for t in range(T):
        m = max(z[t])
        lse.append(m + math.log(math.fsum(math.exp(zv - m) for zv in z[t])))
    valid = [0 <= y[t] < V_real for t in range(T)]
    loss = [lse[t] - z[t][y[t]] if valid[t] else 0.0 for t in range(T)]
    nv = sum(valid)
    scale = grad_loss / max(nv, 1) if reduction == MEAN else grad_loss
    G = [[(math.exp(z[t][v] - lse[t]) - (1.0 if v == y[t] else 0.0)) * scale if valid[t] else 0.0
          for v in range(V_real)] for t in range(T)]
    dh = [[math.fsum(G[t][v] * W[v][j] for v in range(V_real)) for j in range(H)] for t in range(T)]
    dW = [[math.fsum(G[t][v] * h[t][j] for t in range(T)) for j in range(H)] for v in range(V_real)]
    return lse, loss, nv, dh, dW


@pytest.mark.parametrize("V_real,V_pad,n", [(1, 2, 2), (3, 4, 4), (7, 8, 2), (9, 12, 3),
                                             (16, 16, 1), (13, 16, 8)])
def test_bruteforce_tiny(V_real, V_pad, n):
    rng = np.random.default_rng(V_real * 100 + V_pad)
    T, H = 6, 3
    h = rng.standard_normal((T, H))
    W = rng.standard_normal((V_pad, H))
    W[V_real:] = np.nan                      # padded rows must never be read
    y = rng.integers(0, V_real, T)
    y[1] = -100
    y[4] = V_real + (V_pad - V_real) // 2     # a padded row: bad target
    for red in (MEAN, SUM):
        r = oracle.cross_entropy(h, W, y, V_real, V_pad, n, -100, 0.7, red)
        lse, loss, nv, dh, dW = _bruteforce_ce(h.tolist(), W.tolist(), y.tolist(), V_real,
                                               -100, 0.7, red)
        assert np.allclose(r["lse"], lse, rtol=1e-13, atol=1e-13)
        assert np.allclose(r["loss"], loss, rtol=1e-13, atol=1e-13)
        assert r["n_valid"] == nv and r["n_bad"] == 1
        assert np.allclose(r["dh"], dh, rtol=1e-12, atol=1e-13)
        assert np.allclose(r["dW"][:V_real], dW, rtol=1e-12, atol=1e-13)
        assert not r["dW"][V_real:].any()


def test_binomial_page_numbers():
    g = _golden("binomial_softmax.txt")
    w = g["weights"]
    denom = g["denominator"][0]
    assert sum(w) == denom
    V_real, V_pad = 5, 8
    W = np.zeros((V_pad, 1))
    W[:5, 0] = [math.log(math.comb(4, k)) for k in range(5)]
    for garbage in (8.0, np.nan, np.inf):
        W[5:, 0] = garbage
        h = np.ones((5, 1))
        y = np.array([0, 1, 2, 3, 4])
        for n in (1, 2, 4, 8):
            r = oracle.cross_entropy(h, W, y, V_real, V_pad, n, -100, 1.0, SUM)
            assert np.allclose(r["lse"], math.log(denom), rtol=0, atol=1e-14)
            # loss of target k is -log(w_k / 16)
            assert np.allclose(r["loss"], [-math.log(wk / denom) for wk in w], atol=1e-14)
            # the gradient row of token t is p - onehot(t)
            p = np.array(w) / denom
            G = np.tile(p, (5, 1)) - np.eye(5)
            assert np.allclose(r["dh"][:, 0], (G * W[:5, 0]).sum(axis=1), atol=1e-14)
            m, s = r["shard_m"], r["shard_s"]
            assert np.allclose(oracle.merge_shard_stats(m, s), math.log(denom), atol=1e-14)


def test_padded_mass_page_demo():
    g = _golden("padded_mass.txt")
    V_real, V_pad = int(g["V_real"][0]), int(g["V_pad"][0])
    rng = np.random.default_rng(3)
    row = rng.standard_normal(V_pad)
    row[V_real:] = g["pad_logit"][0]
    # W = identity so that the logits of h = row are row itself
    W = np.eye(V_pad)
    h = row[None, :]
    f = oracle.ce_forward(h, W, np.array([0]), V_real, V_pad, 1)
    p_real = np.exp(row[:V_real] - f["lse"][0])
    assert abs(p_real.sum() - g["masked_real_mass"][0]) < 1e-14
    # without the mask the padded columns take almost all the mass
    lse_unmasked = oracle.lse_rows(row[None, :])[0]
    assert np.exp(row[:V_real] - lse_unmasked).sum() < g["unmasked_real_mass_below"][0]


def test_lse_closed_forms():
    # h = 0 gives equal logits over the real rows: lse = ln V_real exactly,
    # and the gradient row is 1/V_real - onehot
    V_real, V_pad, H = 1000, 1024, 64
    rng = np.random.default_rng(11)
    W = rng.standard_normal((V_pad, H)) * 0.02
    W[V_real:] = 8.0
    h = np.zeros((3, H))
    y = np.array([5, 999, -100])
    r = oracle.cross_entropy(h, W, y, V_real, V_pad, 4, -100, 1.0, SUM)
    assert np.allclose(r["lse"], math.log(V_real), rtol=0, atol=1e-12)
    assert abs(math.log(V_real) - math.log(V_pad)) > 0.02
    # dW row v = sum_t G[t, v] h[t] = 0 since h = 0; dh[t] = sum_v (1/V - [v=y]) W[v]
    want = W[:V_real].mean(axis=0) - W[5]
    assert np.allclose(r["dh"][0], want, atol=1e-15)
    assert not r["dh"][2].any()


def test_max_shift_large_logits():
    # logits of +-1000 overflow exp() without the shift; with it the
    # normaliser is exactly 1000 + ln 2 when two logits share the top value
    V_real, V_pad = 10, 16
    W = np.zeros((V_pad, 2))
    W[0] = [1000.0, 0.0]
    W[1] = [1000.0, 0.0]
    W[2] = [-1000.0, 0.0]
    W[3:V_real] = [0.0, 1.0]
    h = np.array([[1.0, 0.0]])
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.log(np.exp(h @ W[:V_real].T).sum()))
    f = oracle.ce_forward(h, W, np.array([0]), V_real, V_pad, 2)
    assert abs(f["lse"][0] - (1000.0 + math.log(2.0))) < 1e-12
    assert abs(f["loss"][0] - math.log(2.0)) < 1e-12


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_sharded_lse_equals_unsharded(n):
    inp = config_inputs("c1")
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    z = oracle.logits(h, W, inp.V_real) * 40.0    # spread the logits out
    ref = oracle.lse_rows(z)
    a = oracle.lse_two_phase(z, inp.V_real, inp.V_pad, n)
    m, s = oracle.shard_stats(z, inp.V_real, inp.V_pad, n)
    b = oracle.merge_shard_stats(m, s)
    assert np.allclose(a, ref, rtol=1e-12, atol=0)
    assert np.allclose(b, ref, rtol=1e-12, atol=0)


def test_empty_shard_stats():
    # V_real = 5 of V_pad = 8 over 8 shards: shards 5..7 own no real row
    z = np.arange(10, dtype=np.float64).reshape(2, 5)
    m, s = oracle.shard_stats(z, 5, 8, 8)
    assert np.all(m[5:] == -np.inf) and not s[5:].any()
    assert np.allclose(oracle.merge_shard_stats(m, s), oracle.lse_rows(z), rtol=1e-14)


def test_local_softmax_negative_control():
    # a planted mistake: each shard normalises over its own rows only.
    # The parity tolerance of the bf16 path (2e-3 relative on the loss) must reject it.
    inp = config_inputs("c1")
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    f = oracle.ce_forward(h, W, inp.targets, inp.V_real, inp.V_pad, inp.num_shards)
    S = inp.S
    z = oracle.logits(h, W, inp.V_real)
    wrong = 0.0
    for t, y in enumerate(inp.targets):
        if f["valid"][t]:
            k = y // S
            zk = z[t, k * S:min((k + 1) * S, inp.V_real)]
            wrong += oracle.lse_rows(zk[None, :])[0] - z[t, y]
    assert abs(wrong - f["loss_sum"]) / f["loss_sum"] > 2e-3


def test_padded_rows_do_not_matter():
    inp = make_ce_inputs(16, 8, 37, 40, 4, "f32", seed=5, ignore_frac=0.2)
    h = oracle.decode(inp.h, "f32")
    base = oracle.decode(inp.W, "f32")
    outs = []
    for fill in (0.0, 8.0, np.nan, -np.inf):
        W = base.copy()
        W[37:] = fill
        outs.append(oracle.cross_entropy(h, W, inp.targets, 37, 40, 4))
    for o in outs[1:]:
        for key in ("lse", "loss", "dh", "dW"):
            assert np.array_equal(o[key], outs[0][key])
        assert not o["dW"][37:].any()


# ---------------------------------------------------------------- CE backward

def _loss_mean(h, W, y, V_real, V_pad, n):
    f = oracle.ce_forward(h, W, y, V_real, V_pad, n)
    return f["loss_sum"] / max(f["n_valid"], 1)


def test_gradient_finite_difference():
    rng = np.random.default_rng(1)
    T, H, V_real, V_pad, n = 3, 4, 7, 8, 2
    h = rng.standard_normal((T, H))
    W = rng.standard_normal((V_pad, H))
    y = np.array([6, -100, 3])
    r = oracle.cross_entropy(h, W, y, V_real, V_pad, n)
    eps = 1e-6
    for t in range(T):
        for j in range(H):
            hp, hm = h.copy(), h.copy()
            hp[t, j] += eps
            hm[t, j] -= eps
            num = (_loss_mean(hp, W, y, V_real, V_pad, n) - _loss_mean(hm, W, y, V_real, V_pad, n)) / (2 * eps)
            assert abs(num - r["dh"][t, j]) < 1e-8
    for v in range(V_pad):
        for j in range(H):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, j] += eps
            Wm[v, j] -= eps
            num = (_loss_mean(h, Wp, y, V_real, V_pad, n) - _loss_mean(h, Wm, y, V_real, V_pad, n)) / (2 * eps)
            assert abs(num - r["dW"][v, j]) < 1e-8
    assert not r["dh"][1].any()


def test_gradient_rows_sum_to_zero():
    inp = config_inputs("c1")
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    r = oracle.cross_entropy(h, W, inp.targets, inp.V_real, inp.V_pad, inp.num_shards)
    # each G row sums to zero, so the dW rows sum to zero
    assert np.abs(r["dW"].sum(axis=0)).max() < 1e-12
    assert not r["dW"][inp.V_real:].any()
    ign = ~r["valid"]
    assert ign.any() and not r["dh"][ign].any()
    assert r["n_valid"] == int(np.sum((inp.targets >= 0) & (inp.targets < inp.V_real)))


def test_mean_normalised_once_and_no_valid_tokens():
    inp = make_ce_inputs(8, 8, 20, 24, 2, "f32", seed=2)
    h = oracle.decode(inp.h, "f32")
    W = oracle.decode(inp.W, "f32")
    r_sum = oracle.cross_entropy(h, W, inp.targets, 20, 24, 2, grad_loss=1.0, reduction=SUM)
    r_mean = oracle.cross_entropy(h, W, inp.targets, 20, 24, 2, grad_loss=1.0, reduction=MEAN)
    assert r_mean["loss_reduced"] == pytest.approx(r_sum["loss_sum"] / 8, rel=1e-15)
    assert np.allclose(r_mean["dh"] * 8, r_sum["dh"], rtol=1e-13, atol=1e-15)
    none = np.full(8, -100)
    r0 = oracle.cross_entropy(h, W, none, 20, 24, 2)
    assert r0["loss_reduced"] == 0.0 and r0["n_valid"] == 0
    assert not r0["dh"].any() and not r0["dW"].any()
    assert np.all(np.isfinite(r0["lse"]))


def test_c1_has_argmax_and_target_on_different_shards():
    inp = config_inputs("c1")
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    z = oracle.logits(h, W, inp.V_real)
    am = z.argmax(axis=1)
    y = inp.targets
    ok = (y >= 0) & (y < inp.V_real)
    assert int(np.sum(ok & (am // inp.S != y // inp.S))) >= 4
    for v in (255, 256, 511, 512, 990, 999):
        assert v in set(y.tolist())


# ---------------------------------------------------------------- tied step

def test_tied_step_finite_difference():
    rng = np.random.default_rng(4)
    T, H, V_real, V_pad, n = 5, 3, 6, 8, 2
    W = rng.standard_normal((V_pad, H))
    ids = np.array([2, 2, 7, 5, -3])        # a repeat, a padded ID, an out-of-range ID
    y = np.array([1, 5, -100, 2, 0])
    r = oracle.tied_step(ids, y, W, V_real, V_pad, n)

    def loss_of(Wx):
        hx = oracle.gather_direct(ids, Wx, V_real)
        return _loss_mean(hx, Wx, y, V_real, V_pad, n)

    eps = 1e-6
    for v in range(V_pad):
        for j in range(H):
            Wp, Wm = W.copy(), W.copy()
            Wp[v, j] += eps
            Wm[v, j] -= eps
            num = (loss_of(Wp) - loss_of(Wm)) / (2 * eps)
            assert abs(num - r["dW"][v, j]) < 1e-8
    assert list(r["count"]) == [0, 0, 2, 0, 0, 1, 0, 0]


# ---------------------------------------------------------------- parallel schedule

def test_parallel_schedule_matches_sequential():
    """oracle.parallel evaluates the same definitions over token and
    vocabulary chunks on many threads; it must agree with the sequential,
    pinned oracle to float64 rounding (chunks deliberately ragged)."""
    inp = config_inputs("c1")
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    y = inp.targets.copy()
    y[3] = inp.V_real + 5      # a bad target (padded class)
    y[7] = 5000                # a bad target (past the table)
    for red, gl in ((MEAN, 1.0), (SUM, 0.5)):
        ref = oracle.cross_entropy(h, W, y, inp.V_real, inp.V_pad, inp.num_shards,
                                   inp.ignore_index, gl, red)
        got = oracle.parallel.cross_entropy(h, W, y, inp.V_real, inp.V_pad, inp.num_shards,
                                            inp.ignore_index, gl, red, workers=4,
                                            tok_chunk=7, voc_chunk=97)
        assert got["n_valid"] == ref["n_valid"] and got["n_bad"] == ref["n_bad"]
        for k in ("lse", "loss", "zt", "dh", "dW"):
            np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-15, err_msg=k)
        assert abs(got["loss_sum"] - ref["loss_sum"]) <= 1e-12 * abs(ref["loss_sum"])
        assert not got["dW"][inp.V_real:].any()
    ids = inp.ids.copy()
    ids[:4] = [-1, inp.V_real, inp.V_pad - 1, 7]
    ref = oracle.tied_step(ids, y, W, inp.V_real, inp.V_pad, inp.num_shards)
    got = oracle.parallel.tied_step(ids, y, W, inp.V_real, inp.V_pad, inp.num_shards,
                                    workers=3)
    for k in ("lse", "loss", "dh", "dW", "dW_emb"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-15, err_msg=k)
    assert np.array_equal(got["count"], ref["count"])


# ---------------------------------------------------------------- sampled softmax

def test_candidates_bruteforce():
    V, P = 20, 9
    y = np.array([3, 3, 17, -100, 0, 17, 25, 8])
    perm = np.random.default_rng(9).permutation(V)
    cand, pos, nu = oracle.candidates(y, V, -100, perm, P)
    U = sorted(set(int(v) for v in y if 0 <= v < V))
    assert nu == len(U) and list(cand[:nu]) == U
    negs = []
    for v in perm:
        if int(v) not in U and len(negs) < P - len(U):
            negs.append(int(v))
    assert list(cand[nu:]) == negs and len(cand) == P
    assert len(set(cand.tolist())) == P
    for t, v in enumerate(y):
        if 0 <= v < V:
            assert cand[pos[t]] == v
        else:
            assert pos[t] == v
    # more unique targets than P: the candidates are the unique targets alone
    cand2, _, nu2 = oracle.candidates(np.arange(12), V, -100, perm, 5)
    assert nu2 == 12 and list(cand2) == list(range(12))


def test_sampled_full_candidate_set_equals_full_ce():
    inp = make_ce_inputs(12, 6, 30, 30, 1, "f32", seed=8, ignore_frac=0.2)
    h = oracle.decode(inp.h, "f32")
    W = oracle.decode(inp.W, "f32")
    perm = np.random.default_rng(2).permutation(30)
    s = oracle.sampled_step(h, W, inp.targets, perm, P=30)
    f = oracle.cross_entropy(h, W, inp.targets, 30, 30, 1)
    assert np.allclose(s["lse"], f["lse"], rtol=1e-13)
    assert np.allclose(s["loss"], f["loss"], rtol=1e-13, atol=1e-15)
    assert np.allclose(s["dh"], f["dh"], rtol=1e-12, atol=1e-15)
    assert np.allclose(s["dW"], f["dW"], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------ greedy argmax

def _bruteforce_argmax(h, W, V_real):
    """Pure-Python: exact logits by math.fsum, first index holding the maximum."""
    out = []
    for row in h:
        best_v, best_i = None, None
        for v in range(V_real):
            z = math.fsum(a * b for a, b in zip(row, W[v]))
            if best_v is None or z > best_v:
                best_v, best_i = z, v
        out.append((best_i, best_v))
    return out


@pytest.mark.parametrize("V_real,V_pad,n", [(1, 2, 2), (3, 4, 4), (7, 8, 2), (9, 12, 3),
                                             (16, 16, 1), (13, 16, 8)])
def test_argmax_bruteforce_tiny(V_real, V_pad, n):
    rng = np.random.default_rng(V_real * 31 + V_pad)
    T, H = 9, 4
    h = rng.standard_normal((T, H))
    W = rng.standard_normal((V_pad, H))
    W[V_real:] = np.nan                     # padded rows must never be read
    r = oracle.greedy_argmax(h, W, V_real, V_pad, n)
    ref = _bruteforce_argmax(h.tolist(), W.tolist(), V_real)
    assert r["index"].tolist() == [i for i, _ in ref]
    assert np.allclose(r["value"], [v for _, v in ref], rtol=1e-14, atol=1e-14)


def test_argmax_padded_rows_never_chosen():
    rng = np.random.default_rng(8)
    T, H, V_real, V_pad = 5, 6, 10, 16
    h = np.abs(rng.standard_normal((T, H)))
    W = rng.standard_normal((V_pad, H))
    for pad in (1e30, np.inf, np.nan):
        W[V_real:] = pad
        for n in (1, 2, 4, 8):
            r = oracle.greedy_argmax(h, W, V_real, V_pad, n)
            assert (r["index"] < V_real).all() and (r["index"] >= 0).all()
    # the last shard of n = 8 (rows 14, 15) owns no real row
    r = oracle.greedy_argmax(h, W, V_real, V_pad, 8)
    assert (r["shard_index"][5:] == -1).all() and np.isneginf(r["shard_value"][5:]).all()


def test_argmax_ties_take_lowest_index():
    # rows 2, 5, 9 and 13 are copies of one row that beats every other row;
    # with 4 shards of 4 rows the copies sit in shards 0, 1, 2 and 3
    rng = np.random.default_rng(9)
    T, H, V = 4, 3, 16
    h = np.abs(rng.standard_normal((T, H))) + 0.1
    W = -np.abs(rng.standard_normal((V, H)))
    top = np.array([3.0, 2.0, 1.0])
    for v in (13, 9, 5, 2):
        W[v] = top
    for n in (1, 2, 4, 8, 16):
        r = oracle.greedy_argmax(h, W, V, V, n)
        assert (r["index"] == 2).all()
    # without row 2 the lowest copy left is row 5 (shard 1 of 4)
    W[2] = -top
    r = oracle.greedy_argmax(h, W, V, V, 4)
    assert (r["index"] == 5).all()
    assert (r["shard_index"][1:, 0] == [5, 9, 13]).all()


def test_argmax_one_hot_hidden_rows():
    # h_t = e_j makes z[t, v] = W[v, j]: the argmax is the row holding the
    # largest entry of column j
    V_real, V_pad, H = 37, 40, 5
    W = np.tile(np.arange(V_pad, dtype=np.float64)[:, None] * 0.0, (1, H))
    winners = [3, 36, 17, 0, 22]
    for j, v in enumerate(winners):
        W[:, j] = -1.0
        W[v, j] = 2.0 + j
    W[V_real:] = 100.0                       # padding: larger, but not classes
    h = np.eye(H)
    for n in (1, 2, 4, 5, 8):
        r = oracle.greedy_argmax(h, W, V_real, V_pad, n)
        assert r["index"].tolist() == winners
        assert r["value"].tolist() == [2.0 + j for j in range(H)]


@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_argmax_sharded_equals_unsharded(n):
    inp = config_inputs("c1")
    h = oracle.decode(inp.h, inp.dtype)
    W = oracle.decode(inp.W, inp.dtype)
    z = h @ W[:inp.V_real].T
    r = oracle.greedy_argmax(h, W, inp.V_real, inp.V_pad, n)
    # the global maximum of the merged reports equals the unsharded maximum,
    # and the chosen index holds it
    assert np.array_equal(r["value"], z.max(axis=1))
    assert np.array_equal(z[np.arange(z.shape[0]), r["index"]], r["value"])
    one = oracle.greedy_argmax(h, W, inp.V_real, inp.V_pad, 1)
    assert np.array_equal(r["index"], one["index"])


# ------------------------------------------------------------------ OT-H step

def test_ot_h_step_finite_difference():
    """Central differences of the OT-H loss in every entry of W and W2 equal
    the step's dW and dW2; the first head's loss plus 0.1 times the second's."""
    rng = np.random.default_rng(14)
    T, H, V_real, V_pad, n = 6, 3, 6, 8, 2
    W = rng.standard_normal((V_pad, H))
    W2 = rng.standard_normal((V_pad, H))
    tokens = np.array([2, 2, 7, 5, 1, 3, 0, 4])   # a repeat, a padded ID
    ids = tokens[:T].copy()
    ids[4] = -3                                    # an out-of-range ID
    y1 = tokens[1:T + 1].copy()
    y1[2] = -100                                   # ignored in the first head only
    y2 = tokens[2:T + 1].copy()
    y2[0] = 7                                      # a padded class: a bad target
    r = oracle.ot_h_step(ids, y1, y2, W, W2, V_real, V_pad, n)

    def loss_of(Wx, W2x):
        hx = oracle.gather_direct(ids, Wx, V_real)
        return (_loss_mean(hx, Wx, y1, V_real, V_pad, n) +
                0.1 * _loss_mean(hx[:T - 1], W2x, y2, V_real, V_pad, n))

    assert abs(loss_of(W, W2) - r["loss"]) < 1e-12
    eps = 1e-6
    for v in range(V_pad):
        for j in range(H):
            for which, G in ((0, r["dW"]), (1, r["dW2"])):
                P = [W.copy(), W2.copy()]
                M = [W.copy(), W2.copy()]
                P[which][v, j] += eps
                M[which][v, j] -= eps
                num = (loss_of(*P) - loss_of(*M)) / (2 * eps)
                assert abs(num - G[v, j]) < 1e-8, (which, v, j, num, G[v, j])
    # the second head never sees the last row, and its padded rows stay zero
    assert not r["dW2"][V_real:].any()
    assert r["f2"]["n_bad"] == 1


# ------------------------------------------------------------------ hashed n-gram embeddings

def test_ngram_ids_exist_only_for_whole_valid_ngrams():
    V_real, r2, r3 = 50, 97, 101
    ids = np.array([3, 7, -1, 8, 9, 10, 50, 11, 12, 13, 3, 7])
    i2, i3 = oracle.ngram_ids(ids, V_real, r2, r3)
    ok = [(0 <= x < V_real) for x in ids]
    for t in range(len(ids)):
        assert (i2[t] >= 0) == (t >= 1 and ok[t - 1] and ok[t])
        assert (i3[t] >= 0) == (t >= 2 and ok[t - 2] and ok[t - 1] and ok[t])
    assert ((i2 >= -1) & (i2 < r2)).all() and ((i3 >= -1) & (i3 < r3)).all()
    # the same n-gram maps to the same row wherever it occurs, and order matters
    assert i2[1] == i2[11] and i2[1] >= 0
    rev, _ = oracle.ngram_ids(np.array([7, 3]), V_real, r2, r3)
    assert rev[1] != i2[1]


def test_ngram_rows_spread_uniformly():
    # 40000 distinct 2-grams into 64 rows: chi-square of the counts within the
    # 1e-6 tail of its distribution (63 degrees of freedom: < 140)
    V_real, rows = 200, 64
    a = np.repeat(np.arange(200), 200)
    b = np.tile(np.arange(200), 200)
    rows_of = np.array([oracle.mix64(int(x) * V_real + int(y)) % rows for x, y in zip(a, b)])
    counts = np.bincount(rows_of, minlength=rows)
    expect = len(a) / rows
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 140, chi2
    # the finaliser is a bijection on 64 bits: no collisions among distinct keys
    keys = np.arange(1, 200001) * 1000003
    assert len({oracle.mix64(int(k)) for k in keys}) == len(keys)


def test_mix64_is_the_splitmix64_finaliser():
    """Known answers: the SplitMix64 generator (state advanced by its golden
    gamma, each output the finaliser of the new state) started from state 0
    yields the published first outputs (tests/golden/splitmix64_seed0.txt).
    A changed shift or multiplier of the finaliser changes all three."""
    gamma = seed = None
    outs = []
    with open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split()
            if key == "gamma":
                gamma = int(val, 16)
            elif key == "seed":
                seed = int(val)
            elif key == "output":
                outs.append(int(val, 16))
    assert gamma is not None and seed is not None and len(outs) == 3
    state = seed
    for want in outs:
        state = (state + gamma) & ((1 << 64) - 1)
        assert oracle.mix64(state) == want, hex(oracle.mix64(state))


def test_ngram_embed_bruteforce():
    rng = np.random.default_rng(21)
    T, H, V_real, V_pad, r2, r3 = 9, 4, 12, 16, 10, 14
    E = rng.standard_normal((V_pad, H))
    E[V_real:] = np.nan                      # padded unigram rows are never read
    E2 = rng.standard_normal((r2, H))
    E3 = rng.standard_normal((r3, H))
    ids = np.array([1, 5, 5, 13, 2, 11, 0, -4, 6])
    x, i2, i3 = oracle.ngram_embed(ids, E, E2, E3, V_real)
    for t in range(T):
        want = [0.0] * H
        if 0 <= ids[t] < V_real:
            want = [w + e for w, e in zip(want, E[ids[t]])]
        if i2[t] >= 0:
            want = [w + e for w, e in zip(want, E2[i2[t]])]
        if i3[t] >= 0:
            want = [w + e for w, e in zip(want, E3[i3[t]])]
        assert np.allclose(x[t], want, rtol=0, atol=1e-15)
    assert not np.isnan(x).any()


def test_ngram_backward_finite_difference():
    rng = np.random.default_rng(22)
    T, H, V_real, V_pad, r2, r3 = 8, 3, 6, 8, 5, 7
    E = rng.standard_normal((V_pad, H))
    E2 = rng.standard_normal((r2, H))
    E3 = rng.standard_normal((r3, H))
    ids = np.array([1, 2, 1, 2, 7, 3, 1, 2])   # repeated n-grams, a padded ID
    c = rng.standard_normal((T, H))

    def loss(E_, E2_, E3_):
        x, _, _ = oracle.ngram_embed(ids, E_, E2_, E3_, V_real)
        return 0.5 * float((c * x * x).sum())

    x, _, _ = oracle.ngram_embed(ids, E, E2, E3, V_real)
    dE, dE2, dE3 = oracle.ngram_backward(ids, c * x, V_real, V_pad, r2, r3)
    eps = 1e-6
    for which, (tab, grad) in enumerate(((E, dE), (E2, dE2), (E3, dE3))):
        for v in range(tab.shape[0]):
            for j in range(H):
                args_p = [E.copy(), E2.copy(), E3.copy()]
                args_m = [E.copy(), E2.copy(), E3.copy()]
                args_p[which][v, j] += eps
                args_m[which][v, j] -= eps
                num = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                assert abs(num - grad[v, j]) < 1e-7, (which, v, j)


# ------------------------------------------------------------------ uneven and mapped shards

UNEVEN = [
    (1000, 1024, [0, 100, 100, 613, 1000, 1024]),    # an empty shard, the padding its own shard
    (1000, 1024, [0, 1, 2, 900, 1024]),               # one-row shards, padding inside the last
    (37, 64, [0, 64]),                                # one shard
    (50, 64, [0, 10, 20, 30, 40, 50, 60, 64]),        # uneven tail
]


@pytest.mark.parametrize("V_real,V_pad,rows", UNEVEN)
def test_uneven_owner_and_gather(V_real, V_pad, rows):
    n = len(rows) - 1
    ids = np.arange(-3, V_pad + 3)
    owner, local = oracle.owner_and_local(ids, V_real, V_pad, n, shard_rows=rows)
    for i, o, l in zip(ids, owner, local):
        if 0 <= i < V_real:
            assert rows[o] <= i < rows[o + 1] and rows[o] + l == i
        else:
            assert o == -1 and l == 0
    W = np.random.default_rng(3).standard_normal((V_pad, 5))
    W[V_real:] = np.nan
    a = oracle.gather_masked_shards(ids, W, V_real, V_pad, n, shard_rows=rows)
    b = oracle.gather_direct(ids, W, V_real)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("V_real,V_pad,rows", UNEVEN)
def test_uneven_sharded_lse_and_argmax_equal_unsharded(V_real, V_pad, rows):
    n = len(rows) - 1
    rng = np.random.default_rng(V_real + n)
    z = rng.standard_normal((7, V_real)) * 3
    ref = oracle.lse_rows(z)
    m, s = oracle.shard_stats(z, V_real, V_pad, n, shard_rows=rows)
    assert np.allclose(oracle.merge_shard_stats(m, s), ref, rtol=1e-12, atol=0)
    assert np.allclose(oracle.lse_two_phase(z, V_real, V_pad, n, shard_rows=rows), ref,
                       rtol=1e-12, atol=0)
    for k in range(n):
        if min(rows[k + 1], V_real) <= rows[k]:
            assert np.isneginf(m[k]).all() and not s[k].any()
    v, i = oracle.merge_shard_argmax(*oracle.shard_argmax(z, V_real, V_pad, n, shard_rows=rows))
    assert np.array_equal(i, np.argmax(z, axis=1)) and np.array_equal(v, z.max(axis=1))


def test_uneven_layout_rejected_when_malformed():
    for rows in ([0, 10, 5, 16], [1, 8, 16], [0, 8, 15], [0, 16, 16, 16, 17]):
        with pytest.raises(ValueError):
            oracle.shard_bounds(16, len(rows) - 1, rows)


def test_mapped_ownership_is_a_relabelling():
    """Classes placed at physical rows by a permutation: the table stored in
    physical order with remapped targets and IDs gives the same losses, the
    same lookups and the gradient rows of the same classes; the argmax maps
    back to the same class."""
    rng = np.random.default_rng(31)
    T, H, V_real, V_pad = 9, 6, 40, 48
    rows = [0, 7, 7, 30, 48]
    n = len(rows) - 1
    W = rng.standard_normal((V_pad, H))
    h = rng.standard_normal((T, H))
    y = rng.integers(0, V_real, T)
    y[2] = -100
    row_of = rng.permutation(V_real)
    class_of = np.argsort(row_of)
    Wp = W.copy()
    Wp[row_of] = W[:V_real]
    yp = oracle.remap(y, row_of, V_real)
    assert yp[2] == -100
    a = oracle.cross_entropy(h, W, y, V_real, V_pad, 1)
    b = oracle.cross_entropy(h, Wp, yp, V_real, V_pad, n, shard_rows=rows)
    assert np.allclose(a["lse"], b["lse"], rtol=1e-13, atol=0)
    assert np.allclose(a["loss"], b["loss"], rtol=1e-12, atol=1e-14)
    assert np.allclose(a["dh"], b["dh"], rtol=1e-12, atol=1e-14)
    assert np.allclose(a["dW"][:V_real], b["dW"][row_of], rtol=1e-12, atol=1e-14)
    ids = np.array([3, 39, -1, 40, 0])
    assert np.array_equal(oracle.gather_direct(ids, W, V_real),
                          oracle.gather_direct(oracle.remap(ids, row_of, V_real), Wp, V_real))
    ga = oracle.greedy_argmax(h, W, V_real, V_pad, 1)
    gb = oracle.greedy_argmax(h, Wp, V_real, V_pad, n, shard_rows=rows)
    assert np.array_equal(class_of[gb["index"]], ga["index"])
