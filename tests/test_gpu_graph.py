"""HIP graph capture of whole steps: the library's calls enqueue kernels only
(no allocation, memset, copy or synchronisation inside a call; workspaces are
the caller's), so a step captured once replays as one graph. Each replay is
checked bitwise against eager calls of the same step on the same inputs (the
path is deterministic), with eager work and synchronisations between the
replays, and again after the captured inputs are overwritten in place."""

import sys

import numpy as np
import pytest

from synth import make_sampled_inputs, make_tied_inputs

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


def capture(fn):
    """torch's capture recipe: warm up on a side stream, then record fn()."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def same(a, b, name):
    a, b = a.detach().cpu(), b.detach().cpu()
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    x, y = a.numpy(), b.numpy()
    assert x.dtype == y.dtype and x.shape == y.shape, name
    assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{name}: replay differs from eager"


def test_tied_step_graph_replays(V):
    say("case graph: tied step T=1024 H=256 V=6000/6144 n=4, 3 replays + new inputs")
    dev = torch.device("cuda:0")
    T, H, Vr, Vp, n = 1024, 256, 6000, 6144, 4
    inp = make_tied_inputs(T, H, Vr, Vp, n, "bf16", seed=31)
    inp2 = make_tied_inputs(T, H, Vr, Vp, n, "bf16", seed=32)
    W = V.from_bits(inp.W, "bf16", dev)
    ids = torch.from_numpy(inp.ids).to(dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    gl = torch.ones(1, dtype=torch.float32, device=dev)

    def buffers():
        ws = V.Workspaces(dev, fwd=V.vce_fwd_workspace_bytes(T, H, Vr, Vp, n),
                          bwd=V.vce_bwd_workspace_bytes(T, H, Vr, Vp, n),
                          emb=V.vemb_bwd_workspace_bytes(T, H, Vr, Vp))
        return dict(ws=ws, h=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                    dh=torch.empty(T, H, dtype=torch.float32, device=dev),
                    dW=torch.empty(Vp, H, dtype=torch.float32, device=dev))

    gb, eb = buffers(), buffers()

    def step(b, i, t):
        # no synchronisation inside a captured step: n_bad is checked by the test
        return V.tied_step(i, t, W, Vr, n, inp.ignore_index, grad_loss=gl, ws=b["ws"], h=b["h"],
                           dh=b["dh"], dW=b["dW"], allow_bad=True)

    g, out = capture(lambda: step(gb, ids, tg))

    def check(i, t):
        ref = step(eb, i, t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same(out.fwd.loss_sum, ref.fwd.loss_sum, "loss_sum")
        same(out.fwd.lse, ref.fwd.lse, "lse")
        same(out.fwd.n_valid, ref.fwd.n_valid, "n_valid")
        assert int(out.fwd.n_bad.item()) == 0
        same(out.dh, ref.dh, "dh")
        same(out.dW, ref.dW, "dW")
        same(out.extra["h"], ref.extra["h"], "h")

    for _ in range(3):
        check(ids, tg)
    ids.copy_(torch.from_numpy(inp2.ids))
    tg.copy_(torch.from_numpy(inp2.targets))
    check(ids, tg)


def test_sampled_step_graph_replays(V):
    say("case graph: sampled step T=1024 H=128 V=16384 P=2048, 3 replays")
    dev = torch.device("cuda:0")
    inp = make_sampled_inputs(1024, 128, 16384, 2048, "bf16", seed=33)
    T, H, Vt, P = inp.T, inp.H, inp.V_real, inp.P
    h = V.from_bits(inp.h, "bf16", dev)
    W = V.from_bits(inp.W, "bf16", dev)
    tg = torch.from_numpy(inp.targets).to(dev)
    perm = torch.from_numpy(inp.perm).to(dev)
    gl = torch.ones(1, dtype=torch.float32, device=dev)

    def buffers():
        ws = V.Workspaces(dev, cand=V.vss_candidates_workspace_bytes(T, Vt),
                          fwd=V.vce_fwd_workspace_bytes(T, H, P, P, 1),
                          bwd=V.vce_bwd_workspace_bytes(T, H, P, P, 1))
        return dict(ws=ws, dW=torch.empty(Vt, H, dtype=torch.float32, device=dev))

    gb, eb = buffers(), buffers()

    def step(b):
        # the batch has fewer distinct targets than P, so n_cand = P (checked below)
        return V.sampled_step(h, W, tg, perm, P, inp.ignore_index, grad_loss=gl, ws=b["ws"],
                              dW=b["dW"], n_cand=P, allow_bad=True)

    g, out = capture(lambda: step(gb))
    for _ in range(3):
        ref = step(eb)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same(out.extra["cand"][:P], ref.extra["cand"][:P], "cand")
        assert int(out.extra["n_cand"].item()) == P and int(out.fwd.n_bad.item()) == 0
        same(out.fwd.loss_sum, ref.fwd.loss_sum, "loss_sum")
        same(out.dh, ref.dh, "dh")
        same(out.dW, ref.dW, "dW")
