"""The allocation-free greedy argmax (vce_argmax_noalloc, static device
scratch) against the workspace entry point it shares its kernels with:
bitwise equal results on two calls in a row, the second smaller, so stale
scratch contents from the first call cannot leak into the second."""

import sys

import numpy as np
import pytest

from synth import make_ce_inputs

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


def _both(V, inp):
    dev = "cuda"
    h = V.from_bits(inp.h, inp.dtype, dev)
    W = V.from_bits(inp.W, inp.dtype, dev)
    a = V.vce_argmax_noalloc(h, W, inp.V_real, inp.num_shards, shard_reports=True)
    b = V.vce_argmax(h, W, inp.V_real, inp.num_shards, shard_reports=True)
    torch.cuda.synchronize()
    for name in ("index", "value", "shard_value", "shard_index"):
        x = getattr(a, name).cpu().numpy()
        y = getattr(b, name).cpu().numpy()
        assert np.array_equal(x.view(np.int32), y.view(np.int32)), name
    return a


def test_argmax_noalloc_equals_workspace_call(V):
    # the largest T the 16 MiB scratch takes at the 201088-row table over 8 shards
    say("case noalloc argmax T=2647 H=1024 V=201088 n=8, then T=300 H=512 V=50016 n=8")
    big = make_ce_inputs(2647, 1024, 201088, 201088, 8, "bf16", seed=61)
    small = make_ce_inputs(300, 512, 50000, 50016, 8, "bf16", seed=62)
    _both(V, big)
    _both(V, small)
    # and once more at the large size after the small one
    _both(V, big)


def test_argmax_noalloc_rejects_oversize(V):
    dev = "cuda"
    h = torch.zeros(2648, 64, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(201088, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(V.VceError):
        V.vce_argmax_noalloc(h, W, 201088, 8)
