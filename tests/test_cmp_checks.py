"""The parity checks themselves, on the CPU: a mistake planted in an oracle
result must fail them, and rounding of the size bf16 staging introduces must
not. (Mistakes are planted in copies of oracle outputs, never in the library.)"""

import functools

import numpy as np

import oracle
from synth import config_inputs
from tests._cmp import TOL, check_dw_tiles, rel_l2, tile_rel_l2


@functools.lru_cache(maxsize=1)
def _c2_dW():
    inp = config_inputs("c2", T=512)
    f = oracle.parallel.cross_entropy(oracle.decode(inp.h, "bf16"), oracle.decode(inp.W, "bf16"),
                                      inp.targets, inp.V_real, inp.V_pad, inp.num_shards,
                                      inp.ignore_index, workers=4)
    return inp, f["dW"][:inp.V_real]


def test_tile_check_catches_a_broken_tile_the_whole_tensor_check_misses():
    inp, ref = _c2_dW()
    # the tile of rows [25600, 25856): no target falls there
    y = inp.targets[(inp.targets >= 0) & (inp.targets < inp.V_real)]
    assert not ((y >= 25600) & (y < 25856)).any()
    for planted in ("zero", "negate"):
        got = ref.copy()
        if planted == "zero":
            got[25600:25856] = 0.0
        else:
            got[25600:25856] *= -1.0
        # whole-tensor rel-L2 stays far inside the bar (frequent targets dominate it)
        assert rel_l2(got, ref) < TOL["bf16"]["grad"] / 5
        e = tile_rel_l2(got, ref)
        assert e[100] >= 1.0 and np.delete(e, 100).max() == 0.0
        try:
            check_dw_tiles(got, ref, "bf16")
        except AssertionError:
            pass
        else:
            raise AssertionError(f"a {planted} tile passed the per-tile check")


def test_tile_check_accepts_bf16_sized_rounding():
    inp, ref = _c2_dW()
    rng = np.random.default_rng(0)
    # every element off by up to one bf16 half-ulp (relative 2^-9), random sign
    got = ref * (1.0 + rng.uniform(-1, 1, ref.shape) * 2.0 ** -9)
    assert check_dw_tiles(got, ref, "bf16") < TOL["bf16"]["grad"] / 4
