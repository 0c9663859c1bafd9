"""The five workloads, each with a fixed seed (1000 + its number).

c1  tiny fp32 CE + embedding: T=64, H=64, V_real=1000 -> V_pad=1024, 4 shards of 256 rows.
c2  mid bf16 CE + embedding: T=2048, H=1024, V_real=50000 -> V_pad=50016, 8 shards;
    the 16 padded rows hold +8.0 in every element.
c3  large-vocab bf16 CE: T=8192, H=3072, V=201088, 8 shards of 25136 rows.
c4  tied embedding + LM-head bf16 step: T=16384, H=3072, V=201088, 8 shards.
c5  sampled-softmax bf16 CE: T=16384, H=1536, V=131072, P=16384 candidates.
"""

from __future__ import annotations

import dataclasses

from .gen import make_ce_inputs, make_sampled_inputs, make_tied_inputs


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str          # 'ce', 'tied' or 'sampled'
    T: int
    H: int
    V_real: int
    V_pad: int
    num_shards: int
    dtype: str
    seed: int
    P: int = 0

    @property
    def S(self) -> int:
        return self.V_pad // self.num_shards


CONFIGS = {
    "c1": Config("c1", "ce", 64, 64, 1000, 1024, 4, "f32", 1001),
    "c2": Config("c2", "ce", 2048, 1024, 50000, 50016, 8, "bf16", 1002),
    "c3": Config("c3", "ce", 8192, 3072, 201088, 201088, 8, "bf16", 1003),
    "c4": Config("c4", "tied", 16384, 3072, 201088, 201088, 8, "bf16", 1004),
    "c5": Config("c5", "sampled", 16384, 1536, 131072, 131072, 1, "bf16", 1005, P=16384),
}

# c1: targets on both sides of every shard boundary and in the last real rows
C1_FORCED = (255, 256, 511, 512) + tuple(range(990, 1000))
# c2: the real tail and both sides of three shard boundaries (S = 6252)
C2_FORCED = tuple(range(49990, 50000)) + (6251, 6252, 12503, 12504, 43763, 43764)


def config_inputs(name: str, **overrides):
    """Build the seeded inputs of workload ``name``. ``overrides`` changes the
    size parameters only (T, H, ...) for scaled-down variants of the same recipe."""
    c = CONFIGS[name]
    p = dict(T=c.T, H=c.H, V_real=c.V_real, V_pad=c.V_pad, num_shards=c.num_shards,
             dtype=c.dtype, seed=c.seed)
    p.update(overrides)
    if name == "c1":
        return make_ce_inputs(p["T"], p["H"], p["V_real"], p["V_pad"], p["num_shards"],
                              p["dtype"], p["seed"], target_dist="uniform",
                              ignore_frac=0.10, forced_targets=C1_FORCED,
                              id_dist="uniform", id_repeat_frac=0.20, name="c1")
    if name == "c2":
        Vr = p["V_real"]
        forced = tuple(v for v in C2_FORCED if v < Vr)
        pad_ids = tuple(range(Vr, p["V_pad"]))
        return make_ce_inputs(p["T"], p["H"], Vr, p["V_pad"], p["num_shards"],
                              p["dtype"], p["seed"], target_dist="zipf", zipf_s=1.1,
                              ignore_frac=0.05, forced_targets=forced, pad_fill=8.0,
                              id_dist="zipf", id_extra=pad_ids, name="c2")
    if name == "c3":
        return make_ce_inputs(p["T"], p["H"], p["V_real"], p["V_pad"], p["num_shards"],
                              p["dtype"], p["seed"], target_dist="zipf", zipf_s=1.1,
                              ignore_frac=0.02, h_dist="rms", name="c3")
    if name == "c4":
        return make_tied_inputs(p["T"], p["H"], p["V_real"], p["V_pad"], p["num_shards"],
                                p["dtype"], p["seed"], zipf_s=1.1, oob_frac=0.01,
                                ignore_frac=0.02, name="c4")
    if name == "c5":
        P = overrides.get("P", c.P)
        return make_sampled_inputs(p["T"], p["H"], p["V_real"], P, p["dtype"], p["seed"],
                                   zipf_s=1.1, name="c5")
    raise KeyError(name)
