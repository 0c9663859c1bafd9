"""Over-Tokenized input side: hashed 2-gram and 3-gram embeddings added to
every input token's embedding, and their backward, in float64.

Definition followed: [SS] "Setup" and its loss listing: OT's input side adds,
to the embedding of each input token, a hashed 2-gram embedding and a hashed
3-gram embedding of the n-grams that end at that token:
  x[t] = E[ids[t]] + E2[hash2(ids[t-1], ids[t])] + E3[hash3(ids[t-2], ids[t-1], ids[t])].
The page's related-work list gives the tables' size only as a total (6.5B
parameters at 300m, OT-H); the hash is not on the page.

Readings where the page is silent (also in the design notes):
  - key of an n-gram: its token IDs in base V_real, oldest first:
    key2 = a*V_real + b, key3 = (a*V_real + b)*V_real + c, as unsigned 64-bit;
  - row of an n-gram: mix64(key) mod rows_n, where mix64 is the 64-bit
    finaliser of the SplitMix64 generator (Steele, Lea and Flood, "Fast
    splittable pseudorandom number generators", OOPSLA 2014): three rounds of
    xor-shift and multiplication by odd constants, published with the
    generator, applied as written there;
  - an n-gram exists at position t only if t >= n-1 and all of its n tokens
    are valid IDs (in [0, V_real)); a missing n-gram adds a zero row and gets
    no gradient (the same rule as an invalid unigram ID);
  - the T input tokens form one sequence (no n-gram crosses position 0);
  - the n-gram tables are split into the same number of contiguous, equal
    shards as the unigram table (rows_n % num_shards == 0) and looked up by
    owner and local index the same way.
Pinned by tests/test_oracle_pins.py::test_mix64_is_the_splitmix64_finaliser
(the generator's published first outputs from state 0) and test_ngram_* (brute
force over positions, range and uniformity of the rows, finite differences of
the backward).
"""

from __future__ import annotations

import numpy as np

from .embedding import gather_direct, scatter_add

_M64 = (1 << 64) - 1


def mix64(z: int) -> int:
    """The SplitMix64 output finaliser on one unsigned 64-bit integer."""
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def ngram_ids(ids, V_real: int, rows2: int, rows3: int):
    """(i2, i3) int64 [T]: the table row of the 2-gram / 3-gram ending at each
    position, -1 where that n-gram does not exist."""
    ids = [int(x) for x in np.asarray(ids, dtype=np.int64)]
    T = len(ids)
    ok = [0 <= x < V_real for x in ids]
    i2 = np.full(T, -1, dtype=np.int64)
    i3 = np.full(T, -1, dtype=np.int64)
    for t in range(T):
        if t >= 1 and ok[t - 1] and ok[t]:
            key = ids[t - 1] * V_real + ids[t]
            i2[t] = mix64(key) % rows2
        if t >= 2 and ok[t - 2] and ok[t - 1] and ok[t]:
            key = (ids[t - 2] * V_real + ids[t - 1]) * V_real + ids[t]
            i3[t] = mix64(key) % rows3
    return i2, i3


def ngram_embed(ids, E, E2, E3, V_real: int):
    """x [T, H] float64 = unigram + 2-gram + 3-gram rows (zero rows where missing)."""
    i2, i3 = ngram_ids(ids, V_real, E2.shape[0], E3.shape[0])
    x = gather_direct(ids, E, V_real).astype(np.float64)
    x += gather_direct(i2, E2, E2.shape[0])
    x += gather_direct(i3, E3, E3.shape[0])
    return x, i2, i3


def ngram_backward(ids, dx, V_real: int, V_pad: int, rows2: int, rows3: int):
    """(dE, dE2, dE3): every existing n-gram's dx row added into its table row."""
    i2, i3 = ngram_ids(ids, V_real, rows2, rows3)
    dE, _ = scatter_add(ids, dx, V_real, V_pad)
    dE2, _ = scatter_add(i2, dx, rows2, rows2)
    dE3, _ = scatter_add(i3, dx, rows3, rows3)
    return dE, dE2, dE3
