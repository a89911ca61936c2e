"""Philox4x64-10 counter-based generator, plain Python integers.

TEST INFRASTRUCTURE.  Part of the CPU oracle; only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline may use it.

Definition: Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
as 1, 2, 3" (SC'11), the Philox-4x64 bijection with 10 rounds.  One round maps
the counter words (x0, x1, x2, x3) under the round key (k0, k1) to

    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))

with the 128-bit products split into high and low 64-bit halves, and the key
is bumped by the Weyl constants (W0, W1) between rounds.

How the sampler keys it (the engine seeds one generator with 42 and relies
on every tensor-parallel rank making the same calls; a counter-based
generator gives each request its own stream instead):

    key     = (seed mod 2^64, 0)
    counter = (uid mod 2^64 (two's complement), step mod 2^64, 0, 0)
    u       = (word0 >> 40) * 2^-24          -- 24-bit dyadic in [0, 1)

``u`` is exact in float32 and float64.
"""
from __future__ import annotations

M64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1
ROUNDS = 10


def philox4x64(counter, key, rounds: int = ROUNDS):
    """Philox-4x64 bijection: four 64-bit counter words, two key words."""
    x0, x1, x2, x3 = (int(c) & M64 for c in counter)
    k0, k1 = (int(k) & M64 for k in key)
    for r in range(rounds):
        prod0 = PHILOX_M0 * x0
        prod1 = PHILOX_M1 * x2
        x0, x1, x2, x3 = ((prod1 >> 64) ^ x1 ^ k0, prod1 & M64,
                          (prod0 >> 64) ^ x3 ^ k1, prod0 & M64)
        if r + 1 < rounds:
            k0 = (k0 + PHILOX_W0) & M64
            k1 = (k1 + PHILOX_W1) & M64
    return (x0, x1, x2, x3)


def request_word(seed: int, uid: int, step: int) -> int:
    """First output word of the sampler's stream for (seed, uid, step)."""
    return philox4x64((int(uid) & M64, int(step) & M64, 0, 0), (int(seed) & M64, 0))[0]


def uniform24(word0: int) -> float:
    return float((int(word0) & M64) >> 40) * 2.0 ** -24


def request_uniform(seed: int, uid: int, step: int) -> float:
    return uniform24(request_word(seed, uid, step))
