"""Philox4x64-10 in plain Python integers (oracle side).

Test infrastructure only, like the rest of ``oracle/``.

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3" (SC'11), the Philox family with W = 64,
N = 4 and R = 10 rounds. One round takes the counter (c0, c1, c2, c3) and
the round key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

where hi/lo are the upper and lower 64 bits of the 128-bit product. The key
is advanced by the Weyl constants (W0, W1) before every round but the first.

The pages ask for counter-based randomness keyed by (seed, request,
position) but name no generator; this one is chosen because it is a
published, stateless bijection and because numpy ships an independent
implementation of it that the tests use as a pin.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15   # frac(golden ratio) * 2^64
PHILOX_W1 = 0xBB67AE8584CAA73B   # frac(sqrt(3)) * 2^64


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for a 4-word counter and 2-word key."""
    c0, c1, c2, c3 = (int(w) & MASK64 for w in counter)
    k0, k1 = (int(w) & MASK64 for w in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((prod1 >> 64) ^ c1 ^ k0, prod1 & MASK64,
                          (prod0 >> 64) ^ c3 ^ k1, prod0 & MASK64)
    return c0, c1, c2, c3


def uniform24(word):
    """Top 24 bits of a 64-bit word as a float in [0, 1), exact in fp32 and fp64."""
    return (int(word) >> 40) * 2.0 ** -24


def request_uniforms(seed, request, position, offset):
    """The two uniforms of one (request, position): (u_accept, u_sample).

    Counter = (position, request, offset, 0), key = (seed, 0); word 0 drives
    the acceptance test and word 1 the residual/bonus draw, so every
    position of every request gets its own independent pair.
    """
    w = philox4x64_10((position, request, offset, 0), (seed, 0))
    return uniform24(w[0]), uniform24(w[1])
