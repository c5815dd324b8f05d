"""Exact output law of the oracle's verification rule, by enumeration over Fractions.

Helper for the oracle pins (no GPU, no library code). The rule's outcome is
piecewise constant in each uniform; the pieces are cut at the acceptance
threshold min(1, p/q) and at the CDF boundaries C_j / Z of the draw. Each
piece is evaluated at its midpoint and weighted by its length, and the
oracle is also probed at the piece's left end and just below its right end,
so a threshold placed anywhere other than where the mathematics puts it
makes the probe assertion fail.
"""
from collections import defaultdict
from fractions import Fraction
from itertools import product
import math

import oracle.verify as ov

EPS = Fraction(1, 10**15)


def _pieces(cuts):
    cuts = sorted(set([Fraction(0), Fraction(1)] + [c for c in cuts if 0 < c < 1]))
    return [(lo, hi) for lo, hi in zip(cuts[:-1], cuts[1:]) if hi > lo]


def _cdf_cuts(weights):
    Z = sum(weights)
    run, cuts = Fraction(0), []
    for w in weights:
        run += w
        cuts.append(run / Z)
    return cuts


def _threshold(p, q):
    if q == 0:
        return Fraction(1) if p > 0 else Fraction(0)
    return min(Fraction(1), p / q)


def exact_law(p_rows, q_rows, probe=True):
    """Law of the completed emitted sequence (y_0..y_K) under ``oracle.verify``.

    Drafts x_i ~ q_i independently; after the step ends at length a+1 the
    remaining positions are filled with fresh draws from p_{a+1}..p_K, which
    is what later steps would emit when p does not depend on the prefix.
    """
    K = len(q_rows)
    V = len(p_rows[0])
    half = [Fraction(1, 2)] * (K + 1)
    law = defaultdict(Fraction)
    for x in product(range(V), repeat=K):
        x = list(x)
        wx = math.prod((q_rows[i][x[i]] for i in range(K)), start=Fraction(1))
        if wx == 0:
            continue
        acc_pieces = [_pieces([_threshold(p_rows[i][x[i]], q_rows[i][x[i]])]) for i in range(K)]
        for combo in product(*acc_pieces):
            u_acc = [(lo + hi) / 2 for lo, hi in combo] + [Fraction(1, 2)]
            w_acc = math.prod((hi - lo for lo, hi in combo), start=Fraction(1))
            base = ov.verify_request(p_rows, q_rows, x, u_acc, half)
            a = base["a"]
            if probe:
                for i, (lo, hi) in enumerate(combo):
                    for u in (lo, hi - EPS):
                        ua = list(u_acc)
                        ua[i] = u
                        assert ov.verify_request(p_rows, q_rows, x, ua, half)["a"] == a
            for lo, hi in _pieces(_cdf_cuts(base["weights"])):
                u_s = list(half)
                u_s[a] = (lo + hi) / 2
                res = ov.verify_request(p_rows, q_rows, x, u_acc, u_s)
                if probe:
                    for u in (lo, hi - EPS):
                        u2 = list(u_s)
                        u2[a] = u
                        assert ov.verify_request(p_rows, q_rows, x, u_acc, u2)["tokens"] == res["tokens"]
                emitted = tuple(res["tokens"])
                assert len(emitted) == a + 1 == res["accept_len"]
                for rest in product(range(V), repeat=K - a):
                    pr = math.prod((p_rows[a + 1 + j][rest[j]] for j in range(K - a)),
                                   start=Fraction(1))
                    if pr:
                        law[emitted + rest] += wx * w_acc * (hi - lo) * pr
    return {k: v for k, v in law.items() if v}


def product_law(p_rows):
    """The target's own law over K+1 positions: the product of the p_j."""
    V = len(p_rows[0])
    out = {}
    for y in product(range(V), repeat=len(p_rows)):
        pr = math.prod((p_rows[j][y[j]] for j in range(len(p_rows))), start=Fraction(1))
        if pr:
            out[y] = pr
    return out
