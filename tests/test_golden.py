"""Hand-worked fixtures from the pages, checked against the oracle."""
from fractions import Fraction
import json
import os

import oracle
from exact_law import exact_law

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_v3():
    g = _load("worked_example_v3.json")
    p = [Fraction(s) for s in g["p"]]
    q = [Fraction(s) for s in g["q"]]
    for x, want in enumerate(g["accept_probability"]):
        want = Fraction(want)
        # the acceptance event is u * q(x) < p(x): just below the threshold accepts, at it rejects
        assert oracle.accept_length([p[x]], [q[x]], [want - Fraction(1, 10**12)]) == (1 if want > 0 else 0)
        if want < 1:
            assert oracle.accept_length([p[x]], [q[x]], [want]) == 0
    w = oracle.residual_weights(p, q)
    Z = sum(w)
    assert [v / Z for v in w] == [Fraction(s) for s in g["residual_normalised"]]
    law = exact_law([p, p], [q])
    first = [sum(v for k, v in law.items() if k[0] == y) for y in range(3)]
    assert first == [Fraction(s) for s in g["first_token_law"]]
