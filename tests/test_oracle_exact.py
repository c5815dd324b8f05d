"""The pages' exactness guarantee, checked on the oracle by exact enumeration.

The correctness subsection under §2 of "推测解码与 MTP" states that the
verified output has exactly the target's distribution. With Fractions and
tiny vocabularies the oracle's full output law is enumerated and must equal
the product of the target distributions, for explicit, one-hot, identical
and partly disjoint drafts. Planted mistakes in the oracle (on the CPU) must
break the equality, which shows the check has power.
"""
from fractions import Fraction
import random

import pytest

import oracle.verify as ov
from exact_law import exact_law, product_law


def rand_dist(rng, V, zeros=0):
    w = [Fraction(rng.randint(1, 9)) for _ in range(V)]
    for j in rng.sample(range(V), zeros):
        w[j] = Fraction(0)
    s = sum(w)
    return [v / s for v in w]


def onehot(V, x):
    return [Fraction(int(j == x)) for j in range(V)]


def cases():
    rng = random.Random(7)
    out = []
    for V in (2, 3, 4):
        for K in (0, 1, 2, 3):
            if V == 4 and K == 3:
                continue
            p = [rand_dist(rng, V) for _ in range(K + 1)]
            q = [rand_dist(rng, V) for _ in range(K)]
            out.append((f"explicit-V{V}-K{K}", p, q))
            if K:
                pz = [rand_dist(rng, V, zeros=1) for _ in range(K + 1)]
                qz = [rand_dist(rng, V, zeros=1) for _ in range(K)]
                out.append((f"zeros-V{V}-K{K}", pz, qz))
                out.append((f"onehot-V{V}-K{K}", p, [onehot(V, rng.randrange(V)) for _ in range(K)]))
                out.append((f"p_eq_q-V{V}-K{K}", p, [list(r) for r in p[:K]]))
    # one K=3 case at V=4 with mixed rows
    p = [rand_dist(rng, 4) for _ in range(4)]
    q = [rand_dist(rng, 4), onehot(4, 2), rand_dist(rng, 4, zeros=2)]
    out.append(("mixed-V4-K3", p, q))
    return out


CASES = cases()


@pytest.mark.parametrize("name,p,q", CASES, ids=[c[0] for c in CASES])
def test_output_law_equals_target_law(name, p, q):
    assert exact_law(p, q) == product_law(p)


def test_law_with_disjoint_support():
    # draft puts mass where the target has none: those drafts are always rejected
    p = [[Fraction(1, 2), Fraction(1, 2), Fraction(0)], [Fraction(1, 3)] * 3]
    q = [[Fraction(0), Fraction(1, 4), Fraction(3, 4)]]
    assert exact_law(p, q) == product_law(p)


_REAL_INVCDF = ov.inverse_cdf


def _mut_residual_is_p(p, q):
    # the replacement drawn from p instead of the residual
    return list(p)


def _mut_residual_sign(p, q):
    # sign error: max(0, q - p)
    w = [qv - pv if qv > pv else 0 * pv for pv, qv in zip(p, q)]
    return w if any(v > 0 for v in w) else list(p)


def _mut_accept_inverted(p_x, q_x, u_acc):
    # acceptance ratio inverted: min(1, q/p)
    a = 0
    for i in range(len(p_x)):
        if u_acc[i] * p_x[i] < q_x[i]:
            a += 1
        else:
            break
    return a


def _mut_invcdf_off_by_one(w, u):
    # draw shifted by one index
    return (_REAL_INVCDF(w, u) + 1) % len(w)


MUTATIONS = {
    "residual_is_p": ("residual_weights", _mut_residual_is_p),
    "residual_sign": ("residual_weights", _mut_residual_sign),
    "accept_inverted": ("accept_length", _mut_accept_inverted),
    "invcdf_off_by_one": ("inverse_cdf", _mut_invcdf_off_by_one),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistakes_break_the_law(monkeypatch, mutation):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(ov, attr, fn)
    broken = 0
    for name, p, q in CASES:
        try:
            law = exact_law(p, q, probe=False)
        except (AssertionError, ZeroDivisionError, IndexError):
            broken += 1
            continue
        if law != product_law(p):
            broken += 1
    assert broken > 0, f"mutation {mutation} went unnoticed"


def test_bonus_row_index_mistake_is_detected(monkeypatch):
    # all drafts accepted must draw from the LAST target row; using row K-1 breaks exactness
    real = ov.verify_request

    def wrong(p_rows, q_rows, x, u_acc, u_smp):
        K = len(x)
        if K and ov.accept_length([p_rows[i][x[i]] for i in range(K)],
                                  [q_rows[i][x[i]] for i in range(K)], u_acc) == K:
            return real(p_rows[:K] + [p_rows[K - 1]], q_rows, x, u_acc, u_smp)
        return real(p_rows, q_rows, x, u_acc, u_smp)

    monkeypatch.setattr(ov, "verify_request", wrong)
    name, p, q = next(c for c in CASES if c[0] == "explicit-V3-K2")
    assert exact_law(p, q, probe=False) != product_law(p)
