"""Pins of the oracle's acceptance test and inverse-CDF draw (§2.1 of "推测解码与 MTP")."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import accept_length, inverse_cdf, residual_weights, verify_request
from workloads import make


def test_accept_when_draft_equals_target():
    rng = np.random.default_rng(5)
    for _ in range(200):
        K = int(rng.integers(1, 6))
        p_x = rng.random(K) + 1e-3
        u = rng.random(K) * (1 - 2**-24)
        assert accept_length(p_x, p_x, u) == K


def test_zero_target_mass_always_rejects_and_zero_draft_mass_accepts():
    assert accept_length([0.0], [0.3], [0.0]) == 0
    assert accept_length([0.2, 0.0], [0.2, 0.5], [0.9, 0.0]) == 1
    assert accept_length([0.2], [0.0], [0.999]) == 1


def test_onehot_threshold_is_p_of_draft_strict():
    p = 0.375
    assert accept_length([p], [1.0], [p - 2**-24]) == 1
    assert accept_length([p], [1.0], [p]) == 0
    assert accept_length([p], [1.0], [p + 2**-24]) == 0


def test_ratio_threshold_is_exact_on_rationals():
    p, q = Fraction(1, 3), Fraction(1, 2)           # threshold 2/3
    assert accept_length([p], [q], [Fraction(2, 3) - Fraction(1, 10**9)]) == 1
    assert accept_length([p], [q], [Fraction(2, 3)]) == 0


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(6)
    for _ in range(300):
        V = int(rng.integers(1, 400))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[int(rng.integers(V))] = 1.0
        for u in rng.random(5) * (1 - 2**-24):
            c = np.cumsum(w)
            ref = int(np.searchsorted(c, u * c[-1], side="right"))
            assert inverse_cdf(w.tolist(), float(u)) == ref


def test_inverse_cdf_interval_probes_and_zero_weights():
    w = [Fraction(0), Fraction(1, 4), Fraction(0), Fraction(1, 2), Fraction(1, 4), Fraction(0)]
    # boundaries 0, 1/4, 3/4, 1: token j owns [C_{j-1}, C_j) of the unit interval
    assert inverse_cdf(w, Fraction(0)) == 1
    assert inverse_cdf(w, Fraction(1, 4) - Fraction(1, 10**9)) == 1
    assert inverse_cdf(w, Fraction(1, 4)) == 3
    assert inverse_cdf(w, Fraction(3, 4)) == 4
    assert inverse_cdf(w, Fraction(1) - Fraction(1, 10**9)) == 4
    # rounding overshoot (u*Z >= Z cannot happen for u < 1 exactly): last positive token
    assert inverse_cdf(w, Fraction(1)) == 4
    rng = np.random.default_rng(7)
    wf = [0.0, 0.3, 0.0, 0.0, 0.2, 0.5, 0.0]
    for u in rng.random(2000):
        assert wf[inverse_cdf(wf, float(u))] > 0


def test_residual_is_positive_part_with_fallback():
    p = [0.5, 0.3, 0.2]
    q = [0.2, 0.5, 0.3]
    np.testing.assert_allclose(residual_weights(p, q), [0.3, 0.0, 0.0])
    assert residual_weights(p, p) == p                   # no mass left: fall back to p
    assert residual_weights(p, [0, 1.0, 0]) == [0.5, 0.0, 0.2]   # one-hot q removes x


def test_marginal_acceptance_is_one_minus_total_variation():
    # P(accept at the first position) = sum_v min(p(v), q(v)) when x ~ q (follows from the rule)
    rng = np.random.default_rng(8)
    V = 50
    p = oracle.softmax_t(rng.normal(0, 1, V), 1.0)
    q = oracle.softmax_t(rng.normal(0, 1, V), 1.0)
    n = 40000
    xs = rng.choice(V, size=n, p=q)
    hits = 0
    for t, x in enumerate(xs):
        ua, _ = oracle.request_uniforms(t, 0, 0, 0)
        hits += accept_length([p[x]], [q[x]], [ua])
    expect = np.minimum(p, q).sum()
    sigma = np.sqrt(expect * (1 - expect) / n)
    assert abs(hits / n - expect) < 4 * sigma


@pytest.mark.parametrize("name", ["c1_tiny", "c2_stoch", "c3_onehot"])
def test_batch_invariants(name):
    wl = make(name, data_seed=11, B=6, V=3000)
    tok, alen, pd, qd, tr = oracle.spec_verify_sample(
        wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"], wl["seeds"],
        wl["offset"], target_dtype=wl["dtype"], keep_trace=True)
    K = wl["K"]
    for b in range(wl["B"]):
        a = alen[b]
        assert 1 <= a <= K + 1
        np.testing.assert_array_equal(tok[b, :a - 1], wl["draft_tokens"][b, :a - 1])
        assert np.all(tok[b, a:] == -1)
        y = tok[b, a - 1]
        assert 0 <= y < wl["V"]
        if a - 1 < K:    # the replacement has positive residual mass
            assert tr[b]["weights"][y] > 0
            if wl["draft"] is None:
                assert y != wl["draft_tokens"][b, a - 1]
        assert np.all((pd[b] >= 0) & (pd[b] <= 1))
    if wl["draft"] is None:
        assert np.all(qd == 1.0)


def test_refused_request_for_bad_temperature():
    wl = make("c1_tiny", data_seed=1)
    T = np.array([0.0], np.float32)
    tok, alen, pd, qd, _ = oracle.spec_verify_sample(wl["target"], wl["draft"], wl["draft_tokens"],
                                                     T, wl["seeds"], 0)
    assert alen[0] == 0 and np.all(tok[0] == -1)


def test_out_of_range_draft_is_rejected():
    p_rows = [[0.5, 0.5], [0.5, 0.5]]
    res = verify_request(p_rows, [oracle.onehot(2, 7)], [7], [0.0, 0.0], [0.1, 0.1])
    assert res["a"] == 0 and res["tokens"] == [0]
