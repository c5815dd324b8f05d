"""Pins of the oracle's top-k / top-p filters (no GPU).

The oracle walks distinct values from the top, accumulating mass. The pins
come at it from elsewhere: a brute-force search over every upper set of the
row, hand-computed small rows, the limits that switch the filter off or
leave one token, and the exact output law of the rule on filtered rows.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import oracle.verify as ov
from exact_law import exact_law


def brute_keep(l, T, top_k, top_p):
    """Try every cut value c (kept = {l >= c}), smallest sets first."""
    l = np.asarray(l, dtype=np.float64)
    V = len(l)
    cuts = sorted(set(l.tolist()), reverse=True)     # largest cut = smallest set
    keep = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        for c in cuts:
            if np.count_nonzero(l >= c) >= top_k:
                keep = l >= c
                break
    if top_p < 1:
        e = np.exp(l / T - np.max(l / T)) * keep
        Z = e.sum()
        for c in cuts:
            s = keep & (l >= c)
            if e[s].sum() / Z >= top_p:
                keep = s
                break
    return keep


@pytest.mark.parametrize("seed", range(40))
def test_filter_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 24))
    l = np.round(rng.normal(0, 2, V), 1)            # coarse values: ties are common
    T = float(rng.choice([0.5, 0.8, 1.3]))
    top_k = int(rng.integers(-1, V + 2))
    top_p = float(rng.choice([0.0, 0.3, 0.7, 0.9, 0.95, 1.0]))
    keep, margin = oracle.filter_keep(l, T, top_k, top_p)
    want = brute_keep(l, T, top_k, top_p)
    if margin > 1e-9:                                  # the two sum in different orders
        np.testing.assert_array_equal(keep, want)


def test_filter_hand_computed():
    # logits ln(p) at T = 1 give p = [0.5, 0.3, 0.15, 0.05]
    l = np.log([0.5, 0.3, 0.15, 0.05])
    row, _ = oracle.filtered_row(l, 1.0, 0, 0.79)     # 0.5 + 0.3 reaches 0.79
    np.testing.assert_allclose(row, [0.625, 0.375, 0, 0], atol=1e-12)
    row, _ = oracle.filtered_row(l, 1.0, 0, 0.81)     # needs the third token
    np.testing.assert_allclose(row, [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0], atol=1e-12)
    row, _ = oracle.filtered_row(l, 1.0, 2, 1.0)      # top-2
    np.testing.assert_allclose(row, [0.625, 0.375, 0, 0], atol=1e-12)
    # top-k first, then top-p on the renormalised top-3: 0.5/0.95 < 0.6 <= 0.8/0.95
    row, _ = oracle.filtered_row(l, 1.0, 3, 0.6)
    np.testing.assert_allclose(row, [0.625, 0.375, 0, 0], atol=1e-12)
    # ties at the top-k cut are all kept
    keep, _ = oracle.filter_keep([3.0, 1.0, 3.0, 2.0, 2.0], 1.0, 3, 1.0)
    np.testing.assert_array_equal(keep, [True, False, True, True, True])


def test_filter_limits():
    rng = np.random.default_rng(5)
    l = rng.normal(0, 2, 50)
    for k, p in [(0, 1.0), (50, 1.0), (-3, 1.0), (60, float("nan"))]:
        keep, margin = oracle.filter_keep(l, 0.8, k, p)
        assert keep.all() and margin == math.inf
    for k, p in [(1, 1.0), (0, 0.0), (0, 1e-9), (7, 1e-12)]:
        keep, _ = oracle.filter_keep(l, 0.8, k, p)
        np.testing.assert_array_equal(keep, l == l.max())


def test_unfiltered_sample_is_unchanged():
    from workloads import make
    wl = make("c2_stoch", data_seed=4, B=6, V=300)
    args = (wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"], wl["seeds"], 2)
    a = oracle.spec_verify_sample(*args)
    b = oracle.spec_verify_sample(*args, top_k=np.zeros(6, np.int32), top_p=np.ones(6, np.float32))
    for x, y in zip(a[:4], b[:4]):
        np.testing.assert_array_equal(x, y)


def _frac_rows(rows):
    out = []
    for r in rows:
        f = [Fraction(v).limit_denominator(1 << 20) for v in r]
        s = sum(f)
        out.append([v / s for v in f])
    return out


@pytest.mark.parametrize("top_k,top_p", [(2, 1.0), (0, 0.7), (3, 0.8)])
def test_filtered_rule_emits_filtered_target(top_k, top_p):
    """The rule run on filtered p and q emits the filtered p (exact enumeration)."""
    rng = np.random.default_rng(11)
    V, K = 4, 2
    lp = rng.normal(0, 1.5, (K + 1, V))
    lq = rng.normal(0, 1.5, (K, V))
    p_rows = _frac_rows([ov.filtered_row(lp[i], 0.9, top_k, top_p)[0] for i in range(K + 1)])
    q_rows = _frac_rows([ov.filtered_row(lq[i], 0.9, top_k, top_p)[0] for i in range(K)])
    law = exact_law(p_rows, q_rows)
    for seq, pr in law.items():
        want = math.prod((p_rows[i][seq[i]] for i in range(K + 1)), start=Fraction(1))
        assert pr == want, (seq, pr, want)


@pytest.mark.parametrize("mutation", ["strict", "before_topk", "keep_below"])
def test_planted_filter_mistakes_fail_brute_force(monkeypatch, mutation):
    """A wrong comparison, top-p before top-k, or a cut one value too low is caught."""
    orig = ov.filter_keep

    def bad(logits, T, top_k=0, top_p=1.0):
        l = np.asarray(logits, dtype=np.float64)
        if mutation == "strict":                    # '>' instead of '>=' at the top-p cut
            keep, m = orig(l, T, top_k, top_p)
            t = l[keep].min() if keep.any() else -math.inf
            return keep & (l > t) if top_p < 1 else keep, m
        if mutation == "before_topk":
            k1, m = orig(l, T, 0, top_p)
            k2, _ = orig(l, T, top_k, 1.0)
            return k1 & k2, m
        keep, m = orig(l, T, top_k, top_p)
        vals = np.unique(l)
        below = vals[vals < l[keep].min()] if keep.any() else vals
        if top_p < 1 and len(below):
            keep = keep | (l == below.max())
        return keep, m
    monkeypatch.setattr(ov, "filter_keep", bad)
    failures = 0
    for seed in range(40):
        rng = np.random.default_rng(seed)
        V = int(rng.integers(3, 24))
        l = np.round(rng.normal(0, 2, V), 1)
        top_k = int(rng.integers(2, V + 1))
        top_p = float(rng.choice([0.3, 0.7, 0.9]))
        keep, _ = ov.filter_keep(l, 1.0, top_k, top_p)
        failures += not np.array_equal(keep, brute_keep(l, 1.0, top_k, top_p))
    assert failures > 0
