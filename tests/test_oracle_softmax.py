"""Pins of the oracle's probabilities: library softmax, closed forms, bf16 widening."""
import math

import numpy as np
import pytest
import torch
from scipy import special

from oracle import logits_f64, softmax_t
from workloads import f32_to_bf16_bits


@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_softmax_matches_scipy(T):
    rng = np.random.default_rng(1)
    l = rng.normal(0, 3, size=5000)
    np.testing.assert_allclose(softmax_t(l, T), special.softmax(l / T), rtol=1e-12, atol=1e-300)


def test_uniform_logits_give_uniform_distribution():
    p = softmax_t(np.full(1000, 3.25), 0.7)
    np.testing.assert_allclose(p, 1e-3, rtol=1e-13)


@pytest.mark.parametrize("a,b,T", [(0.0, 1.0, 1.0), (2.0, -3.0, 0.5), (10.0, 10.5, 3.0)])
def test_two_tokens_are_logistic(a, b, T):
    p = softmax_t(np.array([a, b]), T)
    assert p[0] == pytest.approx(1.0 / (1.0 + math.exp((b - a) / T)), rel=1e-14)
    assert p[1] == pytest.approx(1.0 / (1.0 + math.exp((a - b) / T)), rel=1e-14)


def test_shift_invariance_and_masked_entries():
    rng = np.random.default_rng(2)
    l = rng.normal(0, 2, size=300)
    np.testing.assert_allclose(softmax_t(l + 700.0, 0.8), softmax_t(l, 0.8), rtol=1e-9)
    l2 = l.copy()
    l2[::3] = -np.inf
    p = softmax_t(l2, 0.8)
    assert np.all(p[::3] == 0.0)
    np.testing.assert_allclose(p[1::3].sum() + p[2::3].sum(), 1.0, rtol=1e-14)


def test_temperature_is_a_logit_scale():
    rng = np.random.default_rng(3)
    l = rng.normal(0, 2, size=777)
    np.testing.assert_allclose(softmax_t(l, 0.5), softmax_t(2.0 * l, 1.0), rtol=1e-13)


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.normal(0, 3, 4000).astype(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, 3.4e38], np.float32)])
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().double().numpy()
    got = logits_f64(bits, "bf16")
    np.testing.assert_array_equal(got, ref)
    # and the generator's rounding is torch's round-to-nearest-even
    ref_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref_bits)


def test_f32_widening_is_exact():
    x = np.array([1.5, -2.25, 3.0e-38, 1.0e38], np.float32)
    np.testing.assert_array_equal(logits_f64(x, "f32"), x.astype(np.float64))
