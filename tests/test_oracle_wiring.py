"""The batched oracle entry point itself, driven end to end at the tiny shape.

The exact-law and chi-square pins call the decision core with uniforms the
test supplies, so they do not see how ``oracle.spec_verify_sample`` hands
each position its pair of uniforms (word 0 for the acceptance test, word 1
for the draw, per (seed, request, position, offset)). Here the batched call
runs 10^6 requests of the 1000-token workload's rows, broadcast with stride
0 over the batch, each with its own seed (the trial index) and a draft
token x ~ q drawn by the test. The first emitted token must follow p_1 and
the completed second token p_2 ("推测解码与 MTP" §2: the output law equals
the target's). Two planted wiring mistakes must fail the same test: drawing
the replacement with the uniform that just decided the rejection, and
uniforms that ignore the request's seed.
"""
from concurrent.futures import ProcessPoolExecutor
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import oracle.verify as oracle_verify
from chisq import chisq_pvalue
from workloads import make

N_TRIALS = 1_000_000
SUB = 2000                                         # requests per batched oracle call
WORKERS = min(8, os.cpu_count() or 1)


def _c1():
    wl = make("c1_tiny", data_seed=3)
    T = float(wl["temperature"][0])
    # expected laws from scipy's softmax, independent of the oracle's own
    p = [softmax(wl["target"][0, i].astype(np.float64) / T) for i in range(2)]
    q = softmax(wl["draft"][0, 0].astype(np.float64) / T)
    return wl, p, q


def _plant(mutation):
    real = oracle_verify.request_uniforms
    if mutation == "draw_with_accept_uniform":
        oracle_verify.request_uniforms = lambda s, b, i, o: (real(s, b, i, o)[0],) * 2
    elif mutation == "seed_ignored":
        oracle_verify.request_uniforms = lambda s, b, i, o: real(0, b, i, o)
    return real


def _chunk(args):
    lo, hi, mutation = args
    wl, p, q = _c1()
    V = wl["V"]
    rng = np.random.default_rng(np.random.PCG64([lo, 7]))
    cdf_q, cdf_p2 = np.cumsum(q), np.cumsum(p[1])
    counts = np.zeros((2, V), np.int64)
    real = _plant(mutation)
    try:
        for s0 in range(lo, hi, SUB):
            n = min(SUB, hi - s0)
            x = np.minimum(np.searchsorted(cdf_q, rng.random(n) * cdf_q[-1], side="right"), V - 1)
            tgt = np.broadcast_to(wl["target"], (n,) + wl["target"].shape[1:])
            drf = np.broadcast_to(wl["draft"], (n,) + wl["draft"].shape[1:])
            tok, alen, _, _, _ = oracle.spec_verify_sample(
                tgt, drf, x.astype(np.int32).reshape(n, 1), np.broadcast_to(wl["temperature"], (n,)),
                np.arange(s0, s0 + n, dtype=np.uint64), 0)
            second = np.where(alen == 2, tok[:, 1],
                              np.minimum(np.searchsorted(cdf_p2, rng.random(n) * cdf_p2[-1],
                                                         side="right"), V - 1))
            np.add.at(counts[0], tok[:, 0], 1)
            np.add.at(counts[1], second, 1)
    finally:
        oracle_verify.request_uniforms = real
    return counts


def _run(n, mutation=None):
    step = (n + WORKERS * 4 - 1) // (WORKERS * 4)
    jobs = [(lo, min(n, lo + step), mutation) for lo in range(0, n, step)]
    with ProcessPoolExecutor(WORKERS) as ex:
        return sum(ex.map(_chunk, jobs))


@pytest.mark.slow
def test_batched_oracle_law_1e6_requests():
    _, p, _ = _c1()
    counts = _run(N_TRIALS)
    assert counts.sum(axis=1).tolist() == [N_TRIALS, N_TRIALS]
    assert chisq_pvalue(counts[0], p[0]) > 1e-4
    assert chisq_pvalue(counts[1], p[1]) > 1e-4


@pytest.mark.parametrize("mutation", ["draw_with_accept_uniform", "seed_ignored"])
def test_batched_oracle_law_catches_wiring_mistakes(mutation):
    _, p, _ = _c1()
    counts = _run(200_000, mutation)
    assert min(chisq_pvalue(counts[0], p[0]), chisq_pvalue(counts[1], p[1])) < 1e-6
