"""Statistical exactness of the oracle at the tiny workload's shape (V=1000, K=1).

10^6 seeded trials (seed = trial index, drafts x ~ q drawn by the test from
its own generator): the first emitted token must follow p_1 and the
completed second token p_2; a joint test over 8^3 cells at V=8, K=2. The
p-value bar is 1e-4 with fixed seeds, so the test is deterministic.
"""
from concurrent.futures import ProcessPoolExecutor
import os

import numpy as np
import pytest

import oracle
from chisq import chisq_pvalue
from workloads import make

N_TRIALS = 1_000_000
WORKERS = min(8, os.cpu_count() or 1)


def _rows_c1():
    wl = make("c1_tiny", data_seed=3)
    T = float(wl["temperature"][0])
    p = [oracle.softmax_t(oracle.logits_f64(wl["target"][0, i], "f32"), T) for i in range(2)]
    q = [oracle.softmax_t(oracle.logits_f64(wl["draft"][0, 0], "f32"), T)]
    return p, q


def _chunk(args):
    lo, hi, p, q, mutate = args
    K = len(q)
    V = len(p[0])
    p_l = [r.tolist() for r in p]
    q_l = [r.tolist() for r in q]
    rng = np.random.default_rng(np.random.PCG64([lo, 99]))
    cdf_q = [np.cumsum(r) for r in q]
    cdf_p = [np.cumsum(r) for r in p]
    counts = np.zeros((K + 1, V), np.int64)
    joint = {}
    for t in range(lo, hi):
        x = [min(int(np.searchsorted(cdf_q[i], rng.random() * cdf_q[i][-1], side="right")), V - 1)
             for i in range(K)]
        pairs = [oracle.request_uniforms(t, 0, i, 0) for i in range(K + 1)]
        if mutate:
            res = oracle.verify_request(p_l, [p_l[0]] * K, x, [u for u, _ in pairs],
                                        [u for _, u in pairs])
        else:
            res = oracle.verify_request(p_l, q_l, x, [u for u, _ in pairs], [u for _, u in pairs])
        seq = list(res["tokens"])
        while len(seq) < K + 1:      # completion with fresh target draws
            j = len(seq)
            seq.append(min(int(np.searchsorted(cdf_p[j], rng.random() * cdf_p[j][-1], side="right")),
                           V - 1))
        for j, y in enumerate(seq):
            counts[j, y] += 1
        if V <= 8:
            key = tuple(seq)
            joint[key] = joint.get(key, 0) + 1
    return counts, joint


def _run(p, q, n, mutate=False):
    step = (n + WORKERS * 4 - 1) // (WORKERS * 4)
    jobs = [(lo, min(n, lo + step), p, q, mutate) for lo in range(0, n, step)]
    counts = None
    joint = {}
    with ProcessPoolExecutor(WORKERS) as ex:
        for c, j in ex.map(_chunk, jobs):
            counts = c if counts is None else counts + c
            for k, v in j.items():
                joint[k] = joint.get(k, 0) + v
    return counts, joint


_chisq_p = chisq_pvalue


@pytest.mark.slow
def test_chisquare_1e6_trials_at_tiny_shape():
    p, q = _rows_c1()
    counts, _ = _run(p, q, N_TRIALS)
    assert counts.sum(axis=1).tolist() == [N_TRIALS, N_TRIALS]
    assert _chisq_p(counts[0], p[0]) > 1e-4
    assert _chisq_p(counts[1], p[1]) > 1e-4


@pytest.mark.slow
def test_chisquare_joint_small_vocab():
    rng = np.random.default_rng(12)
    p = [oracle.softmax_t(rng.normal(0, 1, 8), 1.0) for _ in range(3)]
    q = [oracle.softmax_t(rng.normal(0, 1, 8), 1.0) for _ in range(2)]
    _, joint = _run(p, q, N_TRIALS)
    cells = [(a, b, c) for a in range(8) for b in range(8) for c in range(8)]
    obs = np.array([joint.get(k, 0) for k in cells], float)
    probs = np.array([p[0][a] * p[1][b] * p[2][c] for a, b, c in cells])
    assert _chisq_p(obs, probs / probs.sum()) > 1e-4


def test_chisquare_has_power_against_a_planted_mistake():
    # treat the draft as if it were the target (q := p) while x ~ q: the law drifts to q
    p, q = _rows_c1()
    counts, _ = _run(p, q, 200_000, mutate=True)
    assert _chisq_p(counts[0], p[0]) < 1e-6
