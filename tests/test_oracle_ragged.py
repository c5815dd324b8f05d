"""Ragged batches in the oracle: the packed layout against the dense rule.

The dense oracle is pinned by exact enumeration and chi-square elsewhere;
here every request of a ragged batch must equal the dense rule run on that
request's own K_b + 1 rows (same request index, so the same uniforms).
"""
import numpy as np
import pytest

import oracle
from workloads import make, pack_ragged


def pack(wl, ks):
    r = pack_ragged(wl, ks)
    return r["target_rows"], r["draft_rows"], r["cu"], r["draft_tokens"]


@pytest.mark.parametrize("cfg", ["c2_stoch", "c3_onehot"])
def test_ragged_sample_equals_dense_per_request(cfg):
    K = 4
    wl = make(cfg, data_seed=50, B=12, K=K, V=700, offset=3)
    ks = np.random.default_rng(51).integers(0, K + 1, wl["B"])
    ks[0], ks[1] = 0, K
    t_rows, d_rows, cu, toks = pack(wl, ks)
    r_tok, r_len, r_p, r_q, _ = oracle.spec_verify_sample_ragged(
        t_rows, d_rows, cu, toks, wl["temperature"], wl["seeds"], wl["offset"], k_max=K,
        target_dtype=wl["dtype"])
    assert r_tok.shape == (wl["B"], K + 1)
    for k in np.unique(ks):
        reqs = [int(b) for b in np.nonzero(ks == k)[0]]
        d_tok, d_len, d_p, d_q, _ = oracle.spec_verify_sample(
            wl["target"][:, : k + 1], None if wl["draft"] is None else wl["draft"][:, :k],
            wl["draft_tokens"][:, :k], wl["temperature"], wl["seeds"], wl["offset"],
            target_dtype=wl["dtype"], requests=reqs)
        for b in reqs:
            assert r_len[b] == d_len[b]
            np.testing.assert_array_equal(r_tok[b, : k + 1], d_tok[b])
            assert np.all(r_tok[b, k + 1:] == -1)
            np.testing.assert_array_equal(r_p[cu[b]:cu[b + 1]], d_p[b])
            np.testing.assert_array_equal(r_q[cu[b]:cu[b + 1]], d_q[b])


def test_ragged_greedy_equals_dense_per_request():
    K = 5
    wl = make("c4_greedy", data_seed=52, B=16, K=K, V=900)
    ks = np.random.default_rng(53).integers(0, K + 1, wl["B"])
    t_rows, _, cu, toks = pack(wl, ks)
    r_tok, r_len, r_g = oracle.spec_verify_greedy_ragged(t_rows, cu, toks, k_max=K)
    for b in range(wl["B"]):
        k = int(ks[b])
        d_tok, d_len, d_g = oracle.spec_verify_greedy(wl["target"][b:b + 1, : k + 1],
                                                      wl["draft_tokens"][b:b + 1, :k])
        assert r_len[b] == d_len[0]
        np.testing.assert_array_equal(r_tok[b, : k + 1], d_tok[0])
        np.testing.assert_array_equal(r_g[cu[b] + b: cu[b + 1] + b + 1], d_g[0])


def test_ragged_all_zero_drafts_is_plain_sampling():
    wl = make("c3_onehot", data_seed=54, B=6, K=0, V=500)
    t_rows, _, cu, toks = pack(wl, np.zeros(6, np.int64))
    r_tok, r_len, _, _, _ = oracle.spec_verify_sample_ragged(
        t_rows, None, cu, toks, wl["temperature"], wl["seeds"], wl["offset"], k_max=0,
        target_dtype=wl["dtype"])
    d_tok, d_len, _, _, _ = oracle.spec_verify_sample(
        wl["target"], None, wl["draft_tokens"], wl["temperature"], wl["seeds"], wl["offset"],
        target_dtype=wl["dtype"])
    np.testing.assert_array_equal(r_tok, d_tok)
    assert np.all(r_len == 1)


def test_ragged_bad_offsets_refuse_only_their_request():
    K = 3
    wl = make("c2_stoch", data_seed=55, B=5, K=K, V=300)
    ks = np.array([2, 3, 1, 0, 2])
    t_rows, d_rows, cu, toks = pack(wl, ks)
    good = oracle.spec_verify_sample_ragged(t_rows, d_rows, cu, toks, wl["temperature"],
                                            wl["seeds"], wl["offset"], k_max=K)
    bad = cu.copy()
    bad[2] = bad[3] + 1                      # request 1 ends before it starts, request 2 starts after it ends
    out = oracle.spec_verify_sample_ragged(t_rows, d_rows, bad, toks, wl["temperature"],
                                           wl["seeds"], wl["offset"], k_max=K)
    for b in (1, 2):
        assert out[1][b] == 0 and np.all(out[0][b] == -1)
    for b in (0, 3, 4):
        assert out[1][b] == good[1][b]
        np.testing.assert_array_equal(out[0][b], good[0][b])
    # a count above k_max is refused too
    out = oracle.spec_verify_sample_ragged(t_rows, d_rows, cu, toks, wl["temperature"],
                                           wl["seeds"], wl["offset"], k_max=2)
    assert out[1][1] == 0 and out[1][0] == good[1][0]
