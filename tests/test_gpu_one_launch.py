"""One-launch calls: the row pass and the per-request rule in one grid, the
row pass's results handed over through tagged workspace slots. Checked
against the two-launch path (row pass, then a tail launch) and the fp64
oracle, across workspace reuse by other entry points and shapes.
"""
import os
from contextlib import contextmanager

import numpy as np
import pytest
import torch

import draft_verification_05_amd as sv
import oracle
from parity import assert_report, classify_sample, to_device
from workloads import make

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@contextmanager
def two_launch():
    old = os.environ.get("SPECVERIFY_ONE_LAUNCH")
    os.environ["SPECVERIFY_ONE_LAUNCH"] = "0"
    try:
        yield
    finally:
        if old is None:
            del os.environ["SPECVERIFY_ONE_LAUNCH"]
        else:
            os.environ["SPECVERIFY_ONE_LAUNCH"] = old


def run_sample(wl):
    d = to_device(wl, DEV)
    out = sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["temperature"], d["seeds"],
                                wl["offset"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check_both_paths(wl, name):
    print(f"[case] {name} B={wl['B']} K={wl['K']} V={wl['V']} dtype={wl['dtype']}", flush=True)
    one = run_sample(wl)
    with two_launch():
        two = run_sample(wl)
    for res, path in ((one, "one launch"), (two, "two launches")):
        assert_report(classify_sample(wl, *res), f"{name} ({path})")
    # the two paths merge the same chunk partials in different orders
    np.testing.assert_allclose(one[2], two[2], rtol=0, atol=2e-6)
    np.testing.assert_allclose(one[3], two[3], rtol=0, atol=2e-6)
    same = (one[1] == two[1]) & np.all(one[0] == two[0], axis=1)
    assert same.mean() >= 0.95, f"{name}: {int((~same).sum())} of {len(same)} requests differ"
    print(f"[one-launch] {name}: {int(same.sum())}/{len(same)} requests identical across paths",
          flush=True)


# Calls with draft logits (c2, c1) take the row pass and a residual pass that
# runs the rule on either setting; they stay here as parity cases for that path.
ONE_LAUNCH_SAMPLE = [
    ("c3-onehot-bf16", "c3_onehot", dict(B=48, V=3 * 8192 + 1232)),
    ("c3-onehot-scalar-path", "c3_onehot", dict(B=24, V=2 * 8192 + 777)),
    ("c2-explicit-f32", "c2_stoch", dict(B=20, V=20001)),
    ("c1-tiny", "c1_tiny", {}),
    ("c3-K0", "c3_onehot", dict(B=16, K=0, V=9000)),
    # more chunk partials per lane than one load (rows over 64 chunks)
    ("c3-long-rows", "c3_onehot", dict(B=6, K=1, V=3 * 65536 + 11)),
]


@pytest.mark.parametrize("name,cfg,kw", ONE_LAUNCH_SAMPLE, ids=[c[0] for c in ONE_LAUNCH_SAMPLE])
def test_one_launch_sample_matches_two_launches(name, cfg, kw):
    check_both_paths(make(cfg, data_seed=500, offset=3, **kw), name)


def test_one_launch_greedy_and_tree_bitwise():
    wl = make("c4_greedy", data_seed=501, B=24, V=20001)
    print(f"[case] greedy B=24 K={wl['K']} V=20001", flush=True)
    d = to_device(wl, DEV)
    one = [t.cpu().numpy() for t in sv.spec_verify_greedy(d["target"], d["tokens"])]
    with two_launch():
        two = [t.cpu().numpy() for t in sv.spec_verify_greedy(d["target"], d["tokens"])]
    o_tok, o_len, o_g = oracle.spec_verify_greedy(wl["target"], wl["draft_tokens"], wl["dtype"])
    for a, b in zip(one, two):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(one[0], o_tok)
    np.testing.assert_array_equal(one[1], o_len)
    tw = make("c5_tree", data_seed=502, B=8)
    print(f"[case] tree B=8 N={len(tw['parents'])} V={tw['V']}", flush=True)
    d = to_device(tw, DEV)
    one = [t.cpu().numpy() for t in sv.spec_verify_tree(d["target"], d["tokens"], list(tw["parents"]))]
    with two_launch():
        two = [t.cpu().numpy() for t in sv.spec_verify_tree(d["target"], d["tokens"], list(tw["parents"]))]
    for a, b in zip(one, two):
        np.testing.assert_array_equal(a, b)
    o_tok, o_len, o_best = oracle.spec_verify_tree(tw["target"], tw["draft_tokens"], tw["parents"], tw["dtype"])
    np.testing.assert_array_equal(one[0], o_tok)
    np.testing.assert_array_equal(one[1], o_len)
    np.testing.assert_array_equal(one[2], o_best)


def test_one_launch_after_other_entry_points_share_the_workspace():
    """Other entry points and shapes write the same workspace bytes in other
    layouts between one-launch calls; every one-launch call must still wait
    for its own row pass and match the oracle."""
    a = make("c3_onehot", data_seed=503, B=40, V=2 * 8192 + 100, offset=1)
    b = make("c2_stoch", data_seed=504, B=12, V=9000, offset=2)
    c = make("c4_greedy", data_seed=505, B=16, V=30000)
    for step in range(3):
        print(f"[case] shared workspace, step {step}", flush=True)
        assert_report(classify_sample(a, *run_sample(a)), f"one-hot step {step}")
        d = to_device(b, DEV)
        lazy = sv.spec_verify_sample_lazy(d["target"], d["draft"], d["tokens"], d["temperature"],
                                          d["seeds"], b["offset"])
        top_p = torch.full((b["B"],), 0.9, dtype=torch.float32, device=DEV)
        filt = sv.spec_verify_sample_filtered(d["target"], d["draft"], d["tokens"], d["temperature"],
                                              None, top_p, d["seeds"], b["offset"])
        torch.cuda.synchronize()
        del lazy, filt
        assert_report(classify_sample(b, *run_sample(b)), f"explicit step {step}")
        d = to_device(c, DEV)
        g_tok, g_len, _ = sv.spec_verify_greedy(d["target"], d["tokens"])
        o_tok, o_len, _ = oracle.spec_verify_greedy(c["target"], c["draft_tokens"], c["dtype"])
        np.testing.assert_array_equal(g_tok.cpu().numpy(), o_tok)
        np.testing.assert_array_equal(g_len.cpu().numpy(), o_len)
        # new data in the same shape: the previous call's slots are stale
        a = make("c3_onehot", data_seed=506 + step, B=40, V=2 * 8192 + 100, offset=step)


def test_two_launch_fallback_shapes():
    """Shapes outside the one-launch limits take the two-launch path: more
    rows than the tail's loads hold (explicit drafts, K = 6) and more than
    1024 requests."""
    check_both_paths(make("c2_stoch", data_seed=507, B=8, K=6, V=5000), "explicit K=6")
    wl = make("c3_onehot", data_seed=508, B=1100, K=2, V=3000)
    print("[case] B=1100 K=2 V=3000", flush=True)
    assert_report(classify_sample(wl, *run_sample(wl)), "B=1100")
    # the two-launch tail's serial merge of more than 64 workgroups per row
    wl = make("c3_onehot", data_seed=509, B=2, K=0, V=1 << 20)
    print("[case] two launches, B=2 K=0 V=2^20", flush=True)
    with two_launch():
        res = run_sample(wl)
    assert_report(classify_sample(wl, *res), "two launches, V=2^20")


@contextmanager
def env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    os.environ.update({k: str(v) for k, v in kv.items()})
    try:
        yield
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


def test_repeated_tags_never_match_an_earlier_calls_words():
    """The call tag repeats after 2^23 - 1 calls; the test hook SPECVERIFY_TAG
    gives consecutive calls the same tag, of the same shape with new data and
    of other shapes. The rule's workgroups clear every tagged word they read,
    so each call still waits for its own row pass and matches the oracle."""
    ws_errs = sv.spec_verify_errors(DEV)            # start from a clean count
    assert ws_errs == 0, ws_errs
    shapes = [("c3_onehot", dict(B=64, V=3 * 8192 + 1232)), ("c3_onehot", dict(B=64, V=3 * 8192 + 1232)),
              ("c3_onehot", dict(B=40, K=3, V=9000)), ("c3_onehot", dict(B=64, V=3 * 8192 + 1232))]
    with env(SPECVERIFY_TAG="7ffff0"):
        for i, (cfg, kw) in enumerate(shapes):
            wl = make(cfg, data_seed=520 + i, offset=i, **kw)
            print(f"[case] repeated tag, call {i} B={wl['B']} K={wl['K']} V={wl['V']}", flush=True)
            assert_report(classify_sample(wl, *run_sample(wl)), f"repeated tag call {i}")
            c = make("c4_greedy", data_seed=530 + i, B=16 + 8 * i, V=20000 + 1000 * i)
            d = to_device(c, DEV)
            g_tok, g_len, _ = sv.spec_verify_greedy(d["target"], d["tokens"])
            o_tok, o_len, _ = oracle.spec_verify_greedy(c["target"], c["draft_tokens"], c["dtype"])
            np.testing.assert_array_equal(g_tok.cpu().numpy(), o_tok)
            np.testing.assert_array_equal(g_len.cpu().numpy(), o_len)
    assert sv.spec_verify_errors(DEV) == 0


def test_a_wait_that_gives_up_is_counted():
    """Test hook: the row pass of one request skips its tagged stores, so that
    request's rule gives up after a short bounded wait (every kernel still
    ends). It is refused, the workspace's give-up count reads 1, and every
    other request is unchanged; the next normal call counts nothing."""
    wl = make("c3_onehot", data_seed=540, B=24, V=2 * 8192 + 100, offset=4)
    assert sv.spec_verify_errors(DEV) == 0
    ref = run_sample(wl)
    print("[case] give-up: one request's tagged stores dropped", flush=True)
    with env(SPECVERIFY_DROP_TAGGED_REQUEST=5, SPECVERIFY_SPIN_LIMIT=4096):
        got = run_sample(wl)
    assert sv.spec_verify_errors(DEV) == 1
    assert got[1][5] == 0 and np.all(got[0][5] == -1)
    keep = np.arange(wl["B"]) != 5
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a[keep], b[keep])
    c = make("c4_greedy", data_seed=541, B=16, V=20000)
    d = to_device(c, DEV)
    with env(SPECVERIFY_DROP_TAGGED_REQUEST=3, SPECVERIFY_SPIN_LIMIT=4096):
        g_tok, g_len, _ = sv.spec_verify_greedy(d["target"], d["tokens"])
    g_len = g_len.cpu().numpy()
    assert sv.spec_verify_errors(DEV) == 1 and g_len[3] == 0
    o_tok, o_len, _ = oracle.spec_verify_greedy(c["target"], c["draft_tokens"], c["dtype"])
    np.testing.assert_array_equal(g_len[np.arange(16) != 3], o_len[np.arange(16) != 3])
    assert_report(classify_sample(wl, *run_sample(wl)), "after a give-up")
    assert sv.spec_verify_errors(DEV) == 0
