"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Reduced sizes span several 4 KiB chunks (2048 bf16 or 1024 fp32 logits) plus
a ragged tail, in both the 128-bit and the scalar (misaligned) load paths;
the five named workloads run at their full sizes in the launch configuration
the benchmark times. With SV_PARITY_LOG set, every report's counts are
appended to that file as JSON lines.
"""
import numpy as np
import pytest
import torch

import draft_verification_05_amd as sv
import oracle
from chisq import chisq_pvalue
from parity import assert_report, classify_sample, new_report, to_device
from workloads import f32_to_bf16_bits, make, medusa_tree_parents
from workloads import pack_ragged as workloads_pack_ragged

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run_sample(wl, draft_bf16=False, offset=None):
    d = to_device(wl, DEV, draft_bf16=draft_bf16)
    off = wl["offset"] if offset is None else offset
    tok, alen, p, q = sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["temperature"],
                                            d["seeds"], off)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), alen.cpu().numpy(), p.cpu().numpy(), q.cpu().numpy()


def check_sample(wl, name, requests=None, draft_bf16=False):
    print(f"[case] {name} B={wl['B']} K={wl['K']} V={wl['V']} dtype={wl['dtype']}", flush=True)
    if draft_bf16:
        wl = dict(wl, draft=f32_to_bf16_bits(wl["draft"]))
    g = run_sample(wl, draft_bf16=draft_bf16)
    rep = classify_sample(wl, *g, requests=requests, draft_dtype="bf16" if draft_bf16 else "f32")
    assert_report(rep, name)
    return rep


# ---------------------------------------------------------------- sample ---
SAMPLE_REDUCED = [
    # name, workload, overrides
    ("c1-full", "c1_tiny", {}),
    ("c2-ragged", "c2_stoch", dict(B=16, V=3 * 8192 + 1234)),
    ("c2-odd-V-scalar-path", "c2_stoch", dict(B=12, V=20001)),
    ("c2-one-segment", "c2_stoch", dict(B=8, V=777)),
    ("c3-ragged-aligned", "c3_onehot", dict(B=32, V=2 * 8192 + 1232)),
    ("c3-odd-V-scalar-path", "c3_onehot", dict(B=24, V=2 * 8192 + 777)),
    ("c3-K1", "c3_onehot", dict(B=40, K=1, V=9000)),
]


@pytest.mark.parametrize("name,cfg,kw", SAMPLE_REDUCED, ids=[c[0] for c in SAMPLE_REDUCED])
def test_sample_reduced(name, cfg, kw):
    rep = new_report()
    for offset in range(3):
        wl = make(cfg, data_seed=100 + offset, offset=offset, **kw)
        check_sample(wl, f"{name}/off{offset}", requests=None)
        rep["requests"] += wl["B"]


def test_sample_c1_many_offsets():
    wl = make("c1_tiny", data_seed=5)
    d = to_device(wl, DEV)
    rep = new_report()
    for off in range(200):
        tok, alen, p, q = sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["temperature"],
                                                d["seeds"], off)
        w = dict(wl, offset=off)
        classify_sample(w, tok.cpu().numpy(), alen.cpu().numpy(), p.cpu().numpy(), q.cpu().numpy(),
                        report=rep)
    assert_report(rep, "c1 x 200 offsets")


def test_sample_bf16_explicit_draft():
    wl = make("c2_stoch", data_seed=7, B=10, V=8192 + 100)
    wl = dict(wl, target=f32_to_bf16_bits(wl["target"]), dtype="bf16")
    check_sample(wl, "bf16 target + bf16 draft", draft_bf16=True)


def test_sample_K0_is_plain_sampling():
    wl = make("c3_onehot", data_seed=8, B=64, K=0, V=5000)
    check_sample(wl, "K=0")


def test_sample_vocab_one():
    wl = make("c2_stoch", data_seed=9, B=4, K=2, V=1)
    g_tok, g_len, _, _ = run_sample(wl)
    assert np.all(g_len == 3) and np.all(g_tok == 0)


def test_sample_edge_device_values():
    """Refused temperatures, out-of-range drafts, masked logits."""
    wl = make("c3_onehot", data_seed=10, B=16, V=9000)
    T = wl["temperature"].copy()
    T[[1, 2, 3, 4]] = [0.0, -1.0, np.nan, np.inf]
    tok = wl["draft_tokens"].copy()
    tok[5, 0] = -1
    tok[6, 0] = 9000
    tok[7, 2] = 2**31 - 1
    tgt = wl["target"].copy()
    tgt[8, :, ::3] = 0xFF80                    # bf16 -inf: masked vocabulary entries
    wl = dict(wl, temperature=T, draft_tokens=tok, target=tgt)
    check_sample(wl, "edge device values")


def test_sample_broadcast_and_strided_rows():
    """stride_b = 0 (one row set for every request) and rows cut from wider storage."""
    wl = make("c2_stoch", data_seed=11, B=1, K=3, V=10000)
    base = to_device(wl, DEV)
    B = 48
    tgt = base["target"].expand(B, -1, -1)
    drf = base["draft"].expand(B, -1, -1)
    rng = np.random.default_rng(3)
    tokens = rng.integers(0, 10000, size=(B, 3)).astype(np.int32)
    seeds = rng.integers(0, 2**62, size=B).astype(np.uint64)
    temp = np.full(B, 0.8, np.float32)
    g = sv.spec_verify_sample(tgt, drf, torch.from_numpy(tokens).to(DEV), torch.from_numpy(temp).to(DEV),
                              torch.from_numpy(seeds.view(np.int64)).to(DEV), 3)
    g = [t.cpu().numpy() for t in g]
    wlb = dict(wl, B=B, target=np.broadcast_to(wl["target"], (B, 4, 10000)),
               draft=np.broadcast_to(wl["draft"], (B, 3, 10000)), draft_tokens=tokens, seeds=seeds,
               temperature=temp, offset=3)
    assert_report(classify_sample(wlb, *g), "stride_b=0")
    # rows inside wider storage: stride_k > V
    wide = make("c3_onehot", data_seed=12, B=8, V=12000)
    store = np.zeros((8, 6, 12345), np.uint16)
    store[:, :, :12000] = wide["target"]
    dt = torch.from_numpy(store.view(np.int16)).to(DEV).view(torch.bfloat16)[:, :, :12000]
    d = to_device(wide, DEV)
    out = sv.spec_verify_sample(dt, None, d["tokens"], d["temperature"], d["seeds"], 0)
    assert_report(classify_sample(wide, *[t.cpu().numpy() for t in out]), "stride_k > V")


def test_sample_deterministic_and_workspace_reuse():
    big = make("c3_onehot", data_seed=13, B=64, V=20000)
    small = make("c2_stoch", data_seed=14, B=3, V=5000)
    r1 = run_sample(big)
    run_sample(small)
    r2 = run_sample(big)
    for a, b in zip(r1, r2):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("cfg", ["c2_stoch", "c3_onehot"])
def test_sample_full_size(cfg):
    wl = make(cfg, data_seed=1)
    check_sample(wl, f"{cfg} full")


def test_gpu_chisquare_exactness():
    """10^6 GPU draws at the tiny workload's shape follow the target law."""
    wl = make("c1_tiny", data_seed=3)
    T = float(wl["temperature"][0])
    p0 = oracle.softmax_t(oracle.logits_f64(wl["target"][0, 0], "f32"), T)
    p1 = oracle.softmax_t(oracle.logits_f64(wl["target"][0, 1], "f32"), T)
    q0 = oracle.softmax_t(oracle.logits_f64(wl["draft"][0, 0], "f32"), T)
    d = to_device(wl, DEV)
    B, calls = 65536, 16
    tgt = d["target"].expand(B, -1, -1)
    drf = d["draft"].expand(B, -1, -1)
    temp = torch.full((B,), T, dtype=torch.float32, device=DEV)
    rng = np.random.default_rng(77)
    c0 = np.zeros(1000, np.int64)
    c1 = np.zeros(1000, np.int64)
    cq, cp1 = np.cumsum(q0), np.cumsum(p1)
    for call in range(calls):
        x = np.minimum(np.searchsorted(cq, rng.random(B) * cq[-1], side="right"), 999).astype(np.int32)
        seeds = rng.integers(0, 2**62, size=B).astype(np.int64)
        tok, alen, _, _ = sv.spec_verify_sample(tgt, drf, torch.from_numpy(np.ascontiguousarray(x[:, None])).to(DEV), temp,
                                                torch.from_numpy(seeds).to(DEV), call)
        tok = tok.cpu().numpy()
        alen = alen.cpu().numpy()
        first = tok[:, 0]
        second = np.where(alen == 2, tok[:, 1],
                          np.minimum(np.searchsorted(cp1, rng.random(B) * cp1[-1], side="right"), 999))
        c0 += np.bincount(first, minlength=1000)
        c1 += np.bincount(second, minlength=1000)

    pval = chisq_pvalue
    p_first, p_second = pval(c0, p0), pval(c1, p1)
    print(f"[chisq] gpu first-token p={p_first:.3g} second-token p={p_second:.3g}", flush=True)
    assert p_first > 1e-4 and p_second > 1e-4


# ---------------------------------------------------------------- greedy ---
def check_greedy(wl, name):
    print(f"[case] {name} B={wl['B']} K={wl['K']} V={wl['V']} dtype={wl['dtype']}", flush=True)
    d = to_device(wl, DEV)
    tok, alen, g = sv.spec_verify_greedy(d["target"], d["tokens"])
    torch.cuda.synchronize()
    o_tok, o_len, o_g = oracle.spec_verify_greedy(wl["target"], wl["draft_tokens"], wl["dtype"])
    np.testing.assert_array_equal(g.cpu().numpy(), o_g)
    np.testing.assert_array_equal(alen.cpu().numpy(), o_len)
    np.testing.assert_array_equal(tok.cpu().numpy(), o_tok)
    print(f"[parity] {name}: exact, mean accept_len={o_len.mean():.3f}", flush=True)


@pytest.mark.parametrize("V", [1, 100, 8192, 3 * 8192 + 5, 20001])
def test_greedy_reduced(V):
    check_greedy(make("c4_greedy", data_seed=20, B=16, V=V), f"greedy V={V}")


def test_greedy_bf16_ties():
    wl = make("c4_greedy", data_seed=21, B=24, K=4, V=9000)
    x = np.round(wl["target"] * 2) / 2             # coarse values: many exact ties
    bits = f32_to_bf16_bits(x.astype(np.float32))
    bits[3, :, :] = f32_to_bf16_bits(np.float32(1.0))   # an all-equal row: index 0 wins
    bits[4, 1, :] = 0xFF80                                 # an all -inf row: index 0 wins
    vals = oracle.logits_f64(bits.reshape(-1), "bf16").reshape(bits.shape)
    am = vals.argmax(-1)
    tok = np.where(np.random.default_rng(1).random((24, 4)) < 0.8, am[:, :4], 5).astype(np.int32)
    tok[0, 0] = -7
    check_greedy(dict(wl, target=bits, dtype="bf16", draft_tokens=tok, K=4), "greedy bf16 ties")


def test_greedy_full_size():
    check_greedy(make("c4_greedy", data_seed=1), "c4 full")


# ------------------------------------------------------------------ tree ---
def check_tree(wl, parents, name):
    print(f"[case] {name} B={wl['B']} N={len(parents)} V={wl['V']}", flush=True)
    d = to_device(wl, DEV)
    tok, alen, best = sv.spec_verify_tree(d["target"], d["tokens"], list(parents))
    torch.cuda.synchronize()
    o_tok, o_len, o_best = oracle.spec_verify_tree(wl["target"], wl["draft_tokens"], parents, wl["dtype"])
    np.testing.assert_array_equal(best.cpu().numpy(), o_best)
    np.testing.assert_array_equal(alen.cpu().numpy(), o_len)
    np.testing.assert_array_equal(tok.cpu().numpy(), o_tok)
    print(f"[parity] {name}: exact, accept_len histogram={np.bincount(o_len).tolist()}", flush=True)


def test_tree_full_size():
    wl = make("c5_tree", data_seed=1)
    check_tree(wl, wl["parents"], "c5 full")


@pytest.mark.parametrize("seed", range(4))
def test_tree_random_shapes(seed):
    rng = np.random.default_rng(300 + seed)
    N = int(rng.choice([2, 5, 31, 64]))
    parents = np.array([-1] + [int(rng.integers(0, n)) for n in range(1, N)], np.int32)
    B, V = 20, int(rng.choice([7, 9000, 20001]))
    tgt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    g = tgt.argmax(-1)
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    for n in range(1, N):                    # make acceptance likely along some edges
        hit = rng.random(B) < 0.7
        tok[hit, n] = g[hit, parents[n]]
    wl = dict(target=tgt, draft_tokens=tok, B=B, V=V, dtype="f32", seeds=np.zeros(B, np.uint64))
    check_tree(wl, parents, f"tree N={N} V={V}")


@pytest.mark.parametrize("one_launch", ["1", "0"])
def test_tree_dynamic_per_request(one_launch, monkeypatch):
    """A tree per request (dynamic trees): random trees of N = 31 nodes, two
    rows that are not trees (refused alone), against the oracle; then every
    row the same tree, bitwise equal to the static call. One launch and two."""
    monkeypatch.setenv("SPECVERIFY_ONE_LAUNCH", one_launch)
    rng = np.random.default_rng(320)
    B, N, V = 24, 31, 9000
    parents = np.array([[-1] + [int(rng.integers(0, n)) for n in range(1, N)] for _ in range(B)], np.int32)
    parents[5, 0] = 3
    parents[17, 20] = 25
    tgt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    g = tgt.argmax(-1)
    tok = rng.integers(0, V, (B, N)).astype(np.int32)
    for b in range(B):                       # make acceptance likely along some edges
        for n in range(1, N):
            if rng.random() < 0.7 and 0 <= parents[b, n] < N:
                tok[b, n] = g[b, parents[b, n]]
    print(f"[case] dynamic trees one_launch={one_launch} B={B} N={N} V={V}", flush=True)
    d_tgt = torch.from_numpy(tgt).to(DEV)
    d_tok = torch.from_numpy(tok).to(DEV)
    d_par = torch.from_numpy(parents).to(DEV)
    out = sv.spec_verify_tree(d_tgt, d_tok, d_par)
    torch.cuda.synchronize()
    o_tok, o_len, o_best = oracle.spec_verify_tree(tgt, tok, parents)
    np.testing.assert_array_equal(out[2].cpu().numpy(), o_best)
    np.testing.assert_array_equal(out[1].cpu().numpy(), o_len)
    np.testing.assert_array_equal(out[0].cpu().numpy(), o_tok)
    assert o_len[5] == 0 and o_len[17] == 0
    shared = parents[0]
    dyn = sv.spec_verify_tree(d_tgt, d_tok, torch.from_numpy(np.tile(shared, (B, 1))).to(DEV))
    sta = sv.spec_verify_tree(d_tgt, d_tok, list(shared))
    torch.cuda.synchronize()
    for x, y in zip(dyn, sta):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
    print(f"[parity] dynamic trees one_launch={one_launch}: exact, accept_len histogram="
          f"{np.bincount(o_len).tolist()}", flush=True)


def test_chain_tree_equals_greedy_on_gpu():
    wl = make("c4_greedy", data_seed=22, B=16, K=5, V=10000)
    d = to_device(wl, DEV)
    g_tok, g_len, _ = sv.spec_verify_greedy(d["target"], d["tokens"])
    node_tok = torch.cat([torch.full((16, 1), -1, dtype=torch.int32, device=DEV), d["tokens"]], 1).contiguous()
    t_tok, t_len, best = sv.spec_verify_tree(d["target"], node_tok, list(range(-1, 5)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t_len.cpu().numpy(), g_len.cpu().numpy())
    np.testing.assert_array_equal(t_tok.cpu().numpy(), g_tok.cpu().numpy())


# ------------------------------------------- numerical stress, merge paths ---
def test_sample_low_temperature_recounts():
    """T = 0.05 turns N(0, 2) logits into scaled logits that span about +-170
    (log2 units): most chunks hold logits more than 64 above a lane's first
    vector, so the row pass recounts them against a raised reference."""
    wl = make("c3_onehot", data_seed=30, B=16, V=2 * 8192 + 1232)
    T = np.full(16, 0.05, np.float32)
    T[::3] = 0.02
    check_sample(dict(wl, temperature=T), "c3 T=0.05")
    # explicit drafts are redrawn from q at the new temperature (Gumbel-max),
    # as the method assumes: x ~ q
    wl2 = make("c2_stoch", data_seed=31, B=12, V=20001)
    T2 = np.full(12, 0.05, np.float32)
    y = oracle.logits_f64(wl2["draft"].reshape(-1), "f32").reshape(wl2["draft"].shape) / 0.05
    tok2 = np.argmax(y + np.random.default_rng(39).gumbel(size=y.shape), -1).astype(np.int32)
    check_sample(dict(wl2, temperature=T2, draft_tokens=tok2), "c2 T=0.05 explicit")


def test_sample_explicit_underflowing_probabilities():
    """Drafts whose target and draft probabilities both lie far below the
    fp32 range (e^-100, e^-110): the acceptance must follow the ratio p / q
    (e^10: always accept; e^-0.5: accept when u < 0.61), not the underflowed
    values."""
    B, K, V = 8, 2, 3000
    wl = make("c2_stoch", data_seed=40, B=B, K=K, V=V)
    rng = np.random.default_rng(41)
    tgt = rng.normal(0, 1, (B, K + 1, V)).astype(np.float32)
    drf = rng.normal(0, 1, (B, K, V)).astype(np.float32)
    tok = rng.integers(0, V, (B, K)).astype(np.int32)
    for b in range(B):
        for i in range(K):
            tgt[b, i, tok[b, i]] = -100.0
            drf[b, i, tok[b, i]] = -110.0 if b % 2 == 0 else -99.5
    wl = dict(wl, target=tgt, draft=drf, draft_tokens=tok, temperature=np.ones(B, np.float32))
    rep = check_sample(wl, "explicit underflow")
    g_tok, g_len, _, _ = run_sample(wl)
    assert np.all(g_len[0::2] == K + 1)            # ratio e^10: every draft accepted


def test_sample_huge_logit_spreads():
    """Rows built to break a running reference: ramps over +-300, isolated
    spikes 150 above the rest, whole -inf vectors before finite logits, a
    row offset by -1000, and -200 / +200 blocks inside and across lanes."""
    B, V = 8, 9000
    wl = make("c3_onehot", data_seed=32, B=B, V=V)
    rng = np.random.default_rng(33)
    x = rng.normal(0, 2, (B, 6, V))
    x[0] = -300.0 + 600.0 * np.arange(V) / V
    spikes = rng.integers(0, V, (6, 5))
    for r in range(6):
        x[1, r, spikes[r]] = 150.0
    x[2, :, :2048] = -np.inf
    x[3, :, :512] = -np.inf
    x[3, :, 600] = 100.0
    x[4] = -1000.0 + rng.normal(0, 2, (6, V))
    # 512-logit blocks: a lane's first vector is -200 and its second +200
    x[5] = np.where((np.arange(V) // 512) % 2 == 0, -200.0, 200.0) + rng.normal(0, 1, (6, V))
    x[6, :, : V // 2] = -np.inf
    # 8-logit blocks: neighbouring lanes alternate -200 / +200
    x[7] = np.where((np.arange(V) // 8) % 2 == 0, -200.0, 200.0) + rng.normal(0, 1, (6, V))
    bits = f32_to_bf16_bits(x.astype(np.float32))
    tok = wl["draft_tokens"].copy()
    tok[1, :] = spikes[:5, 0]                      # drafts on the spikes: p near 1
    tok[5, :] = 600                                # inside a +200 block
    check_sample(dict(wl, target=bits, draft_tokens=tok, temperature=np.ones(B, np.float32)),
                 "c3 huge spreads")


def test_merge_serial_fallback_many_rows():
    """33 rows with 32 workgroups each need 17 staged loads per lane, more
    than the tail's 8: the row merges take the serial path."""
    check_greedy(make("c4_greedy", data_seed=34, B=2, K=32, V=131072), "greedy K=32 V=131072")
    wl = make("c3_onehot", data_seed=35, B=2, K=32, V=262144)
    check_sample(wl, "c3 K=32 V=262144")


def test_merge_serial_fallback_wide_rows():
    """A 2^20-logit vocabulary: more than 64 workgroups per row."""
    wl = make("c3_onehot", data_seed=36, B=2, K=0, V=1 << 20)
    check_sample(wl, "c3 K=0 V=2^20")
    check_greedy(make("c4_greedy", data_seed=37, B=2, K=1, V=1 << 20), "greedy K=1 V=2^20")


def test_tree_deep_chain():
    """A 64-node chain: acceptance settles over 63 depth levels."""
    N, B, V = 64, 8, 5000
    rng = np.random.default_rng(38)
    parents = np.arange(-1, N - 1, dtype=np.int32)
    tgt = rng.normal(0, 1, (B, N, V)).astype(np.float32)
    g = tgt.argmax(-1)
    tok = np.empty((B, N), np.int32)
    tok[:, 0] = -1
    tok[:, 1:] = g[:, :-1]                          # every node accepted ...
    for b in range(B):                              # ... up to a per-request break
        cut = int(rng.integers(1, N + 8))
        if cut < N:
            tok[b, cut] = (g[b, cut - 1] + 1) % V
    wl = dict(target=tgt, draft_tokens=tok, B=B, V=V, dtype="f32", seeds=np.zeros(B, np.uint64))
    check_tree(wl, parents, "tree chain N=64")


# ---------------------------------------------------------------- ragged ---
def pack_ragged(wl, ks):
    r = workloads_pack_ragged(wl, ks)
    return r["target_rows"], r["draft_rows"], r["cu"], r["draft_tokens"]


def run_ragged(wl, ks, K, cu=None):
    t_rows, d_rows, cu0, toks = pack_ragged(wl, ks)
    cu = cu0 if cu is None else cu
    bf16 = wl["dtype"] == "bf16"
    tt = torch.from_numpy(t_rows.view(np.int16) if bf16 else t_rows).to(DEV)
    tt = tt.view(torch.bfloat16) if bf16 else tt
    dd = None if d_rows is None else torch.from_numpy(np.ascontiguousarray(d_rows)).to(DEV)
    out = sv.spec_verify_sample_ragged(
        tt, dd, torch.from_numpy(cu).to(DEV), torch.from_numpy(toks).to(DEV),
        torch.from_numpy(wl["temperature"]).to(DEV),
        torch.from_numpy(wl["seeds"].view(np.int64)).to(DEV), wl["offset"], k_max=K)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out], cu0


@pytest.mark.parametrize("cfg,K,V", [("c3_onehot", 5, 2 * 8192 + 1232), ("c2_stoch", 3, 20001),
                                     ("c2_stoch", 4, 8192)])
def test_ragged_sample(cfg, K, V):
    B = 24
    wl = make(cfg, data_seed=60, B=B, K=K, V=V, offset=2)
    ks = np.random.default_rng(61).integers(0, K + 1, B)
    ks[:3] = [0, K, 0]
    (g_tok, g_len, g_p, g_q), cu = run_ragged(wl, ks, K)
    print(f"[case] ragged {cfg} B={B} K_max={K} V={V} ks={ks.tolist()}", flush=True)
    for b in range(B):
        assert np.all(g_tok[b, ks[b] + 1:] == -1)
    rep = new_report()
    for k in np.unique(ks):
        reqs = [int(b) for b in np.nonzero(ks == k)[0]]
        wl_k = dict(wl, K=int(k), target=wl["target"][:, : k + 1],
                    draft=None if wl["draft"] is None else wl["draft"][:, :k],
                    draft_tokens=np.ascontiguousarray(wl["draft_tokens"][:, :k]))
        tok_k = np.full((B, k + 1), -1, np.int32)
        p_k = np.zeros((B, k), np.float32)
        q_k = np.zeros((B, k), np.float32)
        for b in reqs:
            tok_k[b] = g_tok[b, : k + 1]
            p_k[b] = g_p[cu[b]:cu[b + 1]]
            q_k[b] = g_q[cu[b]:cu[b + 1]]
        classify_sample(wl_k, tok_k, g_len, p_k, q_k, requests=reqs, report=rep)
    assert_report(rep, f"ragged {cfg} V={V}")


def test_ragged_full_counts_equal_dense_bitwise():
    wl = make("c3_onehot", data_seed=62, B=16, K=5, V=9000)
    (r_tok, r_len, r_p, r_q), _ = run_ragged(wl, np.full(16, 5), 5)
    d_tok, d_len, d_p, d_q = run_sample(wl)
    np.testing.assert_array_equal(r_tok, d_tok)
    np.testing.assert_array_equal(r_len, d_len)
    np.testing.assert_array_equal(r_p, d_p.reshape(-1))
    np.testing.assert_array_equal(r_q, d_q.reshape(-1))


def test_ragged_bad_offsets_refuse_only_their_request():
    K = 3
    wl = make("c2_stoch", data_seed=63, B=6, K=K, V=5000)
    ks = np.array([2, 3, 1, 0, 2, 3])
    (good_tok, good_len, _, _), cu = run_ragged(wl, ks, K)
    bad = cu.copy()
    bad[2] = bad[3] + 1                            # request 1: K_b > K_max; request 2: out of order
    bad[5] = 10**6                                 # requests 4 and 5: beyond total_k
    (tok, alen, _, _), _ = run_ragged(wl, ks, K, cu=bad)
    for b in (1, 2, 4, 5):
        assert alen[b] == 0 and np.all(tok[b] == -1), b
    for b in (0, 3):
        assert alen[b] == good_len[b]
        np.testing.assert_array_equal(tok[b], good_tok[b])


def test_ragged_greedy():
    K = 5
    wl = make("c4_greedy", data_seed=64, B=20, K=K, V=3 * 8192 + 5)
    ks = np.random.default_rng(65).integers(0, K + 1, 20)
    t_rows, _, cu, toks = pack_ragged(wl, ks)
    tok, alen, g = sv.spec_verify_greedy_ragged(torch.from_numpy(t_rows).to(DEV),
                                                torch.from_numpy(cu).to(DEV),
                                                torch.from_numpy(toks).to(DEV), k_max=K)
    torch.cuda.synchronize()
    o_tok, o_len, o_g = oracle.spec_verify_greedy_ragged(t_rows, cu, toks, k_max=K)
    np.testing.assert_array_equal(g.cpu().numpy(), o_g)
    np.testing.assert_array_equal(alen.cpu().numpy(), o_len)
    np.testing.assert_array_equal(tok.cpu().numpy(), o_tok)
    print(f"[parity] ragged greedy: exact, ks={ks.tolist()}", flush=True)


# --------------------------------------------------------- grammar masks ---
def pack_bits(allowed):
    """uint32 words (bit v % 32 of word v // 32) from a boolean [B, R, V] array."""
    B, R, V = allowed.shape
    W = (V + 31) // 32
    pad = np.zeros((B, R, W * 32), bool)
    pad[..., :V] = allowed
    by = np.packbits(pad.reshape(B, R, W, 4, 8), axis=-1, bitorder="little")[..., 0]
    return np.ascontiguousarray(by).view("<u4").reshape(B, R, W).astype(np.uint32)


def grammar_mask(rng, B, R, V, kind):
    if kind == "dense":
        allowed = rng.random((B, R, V)) < 0.3
    else:                                          # a few hundred allowed tokens, clustered
        allowed = np.zeros((B, R, V), bool)
        for b in range(B):
            for r in range(R):
                starts = rng.integers(0, V, 6)
                for s in starts:
                    allowed[b, r, s: s + rng.integers(10, 60)] = True
    allowed[..., rng.integers(0, V)] = True
    return allowed


def run_masked(wl, mask):
    d = to_device(wl, DEV)
    out = sv.spec_verify_sample_masked(d["target"], d["draft"], d["tokens"],
                                       torch.from_numpy(mask.view(np.int32)).to(DEV),
                                       d["temperature"], d["seeds"], wl["offset"])
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


@pytest.mark.parametrize("cfg,V,kind", [("c3_onehot", 2 * 8192 + 1232, "dense"),
                                        ("c3_onehot", 20001, "sparse"),
                                        ("c2_stoch", 3 * 8192 + 1234, "dense"),
                                        ("c2_stoch", 20001, "sparse")])
def test_masked_sample(cfg, V, kind):
    rng = np.random.default_rng(80)
    wl = make(cfg, data_seed=81, B=16, V=V)
    R = wl["K"] + 1
    allowed = grammar_mask(rng, 16, R, V, kind)
    tok = wl["draft_tokens"].copy()
    for b in range(16):                            # drafts on allowed tokens, a few on disallowed ones
        for i in range(wl["K"]):
            ok = np.nonzero(allowed[b, i])[0]
            tok[b, i] = ok[rng.integers(0, len(ok))] if b % 4 else tok[b, i]
    wl = dict(wl, draft_tokens=tok)
    mask = pack_bits(allowed)
    print(f"[case] masked {cfg} V={V} {kind}", flush=True)
    g = run_masked(wl, mask)
    for b in range(16):
        for i in range(g[1][b]):
            assert allowed[b, i, g[0][b, i]]
    rep = classify_sample(wl, *g, bitmask=mask)
    assert_report(rep, f"masked {cfg} V={V} {kind}")


def test_masked_all_ones_equals_unmasked_bitwise():
    wl = make("c2_stoch", data_seed=82, B=12, V=9000)
    ones = np.full((12, 4, (9000 + 31) // 32), 0xFFFFFFFF, np.uint32)
    for a, b in zip(run_masked(wl, ones), run_sample(wl)):
        np.testing.assert_array_equal(a, b)


def test_masked_greedy():
    rng = np.random.default_rng(83)
    wl = make("c4_greedy", data_seed=84, B=16, V=3 * 8192 + 5)
    allowed = grammar_mask(rng, 16, wl["K"] + 1, wl["V"], "sparse")
    mask = pack_bits(allowed)
    d = to_device(wl, DEV)
    tok, alen, g = sv.spec_verify_greedy_masked(d["target"], d["tokens"],
                                                torch.from_numpy(mask.view(np.int32)).to(DEV))
    torch.cuda.synchronize()
    o_tok, o_len, o_g = oracle.spec_verify_greedy(wl["target"], wl["draft_tokens"], bitmask=mask)
    np.testing.assert_array_equal(g.cpu().numpy(), o_g)
    np.testing.assert_array_equal(alen.cpu().numpy(), o_len)
    np.testing.assert_array_equal(tok.cpu().numpy(), o_tok)


def test_masked_full_size_c3():
    rng = np.random.default_rng(85)
    wl = make("c3_onehot", data_seed=2)
    allowed = rng.random((wl["B"], wl["K"] + 1, wl["V"])) < 0.5
    mask = pack_bits(allowed)
    g = run_masked(wl, mask)
    reqs = list(rng.choice(wl["B"], 32, replace=False))
    rep = classify_sample(wl, *g, requests=reqs, bitmask=mask)
    assert_report(rep, "masked c3 full size (32 sampled requests)")


# ------------------------------------------------------------ early exit ---
def run_lazy(wl, offset=None):
    d = to_device(wl, DEV)
    off = wl["offset"] if offset is None else offset
    out = sv.spec_verify_sample_lazy(d["target"], d["draft"], d["tokens"], d["temperature"],
                                     d["seeds"], off)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


LAZY_REDUCED = [
    ("c3-ragged-aligned", "c3_onehot", dict(B=32, V=2 * 8192 + 1232)),
    ("c3-odd-V-scalar-path", "c3_onehot", dict(B=24, V=2 * 8192 + 777)),
    ("c3-K1", "c3_onehot", dict(B=40, K=1, V=9000)),
    ("c3-K0", "c3_onehot", dict(B=16, K=0, V=5000)),
    ("c2-ragged", "c2_stoch", dict(B=16, V=3 * 8192 + 1234)),
    ("c2-odd-V-scalar-path", "c2_stoch", dict(B=12, V=20001)),
    ("c1-full", "c1_tiny", {}),
]


@pytest.mark.parametrize("name,cfg,kw", LAZY_REDUCED, ids=[c[0] for c in LAZY_REDUCED])
def test_lazy_sample(name, cfg, kw):
    for offset in range(3):
        wl = make(cfg, data_seed=300 + offset, offset=offset, **kw)
        print(f"[case] lazy {name}/off{offset} B={wl['B']} K={wl['K']} V={wl['V']}", flush=True)
        g = run_lazy(wl)
        assert_report(classify_sample(wl, *g, lazy=True), f"lazy {name}/off{offset}")


def test_lazy_edge_device_values():
    """Refused temperatures and out-of-range drafts stop a request in the first rounds."""
    wl = make("c3_onehot", data_seed=310, B=16, V=9000)
    T = wl["temperature"].copy()
    T[[1, 2, 3, 4]] = [0.0, -1.0, np.nan, np.inf]
    tok = wl["draft_tokens"].copy()
    tok[5, 0] = -1
    tok[6, 3] = 9000
    wl = dict(wl, temperature=T, draft_tokens=tok)
    print("[case] lazy edge values", flush=True)
    assert_report(classify_sample(wl, *run_lazy(wl), lazy=True), "lazy edge values")


def test_lazy_all_accepted_and_first_rejected():
    """Drafts equal to the target's mode at low temperature run every round; drafts the
    target gives no mass stop in round 0."""
    wl = make("c3_onehot", data_seed=311, B=24, V=9000)
    tgt = wl["target"].copy()
    tok = wl["draft_tokens"].copy()
    hi = f32_to_bf16_bits(np.array([60.0], np.float32))[0]
    for b in range(12):                             # mode = draft token, sharp target
        tgt[b, np.arange(wl["K"]), tok[b]] = hi
    for b in range(12, 24):                         # draft token masked out of the target
        tgt[b, 0, tok[b, 0]] = 0xFF80
    wl = dict(wl, target=tgt, temperature=np.full(24, 0.25, np.float32))
    g = run_lazy(wl)
    print("[case] lazy all-accepted / first-rejected", flush=True)
    assert_report(classify_sample(wl, *g, lazy=True), "lazy extremes")
    assert np.all(g[1][:12] == wl["K"] + 1) and np.all(g[1][12:] == 1)


@pytest.mark.parametrize("cfg", ["c2_stoch", "c3_onehot"])
def test_lazy_full_size(cfg):
    wl = make(cfg, data_seed=1)
    print(f"[case] lazy {cfg} full", flush=True)
    assert_report(classify_sample(wl, *run_lazy(wl), lazy=True), f"lazy {cfg} full")


def test_lazy_agrees_with_dense_and_reuses_workspace():
    """Same uniforms as the dense rule: tokens agree with it wherever neither side sits at a
    decision boundary, and interleaved dense / lazy calls do not disturb one another."""
    wl = make("c3_onehot", data_seed=312, B=64, V=20000)
    d1 = run_sample(wl)
    l1 = run_lazy(wl)
    d2 = run_sample(wl)
    l2 = run_lazy(wl)
    for a, b in zip(d1, d2):
        np.testing.assert_array_equal(a, b)
    for a, b in zip(l1, l2):
        np.testing.assert_array_equal(a, b)
    rep = classify_sample(wl, *l1, lazy=True)
    assert_report(rep, "lazy vs oracle")
    differ = int(np.sum(np.any(d1[0] != l1[0], axis=1)))
    assert differ <= rep["near_accept"][1e-5] + rep["near_select"][1e-5]


# ----------------------------------------------------- top-k / top-p filters ---
def run_filtered(wl, top_k, top_p, draft_bf16=False):
    d = to_device(wl, DEV, draft_bf16=draft_bf16)
    tk = None if top_k is None else torch.from_numpy(np.asarray(top_k, np.int32)).to(DEV)
    tp = None if top_p is None else torch.from_numpy(np.asarray(top_p, np.float32)).to(DEV)
    out = sv.spec_verify_sample_filtered(d["target"], d["draft"], d["tokens"], d["temperature"],
                                         tk, tp, d["seeds"], wl["offset"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check_filtered(wl, name, top_k, top_p, near_frac=0.25):
    print(f"[case] filtered {name} B={wl['B']} K={wl['K']} V={wl['V']} dtype={wl['dtype']}", flush=True)
    g = run_filtered(wl, top_k, top_p)
    rep = classify_sample(wl, *g, top_k=top_k, top_p=top_p)
    assert_report(rep, f"filtered {name}")
    assert rep["filter_near"] <= near_frac * rep["requests"] + 1, rep["filter_near"]
    return rep


def mixed_filters(B, V, seed):
    rng = np.random.default_rng(seed)
    top_k = rng.choice([0, 1, 5, 50, 1000, V], size=B).astype(np.int32)
    top_p = rng.choice([1.0, 0.5, 0.8, 0.9, 0.95], size=B).astype(np.float32)
    return top_k, top_p


FILTER_REDUCED = [
    ("c3-topp095", "c3_onehot", dict(B=32, V=2 * 8192 + 1232), "p"),
    ("c3-topk50", "c3_onehot", dict(B=32, V=2 * 8192 + 1232), "k"),
    ("c3-mixed", "c3_onehot", dict(B=48, V=2 * 8192 + 777), "mixed"),
    ("c3-K0", "c3_onehot", dict(B=16, K=0, V=5000), "mixed"),
    ("c2-topp095", "c2_stoch", dict(B=16, V=3 * 8192 + 1234), "p"),
    ("c2-mixed-scalar-path", "c2_stoch", dict(B=24, V=20001), "mixed"),
    ("c1", "c1_tiny", {}, "mixed"),
]


@pytest.mark.parametrize("name,cfg,kw,kind", FILTER_REDUCED, ids=[c[0] for c in FILTER_REDUCED])
def test_filtered_sample(name, cfg, kw, kind):
    for offset in range(2):
        wl = make(cfg, data_seed=400 + offset, offset=offset, **kw)
        B, V = wl["B"], wl["V"]
        if kind == "p":
            top_k, top_p = None, np.full(B, 0.95, np.float32)
        elif kind == "k":
            top_k, top_p = np.full(B, 50, np.int32), None
        else:
            top_k, top_p = mixed_filters(B, V, 410 + offset)
        check_filtered(wl, f"{name}/off{offset}", top_k, top_p)


def test_filtered_off_matches_oracle_unfiltered():
    """No filter (None, or k = 0 and p = 1): the unfiltered rule."""
    wl = make("c3_onehot", data_seed=420, B=32, V=9000)
    for tk, tp in [(None, None), (np.zeros(32, np.int32), np.ones(32, np.float32))]:
        g = run_filtered(wl, tk, tp)
        assert_report(classify_sample(wl, *g), "filters off")


def test_filtered_ties_and_flat_rows():
    """All-equal rows (every cut keeps all: more equal logits than one sort holds), a row
    with a tie at the top-k cut, and top-k = 1 (the largest value only)."""
    wl = make("c2_stoch", data_seed=421, B=8, K=2, V=3 * 8192 + 5)
    tgt = wl["target"].copy()
    drf = wl["draft"].copy()
    tgt[0] = 1.5
    drf[0] = -0.25
    tgt[1, :, :] = np.round(tgt[1], 0)               # few distinct values: wide ties
    drf[1, :, :] = np.round(drf[1], 0)
    wl = dict(wl, target=tgt, draft=drf)
    top_k = np.array([10, 3000, 1, 1, 7, 0, 2, 24581], np.int32)
    top_p = np.array([0.5, 0.9, 1.0, 0.3, 1.0, 0.95, 0.6, 0.99], np.float32)
    check_filtered(wl, "ties", top_k, top_p, near_frac=0.5)


def test_filtered_bf16_rows_outside_the_table():
    """bf16 rows whose values leave the one-pass table or strain it: an all-equal
    row, few distinct values (wide ties), zeros and magnitudes below 2^-16
    mixed in (and a row of zeros only, whose cut falls among them), half the
    vocabulary at -inf, a logit beyond 2^16, and the magnitudes just outside
    the table (the largest below 2^-16, and 2^16); each under a spread of
    top-k and top-p."""
    B, K, V = 12, 3, 3 * 8192 + 5
    wl = make("c3_onehot", data_seed=431, B=B, K=K, V=V)
    vals = oracle.logits_f64(wl["target"].reshape(-1), "bf16").reshape(wl["target"].shape)
    rng = np.random.default_rng(432)
    vals[0] = 1.5
    vals[1] = np.round(vals[1])
    tiny = rng.choice([0.0, -0.0, 2.0 ** -20, -(2.0 ** -18), 3.0 * 2.0 ** -17], size=vals[2].shape)
    vals[2] = np.where(rng.random(vals[2].shape) < 0.3, tiny, vals[2])
    vals[3] = 0.0
    vals[4, :, : V // 2] = -np.inf
    vals[5, :, 17] = 70000.0
    vals[6] = np.where(rng.random(vals[6].shape) < 0.5, 0.0, vals[6])
    vals[7, :, :100] = -np.inf
    vals[7, :, 100:] = np.round(vals[7, :, 100:] * 4) / 4
    # the magnitudes just outside the table, which a clamp maps to themselves:
    # the bf16 value below 2^-16 (0x377F) and 2^16 itself (0x4780), both signs
    below = float(np.array([0x377F << 16], np.uint32).view(np.float32)[0])
    vals[8, :, ::3] = below
    vals[8, :, 1::3] = -below
    vals[9, :, 5] = 65536.0
    vals[10, :, 7] = -65536.0
    vals[10, :, 8] = below
    wl = dict(wl, target=f32_to_bf16_bits(vals.astype(np.float32)))
    top_k = np.array([1, 10, 50, 7, 3, 0, 20000, 2, 0, 5, 100, V], np.int32)
    top_p = np.array([0.9, 0.5, 0.95, 0.3, 0.8, 0.95, 1.0, 0.99, 0.95, 0.0, 0.7, 0.6], np.float32)
    check_filtered(wl, "bf16 rows outside the table", top_k, top_p, near_frac=0.5)
    check_filtered(wl, "bf16 rows outside the table, top-p only", None, np.full(B, 0.9, np.float32),
                   near_frac=0.5)


def test_filtered_bf16_counter_carry():
    """V > 2 * 65535 with every logit equal: each half of a counter word would
    pass 65535 (a carry into the other half); the row takes the general search."""
    wl = make("c3_onehot", data_seed=433, B=3, K=1, V=140001)
    vals = oracle.logits_f64(wl["target"].reshape(-1), "bf16").reshape(wl["target"].shape)
    vals[0] = -2.25
    vals[1, :, ::2] = 0.75
    wl = dict(wl, target=f32_to_bf16_bits(vals.astype(np.float32)))
    check_filtered(wl, "bf16 counter carry", np.array([0, 3, 70000], np.int32),
                   np.array([0.9, 0.95, 0.5], np.float32), near_frac=1.0)


def _onehot_f32(B, V, seed):
    """A one-hot workload with fp32 rows (the C3 generator's values)."""
    wl = make("c3_onehot", data_seed=seed, B=B, V=V)
    vals = oracle.logits_f64(wl["target"].reshape(-1), "bf16").reshape(wl["target"].shape)
    return dict(wl, target=vals.astype(np.float32), dtype="f32")


@pytest.mark.parametrize("V", [32768, 32767, 40000])
def test_filtered_f32_row_lengths(V):
    """fp32 rows at the longest length one workgroup holds in LDS (32768
    logits: whole 16-byte vectors; 32767: the unaligned element path), and
    past it (40000: the row pass, then the streaming select), one-hot and
    with draft logits, under a spread of top-k and top-p."""
    wl = _onehot_f32(12, V, 434)
    top_k, top_p = mixed_filters(12, V, 435)
    check_filtered(wl, f"f32 one-hot V={V}", top_k, top_p)
    check_filtered(wl, f"f32 one-hot V={V} top-p", None, np.full(12, 0.95, np.float32))
    wl = make("c2_stoch", data_seed=436, B=10, V=V)
    top_k, top_p = mixed_filters(10, V, 437)
    check_filtered(wl, f"f32 explicit V={V}", top_k, top_p)


def test_filtered_f32_odd_rows():
    """fp32 rows on the LDS-resident select: a logit far above the rest (it
    alone holds top-p), half the vocabulary at -inf, few distinct values
    (wide ties), every logit equal (more equal values than one sort holds),
    and a logit of 1e4, each with one-hot drafts."""
    B, V = 6, 9000
    wl = _onehot_f32(B, V, 438)
    vals = wl["target"].copy()
    vals[0, :, 11] = 80.0
    vals[1, :, : V // 2] = -np.inf
    vals[2] = np.round(vals[2] * 2) / 2
    vals[3] = 1.5
    vals[4, :, 3] = 1e4
    wl = dict(wl, target=vals)
    top_k = np.array([0, 5, 40, 0, 2, 0], np.int32)
    top_p = np.array([0.9, 0.95, 0.5, 0.8, 0.95, 0.99], np.float32)
    check_filtered(wl, "f32 odd rows", top_k, top_p, near_frac=0.5)


@pytest.mark.parametrize("V", [1000, 40000])
def test_filtered_f32_mostly_neg_inf(V):
    """fp32 rows whose logits are nearly all -inf (a few finite ones per row:
    5, 40 or all but a handful), on the LDS-resident select (V = 1000) and the
    streaming one (V = 40000): top-k above the finite count keeps every
    finite logit, top-k and top-p cuts fall among the few finite values, and
    the slots past V stay out of the cut."""
    B = 8
    rng = np.random.default_rng(443)
    wl = _onehot_f32(B, V, 444)
    vals = np.full_like(wl["target"], -np.inf)
    for b in range(B):
        keep = rng.choice(V, size=(5, 40, V - 3)[b % 3], replace=False)
        vals[b][:, keep] = wl["target"][b][:, keep]
    wl = dict(wl, target=vals)
    # drafts on finite logits, so that the one-hot rule has mass to test
    tok = wl["draft_tokens"].copy()
    for b in range(B):
        fin = np.flatnonzero(np.isfinite(vals[b, 0]))
        tok[b] = fin[rng.integers(0, len(fin), size=tok.shape[1])]
    wl = dict(wl, draft_tokens=tok)
    top_k = np.array([0, 50, 3, 0, 100, 0, 7, 0], np.int32)
    top_p = np.array([0.9, 1.0, 0.95, 0.5, 0.99, 0.0, 0.8, 0.95], np.float32)
    check_filtered(wl, f"f32 mostly -inf V={V}", top_k, top_p, near_frac=0.5)


@pytest.mark.parametrize("V", [1, 3, 17])
def test_filtered_tiny_vocab(V):
    """Rows of 1, 3 and 17 logits (a partial vector in the LDS-resident select,
    a single chunk in the residual pass), fp32 one-hot and with draft logits,
    bf16 one-hot; top_p 0 keeps the largest value only, top_k 1 likewise."""
    top_k = np.array([0, 1, 2, 0, 0, V], np.int32)
    top_p = np.array([0.0, 1.0, 0.9, 0.5, 0.95, 0.99], np.float32)
    check_filtered(_onehot_f32(6, V, 440), f"f32 one-hot V={V}", top_k, top_p, near_frac=0.5)
    check_filtered(make("c2_stoch", data_seed=441, B=6, K=2, V=V), f"f32 explicit V={V}", top_k, top_p,
                   near_frac=0.5)
    check_filtered(make("c3_onehot", data_seed=442, B=6, K=2, V=V), f"bf16 one-hot V={V}", top_k, top_p,
                   near_frac=0.5)


def test_filtered_full_size_c2():
    """C2 at its full size (fp32, draft logits) with top_p 0.95, every request."""
    wl = make("c2_stoch", data_seed=1)
    top_p = np.full(wl["B"], 0.95, np.float32)
    check_filtered(wl, "c2 full top-p 0.95", None, top_p)


def test_filtered_bf16_explicit_draft():
    wl = make("c2_stoch", data_seed=422, B=12, V=8192 + 100)
    wl = dict(wl, target=f32_to_bf16_bits(wl["target"]), dtype="bf16",
              draft=f32_to_bf16_bits(wl["draft"]))
    d = to_device(wl, DEV, draft_bf16=True)
    top_k, top_p = mixed_filters(12, wl["V"], 423)
    out = sv.spec_verify_sample_filtered(d["target"], d["draft"], d["tokens"], d["temperature"],
                                         torch.from_numpy(top_k).to(DEV), torch.from_numpy(top_p).to(DEV),
                                         d["seeds"], wl["offset"])
    g = [t.cpu().numpy() for t in out]
    rep = classify_sample(wl, *g, draft_dtype="bf16", top_k=top_k, top_p=top_p)
    assert_report(rep, "filtered bf16 explicit")


def test_filtered_deterministic():
    wl = make("c3_onehot", data_seed=424, B=32, V=20000)
    top_k, top_p = mixed_filters(32, 20000, 425)
    a = run_filtered(wl, top_k, top_p)
    b = run_filtered(wl, top_k, top_p)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_filtered_full_size_c3():
    """C3 at its full size with top_p 0.95 (the pages' sampling setting), sampled requests."""
    wl = make("c3_onehot", data_seed=1)
    B = wl["B"]
    top_p = np.full(B, 0.95, np.float32)
    print("[case] filtered c3 full", flush=True)
    g = run_filtered(wl, None, top_p)
    reqs = list(range(0, B, 8))
    rep = classify_sample(wl, *g, requests=reqs, top_p=top_p)
    assert_report(rep, "filtered c3 full (sampled)")
    assert rep["filter_near"] <= 0.25 * len(reqs) + 1


def test_filtered_tokens_only_equals_full_outputs():
    """Without p / q outputs the select pass skips the rows past a request's first
    certain rejection (one-hot drafts, top-k off). Tokens and accept lengths must
    equal those of the call with p / q outputs bitwise, including requests whose
    drafts are accepted often (peaked rows, argmax drafts) and requests whose
    filters forbid skipping (top-k on, top_p off or NaN)."""
    full = make("c3_onehot", data_seed=1)
    peaked = make("c3_onehot", data_seed=427, B=40, V=2 * 8192 + 777)
    vals = oracle.logits_f64(peaked["target"].reshape(-1), "bf16").reshape(peaked["target"].shape)
    am = vals.argmax(-1).astype(np.int32)
    rng = np.random.default_rng(428)
    tok = np.where(rng.random((40, peaked["K"])) < 0.9, am[:, :peaked["K"]], 7).astype(np.int32)
    peaked = dict(peaked, draft_tokens=tok, temperature=np.full(40, 0.15, np.float32))
    mixed = make("c3_onehot", data_seed=429, B=48, V=20000)
    mk, mp = mixed_filters(48, 20000, 430)
    mp[::7] = np.nan
    cases = [("c3 full top_p 0.95", full, None, np.full(full["B"], 0.95, np.float32)),
             ("peaked, argmax drafts", peaked, None, rng.choice([0.5, 0.9, 0.99, 1.0], 40).astype(np.float32)),
             ("mixed filters", mixed, mk, mp)]
    for name, wl, top_k, top_p in cases:
        print(f"[case] filtered tokens-only {name} B={wl['B']} V={wl['V']}", flush=True)
        d = to_device(wl, DEV)
        tk = None if top_k is None else torch.from_numpy(top_k).to(DEV)
        tp = torch.from_numpy(top_p).to(DEV)
        args = (d["target"], d["draft"], d["tokens"], d["temperature"], tk, tp, d["seeds"], wl["offset"])
        t1, l1, _, _ = sv.spec_verify_sample_filtered(*args)
        t2, l2, p2, q2 = sv.spec_verify_sample_filtered(*args, want_probs=False)
        torch.cuda.synchronize()
        assert p2 is None and q2 is None
        np.testing.assert_array_equal(l1.cpu().numpy(), l2.cpu().numpy())
        np.testing.assert_array_equal(t1.cpu().numpy(), t2.cpu().numpy())
        hist = np.bincount(l2.cpu().numpy(), minlength=wl["K"] + 2).tolist()
        print(f"[parity] tokens-only {name}: identical, accept_len histogram {hist}", flush=True)


def test_small_batch_long_rows():
    """Small launches of long rows take four-chunk runs per wave: one GPU's
    share of C3 split over 8 GPUs (B=32), and greedy rows of 127 chunks at B=16."""
    check_sample(make("c3_onehot", data_seed=2, B=32), "c3 B=32 (8-way shard)")
    check_greedy(make("c4_greedy", data_seed=3, B=16), "c4 B=16")
