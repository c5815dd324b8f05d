"""Grammar bitmasks in the oracle (LMDeploy "Speculative Decoding", structured
output: the target's logits are masked at every verified position before
rejection sampling; with draft logits the draft rows carry the same mask)."""
import numpy as np

import oracle
from workloads import make


def random_mask(rng, B, R, V, p_allow=0.3):
    allowed = rng.random((B, R, V)) < p_allow
    allowed[..., 0] = True                      # never a row without an allowed token
    return pack_bits(allowed), allowed


def pack_bits(allowed):
    """uint32 words, bit v % 32 of word v // 32, through numpy's bit packing."""
    B, R, V = allowed.shape
    W = (V + 31) // 32
    pad = np.zeros((B, R, W * 32), bool)
    pad[..., :V] = allowed
    by = np.packbits(pad.reshape(B, R, W, 4, 8), axis=-1, bitorder="little")[..., 0]
    return np.ascontiguousarray(by).view("<u4").reshape(B, R, W).astype(np.uint32)


def test_bit_layout_against_numpy_unpacking():
    rng = np.random.default_rng(70)
    V = 77
    words = rng.integers(0, 2**32, 3, dtype=np.uint64).astype(np.uint32)
    bits = np.unpackbits(words.astype("<u4").view(np.uint8), bitorder="little")[:V].astype(bool)
    out = oracle.apply_bitmask(np.zeros(V), words)
    np.testing.assert_array_equal(np.isfinite(out), bits)


def test_all_ones_mask_changes_nothing():
    wl = make("c2_stoch", data_seed=71, B=6, K=3, V=500)
    ones = np.full((6, 4, (500 + 31) // 32), 0xFFFFFFFF, np.uint32)
    a = oracle.spec_verify_sample(wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"],
                                  wl["seeds"], wl["offset"])
    b = oracle.spec_verify_sample(wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"],
                                  wl["seeds"], wl["offset"], bitmask=ones)
    for x, y in zip(a[:4], b[:4]):
        np.testing.assert_array_equal(x, y)
    g = make("c4_greedy", data_seed=72, B=6, K=3, V=500)
    ga = oracle.spec_verify_greedy(g["target"], g["draft_tokens"])
    gb = oracle.spec_verify_greedy(g["target"], g["draft_tokens"], bitmask=ones)
    for x, y in zip(ga, gb):
        np.testing.assert_array_equal(x, y)


def test_emitted_tokens_are_allowed_and_disallowed_drafts_rejected():
    rng = np.random.default_rng(73)
    for cfg in ("c2_stoch", "c3_onehot"):
        wl = make(cfg, data_seed=74, B=40, K=4, V=300)
        mask, allowed = random_mask(rng, 40, 5, 300)
        tok, alen, p, q, _ = oracle.spec_verify_sample(
            wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"], wl["seeds"],
            wl["offset"], target_dtype=wl["dtype"], bitmask=mask)
        for b in range(40):
            for i in range(alen[b]):
                assert allowed[b, i, tok[b, i]]
            for i in range(4):
                if not allowed[b, i, wl["draft_tokens"][b, i]]:
                    assert p[b, i] == 0 and alen[b] <= i + 1


def test_greedy_argmax_over_allowed_tokens():
    rng = np.random.default_rng(75)
    wl = make("c4_greedy", data_seed=76, B=10, K=3, V=400)
    mask, allowed = random_mask(rng, 10, 4, 400)
    _, _, g = oracle.spec_verify_greedy(wl["target"], wl["draft_tokens"], bitmask=mask)
    vals = np.where(allowed, wl["target"].astype(np.float64), -np.inf)
    np.testing.assert_array_equal(g, vals.argmax(-1))
