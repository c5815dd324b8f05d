"""Seeded synthetic inputs for batched speculative-decoding verification.

This module only draws random inputs; it holds none of the verification
arithmetic (no softmax, no acceptance test, no residual, no inverse CDF).
Both the fp64 CPU oracle and the HIP library are fed from here, so the two
see byte-identical logits, draft tokens, temperatures and seeds.

The five named workloads stand in for real model logits: the pages measure
speculative decoding only end to end on trained models (Vicuna, Llama,
Qwen, DeepSeek) and public suites, none of which is used here. Shapes follow
the engines' own limits (FastDeploy's "参数说明": at most 5 draft tokens and
batch 256; LMDeploy's pipeline example: batch 128 with 3 draft tokens) and
the vocabularies of current model families.

Recipes (all draws from numpy PCG64 seeded by ``data_seed``):

* ``c1_tiny``    B=1,  K=1, V=1000,   fp32 target ~ N(0, 1); draft logits =
  target + N(0, 0.5); T = 1.0; draft tokens x_i ~ q_i (Gumbel-max on the
  draft logits / T).
* ``c2_stoch``   B=64, K=3, V=32000,  fp32 target ~ N(0, 2) plus +6 at one
  uniformly chosen token per row; draft = target + N(0, 0.7); T = 0.8;
  x_i ~ q_i.
* ``c3_onehot``  B=256, K=5, V=128256, bf16 target ~ N(0, 2) (fp32 draws
  rounded to nearest-even bf16); deterministic drafts (one-hot q): x_i is
  the row's argmax (lowest index on ties) with probability 0.6, else
  uniform on [0, V); T = 0.7.
* ``c4_greedy``  B=128, K=3, V=129280, fp32 target ~ N(0, 3); x_i is the
  row's argmax with probability 0.85, else uniform over the other V-1
  tokens.
* ``c5_tree``    B=32, V=32000, fp32 ~ N(0, 2) per node of the static
  3x3x2 Medusa tree (31 nodes with the root, 18 leaf paths); node tokens:
  for each parent, with probability 0.8 one uniformly chosen child slot
  carries the parent row's argmax, every other child a distinct uniform
  token different from that argmax.

"N(0, s)" means standard deviation s. Per-request seeds are uint64 draws
from the same generator.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "make", "medusa_tree_parents", "f32_to_bf16_bits",
    "pack_ragged", "make_ragged", "make_masked",
    "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "sample" | "greedy" | "tree"
    B: int
    K: int               # draft tokens per request (tree: unused, 0)
    V: int
    dtype: str           # "f32" | "bf16"
    target_std: float
    draft_std: float | None   # None: no draft logits (one-hot q or greedy)
    temperature: float | None
    peak: float = 0.0         # planted +peak at one token per target row
    p_match: float = 0.0      # deterministic drafts: P(draft = argmax)
    tree: tuple[int, ...] = ()  # branching per depth for "tree"


CONFIGS = {
    "c1_tiny": Workload("c1_tiny", "sample", 1, 1, 1000, "f32", 1.0, 0.5, 1.0),
    "c2_stoch": Workload("c2_stoch", "sample", 64, 3, 32000, "f32", 2.0, 0.7, 0.8,
                         peak=6.0),
    "c3_onehot": Workload("c3_onehot", "sample", 256, 5, 128256, "bf16", 2.0, None,
                          0.7, p_match=0.6),
    "c4_greedy": Workload("c4_greedy", "greedy", 128, 3, 129280, "f32", 3.0, None,
                          None, p_match=0.85),
    "c5_tree": Workload("c5_tree", "tree", 32, 0, 32000, "f32", 2.0, None, None,
                        tree=(3, 3, 2)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def medusa_tree_parents(branching=(3, 3, 2)) -> np.ndarray:
    """Parent index of every node of a full tree, breadth-first, root = 0.

    Every node at depth d has branching[d] children, so (3, 3, 2) gives
    1 + 3 + 9 + 18 = 31 nodes and 18 root-to-leaf paths.
    """
    parents = [-1]
    level = [0]
    for fan in branching:
        nxt = []
        for p in level:
            for _ in range(fan):
                parents.append(p)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.asarray(parents, dtype=np.int32)


def _gumbel_argmax(rng, logits: np.ndarray, T: float) -> np.ndarray:
    """Draw one index per row from softmax(logits / T) by the Gumbel-max trick."""
    g = -np.log(-np.log(rng.random(logits.shape, dtype=np.float64)))
    return np.argmax(logits.astype(np.float64) / T + g, axis=-1).astype(np.int32)


def make(name: str, data_seed: int = 0, *, B: int | None = None, K: int | None = None,
         V: int | None = None, offset: int = 0) -> dict:
    """Build one workload; B, K and V may be overridden for reduced-size tests.

    Returns a dict of host numpy arrays:
      target        [B, R, V] float32, or uint16 bf16 bits when dtype is bf16
                    (R = K+1 for sample/greedy, N nodes for tree)
      draft         [B, K, V] float32 or None
      draft_tokens  [B, K] int32 (tree: node_tokens [B, N], column 0 unused = -1)
      temperature   [B] float32 or None
      seeds         [B] uint64
      parents       [N] int32 (tree only)
    plus the scalars name, mode, dtype, B, K, V, offset.
    """
    cfg = CONFIGS[name]
    B = cfg.B if B is None else B
    K = cfg.K if K is None else K
    V = cfg.V if V is None else V
    rng = np.random.default_rng(np.random.PCG64(data_seed))
    out = dict(name=name, mode=cfg.mode, dtype=cfg.dtype, B=B, K=K, V=V, offset=offset,
               draft=None, temperature=None, parents=None)

    if cfg.mode == "tree":
        parents = medusa_tree_parents(cfg.tree)
        N = len(parents)
        tgt = rng.normal(0.0, cfg.target_std, size=(B, N, V)).astype(np.float32)
        best = np.argmax(tgt, axis=-1)                       # [B, N]
        tok = np.full((B, N), -1, dtype=np.int32)
        children = {}
        for n in range(1, N):
            children.setdefault(int(parents[n]), []).append(n)
        for b in range(B):
            for p, kids in children.items():
                g = int(best[b, p])
                hit = rng.random() < 0.8
                slot = int(rng.integers(len(kids)))
                used = {g}
                for j, n in enumerate(kids):
                    if hit and j == slot:
                        tok[b, n] = g
                        continue
                    while True:
                        t = int(rng.integers(V))
                        if t not in used:
                            break
                    used.add(t)
                    tok[b, n] = t
        out.update(target=tgt, draft_tokens=tok, parents=parents, K=0,
                   seeds=rng.integers(0, 2**63, size=B, dtype=np.uint64) * np.uint64(2)
                   + rng.integers(0, 2, size=B, dtype=np.uint64))
        return out

    R = K + 1
    tgt = rng.normal(0.0, cfg.target_std, size=(B, R, V)).astype(np.float32)
    if cfg.peak:
        where = rng.integers(0, V, size=(B, R))
        np.put_along_axis(tgt, where[..., None],
                          np.take_along_axis(tgt, where[..., None], -1) + np.float32(cfg.peak),
                          axis=-1)
    draft = None
    if cfg.draft_std is not None:
        noise = rng.normal(0.0, cfg.draft_std, size=(B, K, V)).astype(np.float32)
        draft = (tgt[:, :K, :] + noise).astype(np.float32)
    if cfg.dtype == "bf16":
        tgt_store = f32_to_bf16_bits(tgt)
        tgt_vals = bf16_bits_to_f32(tgt_store)
    else:
        tgt_store = tgt
        tgt_vals = tgt

    if draft is not None:
        tokens = _gumbel_argmax(rng, draft, cfg.temperature) if K else np.zeros((B, 0), np.int32)
    else:
        if K:
            am = np.argmax(tgt_vals[:, :K, :], axis=-1)
            hit = rng.random((B, K)) < cfg.p_match
            if cfg.mode == "greedy" and V > 1:
                other = rng.integers(0, V - 1, size=(B, K))
                other = other + (other >= am)          # uniform over tokens != argmax
            elif cfg.mode == "greedy":
                other = am
            else:
                other = rng.integers(0, V, size=(B, K))
            tokens = np.where(hit, am, other).astype(np.int32)
        else:
            tokens = np.zeros((B, 0), np.int32)

    seeds = (rng.integers(0, 2**63, size=B, dtype=np.uint64) * np.uint64(2)
             + rng.integers(0, 2, size=B, dtype=np.uint64))
    temp = None
    if cfg.temperature is not None:
        temp = np.full(B, cfg.temperature, dtype=np.float32)
    out.update(target=tgt_store, draft=draft, draft_tokens=np.ascontiguousarray(tokens),
               temperature=temp, seeds=seeds)
    return out


def pack_ragged(wl: dict, ks) -> dict:
    """Cut a dense workload to per-request draft counts ks[b] <= K and pack it.

    Returns dict(ks, cu [B + 1] int32 prefix sums, target_rows [sum ks + B, V]
    (request b's K_b + 1 rows from cu[b] + b), draft_rows [sum ks, V] or
    None, draft_tokens [sum ks] int32). Layout only: nothing is computed.
    """
    B = wl["B"]
    ks = np.asarray(ks, dtype=np.int64)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(ks)
    rows = np.concatenate([wl["target"][b, : ks[b] + 1] for b in range(B)])
    drows = None
    if wl.get("draft") is not None:
        drows = np.concatenate([wl["draft"][b, : ks[b]] for b in range(B)] +
                               [np.zeros((0, wl["V"]), wl["draft"].dtype)])
    toks = np.concatenate([wl["draft_tokens"][b, : ks[b]] for b in range(B)] +
                          [np.zeros(0, np.int32)]).astype(np.int32)
    return dict(ks=ks, cu=cu, target_rows=np.ascontiguousarray(rows),
                draft_rows=None if drows is None else np.ascontiguousarray(drows),
                draft_tokens=toks)


def make_ragged(name: str, data_seed: int = 0, **kw) -> dict:
    """A named workload with per-request draft counts K_b ~ uniform{0..K}
    (seeded by data_seed), packed. The dense arrays stay in the dict."""
    wl = make(name, data_seed, **kw)
    ks = np.random.default_rng([data_seed, 7]).integers(0, wl["K"] + 1, wl["B"])
    wl = dict(wl, name=name.split("_")[0] + "_ragged", ragged=pack_ragged(wl, ks))
    return wl


def make_masked(name: str, data_seed: int = 0, allow: float = 0.5, **kw) -> dict:
    """A named workload plus a grammar bitmask [B, K+1, ceil(V/32)] uint32 that
    allows each token of each position independently with probability
    ``allow`` (bit v % 32 of word v // 32 set = allowed; token 0 always
    allowed so no position is empty). Layout only: nothing is computed."""
    wl = make(name, data_seed, **kw)
    B, R, V = wl["B"], wl["K"] + 1, wl["V"]
    rng = np.random.default_rng([data_seed, 11])
    allowed = rng.random((B, R, V)) < allow
    allowed[..., 0] = True
    W = (V + 31) // 32
    pad = np.zeros((B, R, W * 32), bool)
    pad[..., :V] = allowed
    by = np.packbits(pad.reshape(B, R, W, 4, 8), axis=-1, bitorder="little")[..., 0]
    mask = np.ascontiguousarray(by).view("<u4").reshape(B, R, W).astype(np.uint32)
    return dict(wl, name=name.split("_")[0] + "_masked", bitmask=mask,
                mask_allowed=float(allowed.mean()))
