"""Plain fp64 CPU oracle for batched speculative-decoding verification.

Test infrastructure only: imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of the benchmark, never by the library's product path.
It shares no code with the HIP library.

Citation key (the pages this follows):
  [SD]  "【大模型基础设施工程】15：推测解码与 MTP" (juejin.cn): §1.2 (one
        target forward scores K+1 positions; accepted length per step),
        §2.1 "算法骨架" (the verification rule), the correctness subsection
        printed as "1.2 正确性保证" under §2 (output law equals the
        target's), §2.3 (accepted length alpha in [1, K+1]), §3.3 "Tree
        Attention" (Medusa tree: each node sees only its ancestors, the
        longest accepted path wins), §11 (code sketch: drafts [B, K],
        target logits [B, K+1, V]; greedy speculation reproduces plain
        greedy output).
  [FD]  FastDeploy "投机解码", "高效投机解码框架设计" (sampling and
        verification run per batch sample in parallel).

What the oracle computes, step by step, for one request b with K drafts:

1. Inputs are widened to fp64 exactly (bf16 bit pattern h is the fp32 with
   bits h << 16).
2. p_i = softmax(l_i / T) for every target position i = 0..K; q_i is the
   draft's softmax(l'_i / T) when draft logits are given, otherwise the
   one-hot vector of the draft token x_i (deterministic drafts: n-gram
   lookup, MTP greedy heads). [SD §2.1]; T applies to both (reading R1).
3. Draft x_i is accepted with probability min(1, p_i(x_i) / q_i(x_i)); with a
   uniform u this is the event u * q_i(x_i) < p_i(x_i) (reading R2). The
   scan stops at the first rejection. [SD §2.1]
4. On a rejection at position a the replacement token is drawn from the
   normalised residual max(0, p_a - q_a); if every draft was accepted a
   bonus token is drawn from p_K (0-based; the pages' p_{K+1}). [SD §2.1]
   A residual of total mass zero falls back to p_a (reading R5).
5. A draw from weights w with uniform u is the inverse CDF: the smallest j
   whose left-to-right cumulative sum C_j exceeds u * C_{V-1}; if rounding
   leaves none, the last token of positive weight (reading R6).
6. Uniforms come from Philox4x64-10 keyed by (seed, request, position,
   offset), see ``oracle.philox``; one pair per position (reading R3).
7. Output: tokens x_0..x_{a-1}, then the drawn token, padded with -1;
   accept_len = a + 1 in [1, K+1] [SD §2.3].

The decision core (``accept_length``, ``residual_weights``, ``inverse_cdf``,
``verify_request``) uses only +, -, *, comparisons and max, so it runs on
``fractions.Fraction`` as well as on floats; the tests use that to compute
the exact output law by enumeration.

Greedy verification: g_i = argmax l_i (lowest index on ties), the longest
prefix with x_i = g_i is accepted and g_a is emitted [SD §11, greedy output
equals plain greedy decoding]. Tree verification: node n is accepted when
its parent is accepted and its token equals the parent's argmax; the
deepest accepted node wins, lowest index on ties [SD §3.3].
"""
from __future__ import annotations

import math

import numpy as np

from .philox import request_uniforms

__all__ = [
    "logits_f64", "softmax_t", "onehot", "accept_length", "residual_weights",
    "inverse_cdf", "verify_request", "spec_verify_sample", "argmax_lowest",
    "spec_verify_greedy", "tree_depths", "spec_verify_tree",
    "ragged_draft_count", "spec_verify_sample_ragged", "spec_verify_greedy_ragged",
    "apply_bitmask", "filter_keep", "filtered_row",
]


# ---------------------------------------------------------------- inputs ---

def logits_f64(row, dtype: str) -> np.ndarray:
    """Widen one logits vector to fp64 exactly. dtype "f32" or "bf16" (uint16 bits)."""
    a = np.asarray(row)
    if dtype == "bf16":
        bits32 = a.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def apply_bitmask(logits: np.ndarray, mask_row) -> np.ndarray:
    """Logits of one position with the tokens a grammar bitmask disallows set to
    -inf (LMDeploy "Speculative Decoding", structured output: the grammar
    mask is applied to the target's logits at every verified position).
    Token v is allowed when bit v % 32 of word v // 32 of ``mask_row`` is 1."""
    V = len(logits)
    out = np.array(logits, dtype=np.float64)
    for v in range(V):
        if not (int(mask_row[v // 32]) >> (v % 32)) & 1:
            out[v] = -math.inf
    return out


# ------------------------------------------------ top-k / top-p filters ---
# The pages run speculative decoding with the sampling parameters
# temperature 0.8 and top_p 0.95 ([VA] "Speculative Decoding Guide", the
# offline-inference examples). Reading: p and q are the distributions the
# sampler would draw from, so both are filtered with the request's (top_k,
# top_p) after the temperature. top-k keeps the tokens whose logit is at
# least the k-th largest logit (ties at the cut are kept). top-p then keeps,
# of those, the tokens whose logit is at least t, where t is the largest
# logit value whose upper set {v : l_v >= t} holds at least top_p of the
# top-k set's mass. The kept set is renormalised. top_k <= 0 or >= V, and
# top_p >= 1 or NaN, switch the filter off.

def filter_keep(logits, T: float, top_k: int = 0, top_p: float = 1.0):
    """Kept tokens of one row under (top_k, top_p), and the top-p decision's
    margin: the distance, as a fraction of the top-k mass, from top_p to the
    nearer of the two cumulative masses that bracket it (inf when top-p is
    off). A computation that rounds its masses by less than the margin
    keeps the same set."""
    l = np.asarray(logits, dtype=np.float64)
    V = len(l)
    keep = np.ones(V, dtype=bool)
    if 0 < int(top_k) < V:
        kth = np.sort(l)[::-1][int(top_k) - 1]
        keep = l >= kth
    margin = math.inf
    if float(top_p) < 1.0:                          # NaN compares false: off
        w = softmax_t(l, T) * keep
        Z = math.fsum(w.tolist())
        # distinct kept values, largest first, with the mass of each
        vals, inv = np.unique(l[keep], return_inverse=True)
        group = np.bincount(inv, weights=w[keep])[::-1] / Z
        vals = vals[::-1]
        upper = np.cumsum(group)                     # mass of {l >= vals[j]}
        hit = np.nonzero(upper >= float(top_p))[0]
        j = int(hit[0]) if len(hit) else len(vals) - 1
        t = vals[j]
        above = upper[j - 1] if j > 0 else 0.0
        # nothing lies above the largest value: that side is exact
        margin = upper[j] - float(top_p) if j == 0 else min(float(top_p) - above,
                                                            upper[j] - float(top_p))
        keep = keep & (l >= t)
    return keep, margin


def filtered_row(logits, T: float, top_k: int = 0, top_p: float = 1.0):
    """softmax(logits / T) restricted to the kept set and renormalised; and the margin."""
    keep, margin = filter_keep(logits, T, top_k, top_p)
    p = softmax_t(logits, T)
    if keep.all():
        return p, margin
    w = p * keep
    return w / math.fsum(w.tolist()), margin


def softmax_t(logits: np.ndarray, T: float) -> np.ndarray:
    """p = softmax(logits / T) in fp64: exp(z - max z) / sum exp(z - max z)."""
    z = np.asarray(logits, dtype=np.float64) / float(T)
    m = np.max(z)
    e = np.exp(z - m)
    return e / math.fsum(e.tolist())


def onehot(V: int, x: int):
    """q for a deterministic draft token: all mass on x (nothing if x is outside [0, V))."""
    q = [0.0] * V
    if 0 <= x < V:
        q[x] = 1.0
    return q


# --------------------------------------------------------- decision core ---

def accept_length(p_x, q_x, u_acc) -> int:
    """Number of leading drafts accepted: stop at the first i with not (u_i q_i(x_i) < p_i(x_i))."""
    a = 0
    for i in range(len(p_x)):
        if u_acc[i] * q_x[i] < p_x[i]:
            a += 1
        else:
            break
    return a


def residual_weights(p_row, q_row):
    """Unnormalised residual max(0, p - q); p itself when that has no mass."""
    w = [pv - qv if pv > qv else 0 * pv for pv, qv in zip(p_row, q_row)]
    if not any(v > 0 for v in w):
        return list(p_row)
    return w


def inverse_cdf(weights, u) -> int:
    """Smallest j with C_j > u * Z, C_j = w_0 + ... + w_j summed left to right, Z = C_last."""
    cum = []
    running = 0 * weights[0]
    for wj in weights:
        running = running + wj
        cum.append(running)
    target = u * running
    for j, c in enumerate(cum):
        if c > target:
            return j
    for j in range(len(weights) - 1, -1, -1):      # rounding overshoot
        if weights[j] > 0:
            return j
    return len(weights) - 1


def verify_request(p_rows, q_rows, x, u_acc, u_smp) -> dict:
    """One request: K+1 target distributions, K draft distributions, K drafts, K+1 uniform pairs."""
    K = len(x)
    V = len(p_rows[0])
    p_x = [p_rows[i][x[i]] if 0 <= x[i] < V else 0 * p_rows[i][0] for i in range(K)]
    q_x = [q_rows[i][x[i]] if 0 <= x[i] < V else 0 * p_rows[i][0] for i in range(K)]
    a = accept_length(p_x, q_x, u_acc)
    if a < K:
        w = residual_weights(p_rows[a], q_rows[a])
    else:
        w = list(p_rows[K])
    y = inverse_cdf(w, u_smp[a])
    return dict(tokens=list(x[:a]) + [y], accept_len=a + 1, a=a, p_x=p_x, q_x=q_x,
                weights=w, u_select=u_smp[a], u_acc=list(u_acc))


def spec_verify_sample(target, draft, draft_tokens, temperature, seeds, offset=0,
                       target_dtype="f32", draft_dtype="f32", requests=None,
                       keep_trace=False, bitmask=None, top_k=None, top_p=None):
    """Batched stochastic verification.

    target [B, K+1, V] (fp32 values or bf16 bit patterns), draft [B, >=K, V]
    or None for one-hot q, draft_tokens [B, K], temperature [B], seeds [B]
    (uint64), offset: step counter. ``requests`` restricts the work to a
    subset of request indices (other rows of the outputs stay -1 / 0).

    Returns (tokens [B, K+1] int32, accept_len [B] int32, p_draft [B, K]
    float64, q_draft [B, K] float64, traces) where traces[b] is the
    per-request record from ``verify_request`` when keep_trace is set.
    A request whose temperature is not a finite positive number is refused:
    accept_len 0, tokens -1, probabilities 0. ``bitmask`` [B, K+1, ceil(V/32)]
    (optional) masks target row i and, with draft logits, draft row i.
    ``top_k`` [B] and ``top_p`` [B] (optional) filter every target row and,
    with draft logits, every draft row (``filter_keep``); the trace then
    holds the smallest top-p margin of the request's rows.
    """
    B, R, V = target.shape
    K = R - 1
    tokens = np.full((B, K + 1), -1, dtype=np.int32)
    accept_len = np.zeros(B, dtype=np.int32)
    p_draft = np.zeros((B, K), dtype=np.float64)
    q_draft = np.zeros((B, K), dtype=np.float64)
    traces = {}
    for b in (range(B) if requests is None else requests):
        T = float(temperature[b])
        if not (math.isfinite(T) and T > 0):
            continue
        def masked(l, i):
            return l if bitmask is None else apply_bitmask(l, bitmask[b, i])
        tk = 0 if top_k is None else int(top_k[b])
        tp = 1.0 if top_p is None else float(top_p[b])
        margins = []

        def dist(l):
            if top_k is None and top_p is None:
                return softmax_t(l, T).tolist()
            row, m = filtered_row(l, T, tk, tp)
            margins.append(m)
            return row.tolist()
        p_rows = [dist(masked(logits_f64(target[b, i], target_dtype), i)) for i in range(K + 1)]
        x = [int(v) for v in draft_tokens[b, :K]]
        if draft is not None:
            q_rows = [dist(masked(logits_f64(draft[b, i], draft_dtype), i)) for i in range(K)]
        else:
            q_rows = [onehot(V, x[i]) for i in range(K)]
        pairs = [request_uniforms(int(seeds[b]), b, i, int(offset)) for i in range(K + 1)]
        res = verify_request(p_rows, q_rows, x, [u for u, _ in pairs], [u for _, u in pairs])
        tokens[b, :res["accept_len"]] = res["tokens"]
        accept_len[b] = res["accept_len"]
        p_draft[b, :] = res["p_x"]
        q_draft[b, :] = res["q_x"]
        if keep_trace:
            res["filter_margin"] = min(margins) if margins else math.inf
            traces[b] = res
    return tokens, accept_len, p_draft, q_draft, traces


# ----------------------------------------------------- ragged batches ---
# Requests with their own draft counts K_b ([FD] "高效投机解码框架设计": one
# forward verifies variable-length queries, and virtual padding maps each
# output row back to its request; [VA] suffix decoding proposes an adaptive
# number of tokens per request; [SD] §10.2 adjusts K per request). Rows are
# packed: with cu[b] = K_0 + ... + K_{b-1}, request b's K_b + 1 target rows
# are rows cu[b] + b ... cu[b] + b + K_b, its draft rows and tokens start at
# cu[b]. The rule per request is the dense one.

def ragged_draft_count(cu, b, total_k, k_max):
    """K_b of request b, or None when its offsets are out of order or range."""
    c0, c1 = int(cu[b]), int(cu[b + 1])
    if not (0 <= c0 <= c1 <= total_k and c1 - c0 <= k_max):
        return None
    return c1 - c0


def spec_verify_sample_ragged(target_rows, draft_rows, cu, draft_tokens, temperature, seeds,
                              offset=0, k_max=None, target_dtype="f32", draft_dtype="f32",
                              keep_trace=False):
    """Stochastic verification of a ragged batch.

    target_rows [total_k + B, V], draft_rows [total_k, V] or None (one-hot q),
    cu [B + 1] prefix sums of the draft counts, draft_tokens [total_k].
    Uniforms are keyed by (seed_b, b, position) exactly as in the dense case.
    Returns (tokens [B, k_max + 1], accept_len [B], p_draft [total_k],
    q_draft [total_k], traces). A request with bad offsets or a temperature
    that is not finite and positive is refused (accept_len 0, tokens -1).
    """
    B = len(cu) - 1
    total_k = len(draft_tokens)
    if k_max is None:
        k_max = max([0] + [int(cu[b + 1]) - int(cu[b]) for b in range(B)])
    V = target_rows.shape[1]
    tokens = np.full((B, k_max + 1), -1, dtype=np.int32)
    accept_len = np.zeros(B, dtype=np.int32)
    p_draft = np.zeros(total_k, dtype=np.float64)
    q_draft = np.zeros(total_k, dtype=np.float64)
    traces = {}
    for b in range(B):
        K = ragged_draft_count(cu, b, total_k, k_max)
        T = float(temperature[b])
        if K is None or not (math.isfinite(T) and T > 0):
            continue
        c0 = int(cu[b])
        p_rows = [softmax_t(logits_f64(target_rows[c0 + b + i], target_dtype), T).tolist()
                  for i in range(K + 1)]
        x = [int(v) for v in draft_tokens[c0:c0 + K]]
        if draft_rows is not None:
            q_rows = [softmax_t(logits_f64(draft_rows[c0 + i], draft_dtype), T).tolist()
                      for i in range(K)]
        else:
            q_rows = [onehot(V, x[i]) for i in range(K)]
        pairs = [request_uniforms(int(seeds[b]), b, i, int(offset)) for i in range(K + 1)]
        res = verify_request(p_rows, q_rows, x, [u for u, _ in pairs], [u for _, u in pairs])
        tokens[b, :res["accept_len"]] = res["tokens"]
        accept_len[b] = res["accept_len"]
        p_draft[c0:c0 + K] = res["p_x"]
        q_draft[c0:c0 + K] = res["q_x"]
        if keep_trace:
            traces[b] = res
    return tokens, accept_len, p_draft, q_draft, traces


def spec_verify_greedy_ragged(target_rows, cu, draft_tokens, k_max=None, dtype="f32"):
    """Greedy verification of a ragged batch (layout as above).

    Returns (tokens [B, k_max + 1], accept_len [B], argmax [total_k + B]);
    argmax rows of refused requests stay -1.
    """
    B = len(cu) - 1
    total_k = len(draft_tokens)
    if k_max is None:
        k_max = max([0] + [int(cu[b + 1]) - int(cu[b]) for b in range(B)])
    tokens = np.full((B, k_max + 1), -1, dtype=np.int32)
    accept_len = np.zeros(B, dtype=np.int32)
    g_all = np.full(total_k + B, -1, dtype=np.int32)
    for b in range(B):
        K = ragged_draft_count(cu, b, total_k, k_max)
        if K is None:
            continue
        c0 = int(cu[b])
        g = [argmax_lowest(logits_f64(target_rows[c0 + b + i], dtype)) for i in range(K + 1)]
        g_all[c0 + b:c0 + b + K + 1] = g
        a = 0
        while a < K and int(draft_tokens[c0 + a]) == g[a]:
            a += 1
        tokens[b, :a] = draft_tokens[c0:c0 + a]
        tokens[b, a] = g[a]
        accept_len[b] = a + 1
    return tokens, accept_len, g_all


# ------------------------------------------------------- greedy and tree ---

def argmax_lowest(row) -> int:
    """Index of the largest value, the lowest such index on ties (numpy's argmax rule)."""
    return int(np.argmax(np.asarray(row, dtype=np.float64)))


def spec_verify_greedy(target, draft_tokens, dtype="f32", bitmask=None):
    """Greedy (argmax-match) verification.

    Returns (tokens [B, K+1] -1 padded, accept_len [B], argmax [B, K+1]).
    ``bitmask`` (optional) as in spec_verify_sample: argmax over allowed tokens.
    """
    B, R, V = target.shape
    K = R - 1
    tokens = np.full((B, K + 1), -1, dtype=np.int32)
    accept_len = np.zeros(B, dtype=np.int32)
    g = np.zeros((B, K + 1), dtype=np.int32)
    for b in range(B):
        for i in range(K + 1):
            l = logits_f64(target[b, i], dtype)
            g[b, i] = argmax_lowest(l if bitmask is None else apply_bitmask(l, bitmask[b, i]))
        a = 0
        while a < K and int(draft_tokens[b, a]) == g[b, a]:
            a += 1
        tokens[b, :a] = draft_tokens[b, :a]
        tokens[b, a] = g[b, a]
        accept_len[b] = a + 1
    return tokens, accept_len, g


def tree_depths(parents) -> list:
    """Depth of every node; parents[0] = -1 and 0 <= parents[n] < n are required."""
    parents = [int(p) for p in parents]
    if not parents or parents[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    depth = [0]
    for n in range(1, len(parents)):
        if not 0 <= parents[n] < n:
            raise ValueError(f"parent of node {n} must precede it")
        depth.append(depth[parents[n]] + 1)
    return depth


def spec_verify_tree(target, node_tokens, parents, dtype="f32"):
    """Greedy verification of a static draft tree (Medusa style), or of a
    tree per request (dynamic trees, EAGLE-2: "推测解码与 MTP" §4.3).

    target [B, N, V]: logits at every node (row n predicts the token after
    node n); node_tokens [B, N] (column 0, the root, is ignored); parents
    [N] (one tree for the batch; a malformed one raises ValueError) or
    [B, N] (row b is request b's tree; a request whose row is not a tree is
    refused: tokens -1, accept_len 0, best_node -1).
    Returns (tokens [B, N] -1 padded, accept_len [B], best_node [B]).
    """
    B, N, V = target.shape
    par = np.asarray(parents)
    per_request = par.ndim == 2
    shared_depth = None if per_request else tree_depths(par)
    tokens = np.full((B, N), -1, dtype=np.int32)
    accept_len = np.zeros(B, dtype=np.int32)
    best_node = np.zeros(B, dtype=np.int32)
    for b in range(B):
        pb = par[b] if per_request else par
        if per_request:
            try:
                depth = tree_depths(pb)
            except ValueError:
                best_node[b] = -1
                continue
        else:
            depth = shared_depth
        g = [argmax_lowest(logits_f64(target[b, n], dtype)) for n in range(N)]
        acc = [True] + [False] * (N - 1)
        for n in range(1, N):
            p = int(pb[n])
            acc[n] = acc[p] and int(node_tokens[b, n]) == g[p]
        best = 0
        for n in range(1, N):
            if acc[n] and depth[n] > depth[best]:
                best = n
        path = []
        n = best
        while n != 0:
            path.append(int(node_tokens[b, n]))
            n = int(pb[n])
        path.reverse()
        row = path + [g[best]]
        tokens[b, :len(row)] = row
        accept_len[b] = len(row)
        best_node[b] = best
    return tokens, accept_len, best_node
