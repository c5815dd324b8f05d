"""Compare the HIP library's outputs with the fp64 oracle's (test helper).

Greedy and tree outputs must match exactly. For stochastic verification the
two sides use the same uniforms, so tokens must match except where a uniform
lies within TOL of a decision boundary of the oracle's fp64 arithmetic:
  * accept/reject at position i: |u_i - min(1, p_i(x_i)/q_i(x_i))| < TOL
  * the drawn token: the library's token must own an interval
    [C_{y-1}/Z, C_y/Z] of the oracle's CDF within TOL of u.
Such divergences are counted (and the rest of that request skipped); any
other difference is a mismatch. Band counts at 1e-5, 1e-6 and 1e-7 record
how many draws were that close to a boundary at all.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

TOL = 1e-5
PROB_TOL = 1e-5
TAUS = (1e-5, 1e-6, 1e-7)
# A top-p cut whose bracketing cumulative masses lie within FILTER_TOL of
# top_p may fall one value either side (the library sums fp64 weights of
# relative error ~1e-15 in another order): such requests are counted and
# only checked for validity.
FILTER_TOL = 1e-9


def to_device(wl, dev, draft_bf16=False):
    """Host workload arrays -> device tensors in the library's layout."""
    if wl["dtype"] == "bf16":
        tgt = torch.from_numpy(np.ascontiguousarray(wl["target"]).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        tgt = torch.from_numpy(np.ascontiguousarray(wl["target"])).to(dev)
    out = dict(target=tgt, tokens=torch.from_numpy(np.ascontiguousarray(wl["draft_tokens"])).to(dev),
               seeds=torch.from_numpy(wl["seeds"].view(np.int64)).to(dev), draft=None, temperature=None)
    if wl.get("draft") is not None:
        d = wl["draft"]
        if draft_bf16:
            out["draft"] = torch.from_numpy(d.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            out["draft"] = torch.from_numpy(np.ascontiguousarray(d)).to(dev)
    if wl.get("temperature") is not None:
        out["temperature"] = torch.from_numpy(wl["temperature"]).to(dev)
    return out


def new_report():
    return dict(requests=0, exact=0, refused=0, accept_div=0, select_div=0, filter_near=0, mismatches=[],
                near_accept={t: 0 for t in TAUS}, near_select={t: 0 for t in TAUS},
                max_p_err=0.0, max_q_err=0.0)


def near_cut_invalid(wl, b, tok, n, top_k, top_p, draft_dtype):
    """Checks a request whose top-p cut lies within FILTER_TOL of a cumulative
    mass, where the library may keep one value more or fewer than the oracle:
    the accepted prefix must be the drafts, the rest -1, and the drawn token
    must lie in the larger of the two candidate kept sets of the row it was
    drawn from (the set kept at top_p + FILTER_TOL), and differ from a
    rejected one-hot draft. Returns what is wrong, or "" when valid."""
    K, V = wl["K"], wl["V"]
    if not 1 <= n <= K + 1:
        return f"accept_len {n}"
    a = n - 1
    if not np.array_equal(tok[:a], wl["draft_tokens"][b, :a]):
        return "accepted prefix differs from the drafts"
    if np.any(tok[a + 1:] != -1):
        return "padding"
    y = int(tok[a])
    if not 0 <= y < V:
        return f"token {y} out of range"
    T = float(wl["temperature"][b])
    tk = 0 if top_k is None else int(top_k[b])
    tp = 1.0 if top_p is None else float(top_p[b])
    row = oracle.logits_f64(wl["target"][b, a], wl["dtype"])
    keep_large, _ = oracle.filter_keep(row, T, tk, min(tp + FILTER_TOL, 1.0))
    if not keep_large[y]:
        return f"token {y} outside both candidate kept sets"
    if wl.get("draft") is None and a < K and y == int(wl["draft_tokens"][b, a]):
        return "the rejected one-hot draft was drawn again"
    return ""


def classify_sample(wl, g_tok, g_len, g_p, g_q, requests=None, draft_dtype="f32", report=None,
                    bitmask=None, lazy=False, top_k=None, top_p=None, oracle_out=None):
    """Run the oracle on `requests` and fold the comparison into a report dict.

    lazy: the outputs of early-exit verification, which computes p and q only
    up to the position where a request stopped and leaves 0 after it.
    g_p / g_q may be None (a call that returned tokens only): p and q are then
    not compared. oracle_out: the oracle's (tokens, accept_len, p, q, traces)
    for these requests, already computed with keep_trace (it is not run again)."""
    rep = new_report() if report is None else report
    B, K, V = wl["B"], wl["K"], wl["V"]
    reqs = list(range(B)) if requests is None else list(requests)
    if oracle_out is None:
        oracle_out = oracle.spec_verify_sample(
            wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"], wl["seeds"],
            wl["offset"], target_dtype=wl["dtype"], draft_dtype=draft_dtype, requests=reqs,
            keep_trace=True, bitmask=bitmask, top_k=top_k, top_p=top_p)
    o_tok, o_len, o_p, o_q, traces = oracle_out
    for b in reqs:
        rep["requests"] += 1
        if b not in traces:                               # refused by the oracle
            if g_len[b] == 0 and np.all(g_tok[b] == -1):
                rep["refused"] += 1
            else:
                rep["mismatches"].append((b, "refusal", int(g_len[b])))
            continue
        tr = traces[b]
        if tr.get("filter_margin", np.inf) < FILTER_TOL:
            rep["filter_near"] += 1
            bad = near_cut_invalid(wl, b, g_tok[b], int(g_len[b]), top_k, top_p, draft_dtype)
            if bad:
                rep["mismatches"].append((b, "invalid output near a top-p cut: " + bad, g_tok[b].tolist()))
            continue
        n = min(max(int(g_len[b]), 0), K) if lazy else K
        if g_p is None:
            n = 0
        elif n:
            rep["max_p_err"] = max(rep["max_p_err"], float(np.max(np.abs(g_p[b, :n] - o_p[b, :n]))))
            rep["max_q_err"] = max(rep["max_q_err"], float(np.max(np.abs(g_q[b, :n] - o_q[b, :n]))))
        if g_p is not None and n < K and (np.any(g_p[b, n:] != 0) or np.any(g_q[b, n:] != 0)):
            rep["mismatches"].append((b, "p/q after the stop", g_p[b, n:].tolist(), g_q[b, n:].tolist()))
            continue
        a_o, a_g = int(o_len[b]) - 1, int(g_len[b]) - 1
        if not 0 <= a_g <= K:
            rep["mismatches"].append((b, "accept_len", a_g + 1))
            continue
        margins = []
        for i in range(min(a_o + 1, K)):
            p, q, u = tr["p_x"][i], tr["q_x"][i], tr["u_acc"][i]
            margins.append(abs(u - min(1.0, p / q)) if q > 0 else np.inf)
        for m in margins:
            for t in TAUS:
                rep["near_accept"][t] += m < t
        if a_o != a_g:
            j = min(a_o, a_g)
            if j < len(margins) and margins[j] < TOL:
                rep["accept_div"] += 1
            else:
                rep["mismatches"].append((b, "accept", a_o, a_g))
            continue
        a = a_o
        if not np.array_equal(g_tok[b, :a], wl["draft_tokens"][b, :a]) or np.any(g_tok[b, a + 1:] != -1):
            rep["mismatches"].append((b, "layout", g_tok[b].tolist()))
            continue
        w = np.asarray(tr["weights"], dtype=np.float64)
        cum = np.cumsum(w)
        Z = cum[-1]
        u = tr["u_select"]
        y_o, y_g = int(o_tok[b, a]), int(g_tok[b, a])

        def interval(y):
            lo = cum[y - 1] / Z if y > 0 else 0.0
            return lo, cum[y] / Z

        lo, hi = interval(y_o)
        d = min(u - lo, hi - u)
        for t in TAUS:
            rep["near_select"][t] += d < t
        if y_g == y_o:
            rep["exact"] += 1
        elif 0 <= y_g < V:
            lo_g, hi_g = interval(y_g)
            if max(lo_g - u, u - hi_g, 0.0) <= TOL:
                rep["select_div"] += 1
            else:
                rep["mismatches"].append((b, "select", y_o, y_g, float(u), float(lo_g), float(hi_g)))
        else:
            rep["mismatches"].append((b, "select_range", y_o, y_g))
    return rep


def record_report(rep, name):
    """Appends the report (counts only) as one JSON line to the file named by
    SV_PARITY_LOG, when that variable is set."""
    path = os.environ.get("SV_PARITY_LOG")
    if not path:
        return
    row = dict(name=name, **{k: rep[k] for k in ("requests", "exact", "refused", "accept_div", "select_div",
                                                  "filter_near")},
               near_accept={str(t): int(v) for t, v in rep["near_accept"].items()},
               near_select={str(t): int(v) for t, v in rep["near_select"].items()},
               max_p_err=rep["max_p_err"], max_q_err=rep["max_q_err"], mismatches=len(rep["mismatches"]))
    with open(path, "a") as f:
        f.write(json.dumps(row) + "\n")


def assert_report(rep, name):
    record_report(rep, name)
    print(f"[parity] {name}: requests={rep['requests']} exact={rep['exact']} refused={rep['refused']} "
          f"accept_div={rep['accept_div']} select_div={rep['select_div']} "
          f"filter_near={rep['filter_near']} "
          f"near_accept={rep['near_accept']} near_select={rep['near_select']} "
          f"max|dp|={rep['max_p_err']:.2e} max|dq|={rep['max_q_err']:.2e} "
          f"mismatches={len(rep['mismatches'])}", flush=True)
    assert not rep["mismatches"], rep["mismatches"][:10]
    assert rep["max_p_err"] < PROB_TOL and rep["max_q_err"] < PROB_TOL
    # divergences only ever happen at near-threshold draws
    assert rep["accept_div"] <= rep["near_accept"][1e-5]
    assert rep["select_div"] <= rep["near_select"][1e-5]
