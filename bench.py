#!/usr/bin/env python3
"""Throughput of batched speculative-decoding verification on one MI355X.

One step = one call of the verification entry point over one batch of
synthetic logits already resident in HBM (all kernels of the path). The
default workload is B=256 requests, K=5 one-hot drafts, V=128256, bf16
target logits, T=0.7 (``c3_onehot`` in ``workloads``). Inputs rotate over
several copies so the 256 MB memory-side cache cannot serve them.

Prints one JSON line: logits GB/s (algorithmic bytes / step time), us/step,
the dominant kernel's roofline, and the fp64 CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import multiprocessing
import os
import sys
import time

# The CPU baseline's worker processes each run one thread of numpy (BLAS
# threads = 1); set before numpy is imported anywhere in this process.
for _v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "spec-verify µs/step and logits GB/s (% HBM peak) at B=256,K=5,V=128256"


def source_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "draft_verification_05_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


CHUNK_BYTES = 4096        # the draw re-reads one 4 KiB chunk of logits per request
RAGGED_BASE = {"c3_ragged": "c3_onehot"}   # ragged workloads: base workload cut to K_b per request
MASKED_BASE = {"c3_masked": "c3_onehot"}   # grammar-masked workloads: base workload + a bitmask
LAZY_BASE = {"c3_lazy": "c3_onehot", "c2_lazy": "c2_stoch"}   # early-exit verification of a workload
# top-k / top-p filtered verification: base workload, top_k, top_p (the pages' top_p 0.95)
FILTER_BASE = {"c3_topp": ("c3_onehot", 0, 0.95), "c2_topp": ("c2_stoch", 0, 0.95),
               "c3_topp_tok": ("c3_onehot", 0, 0.95)}
# calls that ask for tokens and accept lengths only (no p / q outputs), as a
# serving engine would
TOKENS_ONLY = {"c3_topp_tok"}
# one GPU's share of a workload whose requests are split over several GPUs
# (requests are independent: each GPU verifies B / G of them, no exchange)
SHARD_BASE = {"c3_shard8": ("c3_onehot", 8)}


def algorithmic_bytes(wl, rejected=None) -> int:
    """Bytes one call must read: every logits row the rule consults once
    (B*(K+1) target rows, plus B*K draft rows when q is explicit; a ragged
    batch consults sum(K_b + 1) and sum(K_b)), plus the draw's one chunk per
    request, plus (explicit drafts only) the stop rows of target and draft
    again for each request that rejected (`rejected` requests; all B when
    unknown). Greedy and tree draw nothing."""
    es = 2 if wl["dtype"] == "bf16" else 4
    B, V = wl["B"], wl["V"]
    if wl["mode"] == "tree":
        return B * len(wl["parents"]) * V * es
    K = wl["K"]
    explicit = wl.get("draft") is not None
    if wl.get("ragged") is not None:
        nk = int(wl["ragged"]["ks"].sum())
        total = (nk + B + (nk if explicit else 0)) * V * es
    else:
        total = B * (K + 1 + (K if explicit else 0)) * V * es
    if wl.get("bitmask") is not None:               # one mask row per consulted row
        total += wl["bitmask"].nbytes // (K + 1) * (K + 1 + (K if explicit else 0))
    if wl["mode"] == "sample":
        total += B * min(CHUNK_BYTES, V * es)
        if explicit:
            total += (B if rejected is None else rejected) * 2 * V * es
    return total


def lazy_bytes(wl, accept) -> int:
    """Bytes early-exit verification reads: windows of positions [0], then
    [1, K], are read in rounds, so a request that stopped at position a
    (accept length a + 1) read target rows 0..e and draft rows 0..min(e, K - 1),
    with e the end of a's window; plus the draw's chunk, plus (explicit
    drafts) the stop rows again for the residual when a < K."""
    import numpy as np
    es = 2 if wl["dtype"] == "bf16" else 4
    K, V = wl["K"], wl["V"]
    explicit = wl.get("draft") is not None
    a = accept.astype(np.int64) - 1
    ends, lo, w = [], 0, 1
    while lo <= K:
        ends.append(min(lo + w - 1, K))
        lo, w = lo + w, K
    e = np.array([next(x for x in ends if x >= ai) for ai in a], dtype=np.int64)
    rows = (e + 1) + (np.minimum(e + 1, K) if explicit else 0)
    total = int(rows.sum()) * V * es + len(a) * min(CHUNK_BYTES, V * es)
    if explicit:
        total += int((a < K).sum()) * 2 * V * es
    return total


def traffic_record(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def read_ceiling(copies, torch, steps: int) -> dict:
    """Times the read-only probe (draft_verification_05_amd/probe) over the
    logits copies: GB/s of one full read of the same bytes (rounded down to
    whole 4 KiB chunks)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "draft_verification_05_amd", "libsvprobe.so"))
    lib.sv_probe_read.restype = ctypes.c_int
    lib.sv_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.sv_probe_workgroups.restype = ctypes.c_int
    lib.sv_probe_workgroups.argtypes = [ctypes.c_size_t]
    nbytes = copies[0].numel() * copies[0].element_size() // 4096 * 4096
    if nbytes == 0:
        return {"kernel": "read-only probe", "bytes": 0, "us": None, "gbps": None}
    dev = copies[0].device
    out = torch.empty(lib.sv_probe_workgroups(nbytes), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    iters = max(10, min(steps, 100))

    def run(i):
        rc = lib.sv_probe_read(copies[i % len(copies)].data_ptr(), nbytes, out.data_ptr(), stream)
        if rc:
            raise RuntimeError(f"sv_probe_read failed ({rc})")
    for i in range(len(copies)):
        run(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    return {"kernel": "read-only probe over the same logits bytes (4 KiB runs, 16-byte loads)",
            "bytes": nbytes, "us": round(ms * 1e3, 2), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


# The workload the CPU-baseline workers see: set before the pool forks them,
# so each inherits it without a copy through a pipe.
_CPU_WL = None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers() -> int:
    """Worker processes for the CPU baseline: every core the process may use,
    at most 16 (a GPU machine's share of its host for one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, os.cpu_count() or n, 16))


def oracle_request(wl, n, offset):
    """The oracle on request n alone at `offset` (what one CPU unit of work is).
    Returns the oracle's full output tuple (only row n filled)."""
    import numpy as np
    import oracle
    if wl["mode"] == "greedy":
        return oracle.spec_verify_greedy(wl["target"][n:n + 1], wl["draft_tokens"][n:n + 1], wl["dtype"])
    if wl["mode"] == "tree":
        return oracle.spec_verify_tree(wl["target"][n:n + 1], wl["draft_tokens"][n:n + 1], wl["parents"],
                                       wl["dtype"])
    rg = wl.get("ragged")
    if rg is None:
        return oracle.spec_verify_sample(wl["target"], wl["draft"], wl["draft_tokens"], wl["temperature"],
                                         wl["seeds"], offset, target_dtype=wl["dtype"], requests=[n],
                                         keep_trace=True, bitmask=wl.get("bitmask"),
                                         top_k=wl.get("top_k"), top_p=wl.get("top_p"))
    c0, c1 = int(rg["cu"][n]), int(rg["cu"][n + 1])       # request n as a one-request ragged batch
    return oracle.spec_verify_sample_ragged(
        rg["target_rows"][c0 + n: c1 + n + 1], None, np.array([0, c1 - c0], np.int32),
        rg["draft_tokens"][c0:c1], wl["temperature"][n:n + 1], wl["seeds"][n:n + 1], offset,
        k_max=wl["K"], target_dtype=wl["dtype"])


def request_rows(wl, n) -> int:
    """Logits rows request n consults (the unit the sample is stated in)."""
    if wl["mode"] == "tree":
        return len(wl["parents"])
    rg = wl.get("ragged")
    k = int(rg["ks"][n]) if rg is not None else wl["K"]
    return k + 1 + (k if wl.get("draft") is not None else 0)


def _cpu_shard(args):
    """One worker: requests lo, lo + 1, ... < hi, round and round, until
    `seconds` have passed. Returns the requests done and the time taken."""
    lo, hi, seconds, offset = args
    t0 = time.perf_counter()
    done = 0
    while time.perf_counter() - t0 < seconds:
        oracle_request(_CPU_WL, lo + done % (hi - lo), offset)
        done += 1
    return done, time.perf_counter() - t0


def cpu_baseline(wl, seconds: float, pool, offset: int, gpu_out):
    """The fp64 oracle (untuned) on the host cores, on a bounded sample of the
    same workload: (i) one thread in this process, whose requests are also
    compared with the GPU's outputs of the last call at the same offset;
    (ii) `pool`'s worker processes, requests sharded between them. Each leg
    runs about `seconds`; throughput is the bytes of the requests done
    (the step's algorithmic bytes pro rata) over the leg's wall time."""
    import numpy as np
    B = wl["B"]
    per_req = algorithmic_bytes(wl) / B
    # (i) one thread: requests 0, 1, ... (round and round when the batch is
    # quick), the first pass kept for the parity counts
    outs = []
    n1 = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        o = oracle_request(wl, n1 % B, offset)
        if n1 < B:
            outs.append(o)
        n1 += 1
    dt1 = time.perf_counter() - t0
    rows1 = sum(request_rows(wl, n % B) for n in range(n1))
    single = {"value": round(per_req * n1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
              "sample": f"{n1} requests in order from request 0 of {B} ({rows1} logits rows), "
                        f"{dt1:.1f} s",
              "us_per_step_equiv": round(dt1 / n1 * B * 1e6, 1)}
    # (ii) worker processes, a contiguous shard of requests each
    workers = pool._processes
    shard = (B + workers - 1) // workers
    jobs = [(w * shard, min(B, (w + 1) * shard), seconds, offset) for w in range(workers) if w * shard < B]
    t0 = time.perf_counter()
    res = pool.map(_cpu_shard, jobs)
    dtn = time.perf_counter() - t0
    done = sum(r[0] for r in res)
    rowsn = sum(request_rows(wl, j[0] + k % (j[1] - j[0])) for j, r in zip(jobs, res) for k in range(r[0]))
    multi = {"value": round(per_req * done / dtn / 1e9, 4), "unit": "GB/s", "cores": len(jobs),
             "kind": "oracle", "cpu_model": cpu_model(), "host_cores": os.cpu_count(),
             "sample": f"{done} requests of the {B} of {wl['name']} ({rowsn} logits rows), sharded "
                       f"over {len(jobs)} worker processes (one numpy thread each), {dtn:.1f} s wall",
             "us_per_step_equiv": round(dtn / max(done, 1) * B * 1e6, 1),
             "single_thread": single}
    multi["parity"] = parity_of_sample(wl, outs, offset, gpu_out)
    return multi


def parity_of_sample(wl, outs, offset, gpu_out):
    """The GPU's last call against the oracle on the single-thread leg's
    requests: the sound parity counts for sampling (tests/parity.py: exact,
    divergences only at draws within 1e-5 of a threshold, band counts at
    1e-5 / 1e-6 / 1e-7, mismatches), exact-match counts for greedy and tree."""
    import numpy as np
    n = len(outs)
    g_tok, g_len = gpu_out["tokens"], gpu_out["accept_len"]
    if wl["mode"] in ("greedy", "tree"):
        same = sum(int(np.array_equal(o[0][0], g_tok[i]) and o[1][0] == g_len[i]) for i, o in enumerate(outs))
        return {"requests": n, "exact": same, "mismatches": n - same, "offset": offset}
    if wl.get("ragged") is not None:
        same = 0
        for i, o in enumerate(outs):
            k = int(wl["ragged"]["ks"][i])
            same += int(o[1][0] == g_len[i] and np.array_equal(o[0][0][:k + 1], g_tok[i][:k + 1]))
        return {"requests": n, "identical": same, "offset": offset,
                "note": "ragged: requests identical to the oracle (no near-threshold classification)"}
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import classify_sample
    B, K = wl["B"], wl["K"]
    o_tok = np.full((B, K + 1), -1, np.int32)
    o_len = np.zeros(B, np.int32)
    o_p = np.zeros((B, K))
    o_q = np.zeros((B, K))
    traces = {}
    for i, o in enumerate(outs):
        o_tok[i], o_len[i], o_p[i], o_q[i] = o[0][i], o[1][i], o[2][i], o[3][i]
        traces.update(o[4])
    rep = classify_sample(dict(wl, offset=offset), g_tok, g_len, gpu_out.get("p"), gpu_out.get("q"),
                          requests=range(n), bitmask=wl.get("bitmask"), lazy=gpu_out.get("lazy", False),
                          top_k=wl.get("top_k"), top_p=wl.get("top_p"),
                          oracle_out=(o_tok, o_len, o_p, o_q, traces))
    return {"requests": rep["requests"], "exact": rep["exact"], "refused": rep["refused"],
            "accept_div": rep["accept_div"], "select_div": rep["select_div"],
            "filter_near": rep["filter_near"],
            "near_accept": {str(t): int(v) for t, v in rep["near_accept"].items()},
            "near_select": {str(t): int(v) for t, v in rep["near_select"].items()},
            "max_abs_dp": rep["max_p_err"], "max_abs_dq": rep["max_q_err"],
            "mismatches": len(rep["mismatches"]), "offset": offset}


def launches_per_call(wl, workload, lazy, filt, explicit) -> int:
    """Kernel launches one call makes (the library's launch plan for these
    shapes: one-launch calls for one-hot, greedy and tree batches up to 1024
    requests whose rule fits in registers; draft logits add a residual pass;
    early exit takes two rounds; filtered bf16 rows, and fp32 rows of at most
    32768 logits, take one select kernel and then the rule with its draw (or
    the residual pass), longer filtered fp32 rows the row pass, the select
    pass and the rule)."""
    if lazy:
        return 2 + (1 if explicit else 0)
    if filt:
        return 2 if wl["dtype"] == "bf16" or wl["V"] <= 32768 else 3
    if wl["mode"] == "sample" and explicit:
        return 2
    return 1 if wl["B"] <= 1024 else 2


def roofline_kernel(wl, lazy, filt, explicit, n) -> str:
    if n == 1:
        return ("sv_rows_kernel, one launch per call (row pass + per-request rule); "
                "algorithmic bytes of the call / its kernel time")
    if filt and (wl["dtype"] == "bf16" or wl["V"] <= 32768):
        sel = "one-pass select" if wl["dtype"] == "bf16" else "LDS-resident select"
        what = sel + " + " + ("residual pass (rule and draw)" if explicit else "rule and draw")
        return f"whole call, {n} launches ({what}); algorithmic bytes / call time"
    what = ("early-exit rounds over position windows [0], [1, K]" if lazy else
            "row pass + select pass + rule" if filt else "row pass + rule")
    return (f"whole call, {n} launches ({what}{' + residual pass' if explicit else ''}); "
            "algorithmic bytes / call time")


def run_copy(args):
    """Plain device copy of a known size (calibrates the HBM byte counters)."""
    import torch
    n = 1 << 28                                # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                      "launches": args.steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3_onehot",
                    help="c1_tiny, c2_stoch, c3_onehot, c4_greedy, c5_tree, c3_ragged "
                         "(C3 with per-request draft counts K_b ~ uniform{0..5}) or c3_masked "
                         "(C3 with a grammar bitmask allowing each token w.p. 1/2); c3_lazy / c2_lazy "
                         "run C3 / C2 through early-exit verification; c3_topp / c2_topp "
                         "add a top_p 0.95 filter; c3_topp_tok is c3_topp returning tokens "
                         "and accept lengths only; c3_shard8 is one GPU's share of C3 split "
                         "over 8 GPUs (B=32)")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed steps for at least this long before the warmup steps (GPU clocks)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["verify", "copy"], default="verify")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verification path has no multi-GPU form here "
              "(requests would shard across GPUs with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np

    if args.mode == "copy":
        return run_copy(args)

    from workloads import make

    ragged = args.workload in RAGGED_BASE
    masked = args.workload in MASKED_BASE
    lazy = args.workload in LAZY_BASE
    filt = args.workload in FILTER_BASE
    tok_only = args.workload in TOKENS_ONLY
    if filt:
        base, f_k, f_p = FILTER_BASE[args.workload]
        wl = dict(make(base, data_seed=0), name=args.workload)
        wl["top_k"] = np.full(wl["B"], f_k, np.int32)
        wl["top_p"] = np.full(wl["B"], f_p, np.float32)
    elif lazy:
        wl = dict(make(LAZY_BASE[args.workload], data_seed=0), name=args.workload)
    elif ragged:
        from workloads import make_ragged
        wl = make_ragged(RAGGED_BASE[args.workload], data_seed=0)
    elif masked:
        from workloads import make_masked
        wl = make_masked(MASKED_BASE[args.workload], data_seed=0)
    elif args.workload in SHARD_BASE:
        base, g = SHARD_BASE[args.workload]
        full = make(base, data_seed=0)
        wl = dict(make(base, data_seed=0, B=full["B"] // g), name=args.workload)
    else:
        wl = make(args.workload, data_seed=0)
    # The CPU baseline's worker processes are forked now, before this process
    # makes its first GPU call; they inherit the workload.
    pool = None
    if not args.no_cpu_baseline:
        global _CPU_WL
        _CPU_WL = wl
        pool = multiprocessing.get_context("fork").Pool(cpu_workers())

    import torch
    import draft_verification_05_amd as sv

    dev = torch.device("cuda:0")
    lib = sv.load_library()
    B, K, V = wl["B"], wl["K"], wl["V"]
    mode = wl["mode"]

    host_t = wl["ragged"]["target_rows"] if ragged else wl["target"]
    if wl["dtype"] == "bf16":
        tgt0 = torch.from_numpy(host_t.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        tgt0 = torch.from_numpy(host_t).to(dev)
    copies = [tgt0] + [tgt0.clone() for _ in range(max(args.copies, 1) - 1)]
    draft = None
    if wl.get("draft") is not None:
        d0 = torch.from_numpy(wl["draft"]).to(dev)
        draft = [d0] + [d0.clone() for _ in range(max(args.copies, 1) - 1)]
    tokens = torch.from_numpy(wl["ragged"]["draft_tokens"] if ragged else wl["draft_tokens"]).to(dev)
    if ragged:
        cu = torch.from_numpy(wl["ragged"]["cu"]).to(dev)
        total_k = int(wl["ragged"]["ks"].sum())
    if masked:
        bitmask = torch.from_numpy(wl["bitmask"].view(np.int32)).to(dev)
    out_tok = torch.empty((B, tokens.shape[1] if mode == "tree" else K + 1), dtype=torch.int32, device=dev)
    out_len = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    if mode == "sample":
        temp = torch.from_numpy(wl["temperature"]).to(dev)
        seeds = torch.from_numpy(wl["seeds"].view(np.int64)).to(dev)
        out_p = torch.empty((total_k if ragged else B * K,), dtype=torch.float32, device=dev)
        out_q = torch.empty((total_k if ragged else B * K,), dtype=torch.float32, device=dev)
        ws_bytes = sv.spec_verify_workspace_size(sv.SV_OP_SAMPLE, B, K, V, draft is not None)
        if filt:
            top_k = torch.full((B,), f_k, dtype=torch.int32, device=dev)
            top_p = torch.full((B,), f_p, dtype=torch.float32, device=dev)
    elif mode == "greedy":
        out_g = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        ws_bytes = sv.spec_verify_workspace_size(sv.SV_OP_GREEDY, B, K, V)
    else:
        N = len(wl["parents"])
        parents = (ctypes.c_int32 * N)(*[int(v) for v in wl["parents"]])
        out_best = torch.empty(B, dtype=torch.int32, device=dev)
        ws_bytes = sv.spec_verify_workspace_size(sv.SV_OP_TREE, B, N, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    sv.spec_verify_workspace_init(ws)

    descs = [sv._rows_desc(t, "target") if ragged else sv._desc(t, "target") for t in copies]
    ddescs = [sv._desc(t, "draft") for t in draft] if draft is not None else None

    def step(i):
        c = i % len(copies)
        if ragged:
            rc = lib.spec_verify_sample_ragged(ctypes.byref(descs[c]), None, cu.data_ptr(), total_k,
                                               tokens.data_ptr(), temp.data_ptr(), seeds.data_ptr(), i,
                                               B, K, V, out_tok.data_ptr(), out_len.data_ptr(),
                                               out_p.data_ptr(), out_q.data_ptr(), ws.data_ptr(),
                                               ws_bytes, stream)
        elif filt:
            rc = lib.spec_verify_sample_filtered(ctypes.byref(descs[c]),
                                                 ctypes.byref(ddescs[c]) if ddescs else None,
                                                 tokens.data_ptr(), temp.data_ptr(), top_k.data_ptr(),
                                                 top_p.data_ptr(), seeds.data_ptr(), i, B, K, V,
                                                 out_tok.data_ptr(), out_len.data_ptr(),
                                                 None if tok_only else out_p.data_ptr(),
                                                 None if tok_only else out_q.data_ptr(),
                                                 ws.data_ptr(), ws_bytes, stream)
        elif lazy:
            rc = lib.spec_verify_sample_lazy(ctypes.byref(descs[c]),
                                             ctypes.byref(ddescs[c]) if ddescs else None,
                                             tokens.data_ptr(), temp.data_ptr(), seeds.data_ptr(), i,
                                             B, K, V, out_tok.data_ptr(), out_len.data_ptr(),
                                             out_p.data_ptr(), out_q.data_ptr(), ws.data_ptr(),
                                             ws_bytes, stream)
        elif masked:
            rc = lib.spec_verify_sample_masked(ctypes.byref(descs[c]),
                                               ctypes.byref(ddescs[c]) if ddescs else None,
                                               tokens.data_ptr(), bitmask.data_ptr(), temp.data_ptr(),
                                               seeds.data_ptr(), i, B, K, V, out_tok.data_ptr(),
                                               out_len.data_ptr(), out_p.data_ptr(), out_q.data_ptr(),
                                               ws.data_ptr(), ws_bytes, stream)
        elif mode == "sample":
            rc = lib.spec_verify_sample(ctypes.byref(descs[c]),
                                        ctypes.byref(ddescs[c]) if ddescs else None,
                                        tokens.data_ptr(), temp.data_ptr(), seeds.data_ptr(), i, B, K, V,
                                        out_tok.data_ptr(), out_len.data_ptr(), out_p.data_ptr(),
                                        out_q.data_ptr(), ws.data_ptr(), ws_bytes, stream)
        elif mode == "greedy":
            rc = lib.spec_verify_greedy(ctypes.byref(descs[c]), tokens.data_ptr(), B, K, V,
                                        out_tok.data_ptr(), out_len.data_ptr(), out_g.data_ptr(),
                                        ws.data_ptr(), ws_bytes, stream)
        else:
            rc = lib.spec_verify_tree(ctypes.byref(descs[c]), tokens.data_ptr(),
                                      ctypes.cast(parents, ctypes.c_void_p), N, B, V,
                                      out_tok.data_ptr(), out_len.data_ptr(), out_best.data_ptr(),
                                      ws.data_ptr(), ws_bytes, stream)
        if rc:
            raise sv.SpecVerifyError(rc, "bench step")

    # Clock settle: the GPU leaves its idle clocks only after some ms of
    # sustained load (a first round of 200 calls measured ~5% slower than
    # the next), so steps run untimed for at least `settle_s` before the W
    # warmup steps; their offsets are distinct from every timed step's.
    settle_calls = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            step(10_000_000 + settle_calls)
            settle_calls += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly K back-to-back steps between two events on the
    # launch stream (no events in between, so nothing pads the steps).
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    region0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    region1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    region_ms = region0.elapsed_time(region1)

    # Per-call durations: a second pass with an event pair around every call
    # (both launches of the call; the events add a small gap between calls).
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record()
        step(args.warmup + args.steps + i)
        ends[i].record()
    torch.cuda.synchronize()

    # Read-stream ceiling: a read-only probe kernel (4 KiB runs, 16-byte
    # loads, nothing else) over the same logits bytes, rotating over the same
    # copies, timed the same way.
    stream = read_ceiling(copies, torch, args.steps)

    per_launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    mean_launch_ms = sum(per_launch_ms) / len(per_launch_ms)
    ms_per_step = region_ms / args.steps
    last_offset = args.warmup + 2 * args.steps - 1       # the offset of the last call made
    gpu_out = {"tokens": out_tok.cpu().numpy(), "accept_len": out_len.cpu().numpy(), "lazy": lazy}
    if mode == "sample" and not ragged and not tok_only:
        gpu_out["p"] = out_p.cpu().numpy().reshape(B, K)
        gpu_out["q"] = out_q.cpu().numpy().reshape(B, K)
    accept = out_len.cpu().numpy()
    rejected = int((accept < K + 1).sum()) if mode == "sample" else None
    # the last step's accept lengths stand for every step's (the offset changes
    # the uniforms, not the drafts' odds)
    nbytes = lazy_bytes(wl, accept) if lazy else algorithmic_bytes(wl, rejected)
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    # The dominant kernel: a one-launch call is one kernel per step, so its
    # average duration is the timed region over the steps (events on the
    # launch stream); calls of several launches are priced as a whole.
    n_launches = launches_per_call(wl, args.workload, lazy, filt, draft is not None)
    achieved = nbytes / (ms_per_step * 1e-3) / 1e9

    line = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_hbm_peak": round(100 * gbps / PEAK_HBM_GBPS, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"calls": settle_calls, "s": round(settle_s, 3)},
        "ms_per_step": round(ms_per_step, 5),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl["name"], "mode": mode, "B": B, "K": K, "V": V,
                   "logits_dtype": wl["dtype"], "draft": "explicit" if draft is not None else
                   ("one-hot" if mode == "sample" else "tokens"),
                   "temperature": None if wl["temperature"] is None else float(wl["temperature"][0]),
                   "algorithmic_bytes_per_step": nbytes, "input_copies": len(copies),
                   **({"ragged": {"rows_consulted": int(wl["ragged"]["ks"].sum()) + B,
                                  "k_mean": round(float(wl["ragged"]["ks"].mean()), 3),
                                  "K_max": K}} if ragged else {}),
                   **({"lazy": {"rows_read_bytes": nbytes,
                                "dense_bytes": algorithmic_bytes(wl, rejected),
                                "dense_equivalent_gbps": round(algorithmic_bytes(wl, rejected)
                                                               / (ms_per_step * 1e-3) / 1e9, 1)}}
                      if lazy else {}),
                   **({"filter": {"top_k": f_k, "top_p": f_p}} if filt else {}),
                   **({"outputs": "tokens and accept lengths (no p / q)"} if tok_only else {}),
                   **({"bitmask": {"allowed_fraction": round(float(wl["mask_allowed"]), 4),
                                   "bytes": int(wl["bitmask"].nbytes)}} if masked else {})},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic_record(wl["name"]),
                     "kernel": roofline_kernel(wl, lazy, filt, draft is not None, n_launches),
                     "kernel_us": round(ms_per_step * 1e3, 2),
                     "timing": "HIP events on the launch stream around the timed region, / steps",
                     "call_us_median": round(per_launch_ms[len(per_launch_ms) // 2] * 1e3, 2),
                     "call_us_p10": round(per_launch_ms[len(per_launch_ms) // 10] * 1e3, 2),
                     "call_us_p90": round(per_launch_ms[(9 * len(per_launch_ms)) // 10] * 1e3, 2),
                     "call_us_mean": round(mean_launch_ms * 1e3, 2),
                     "call_timing": "a second pass with an event pair around every call"},
        # the probe reads the target logits; with draft logits the call reads
        # more than that, and early exit reads less, so no ratio is given
        "stream_ceiling": dict(stream, call_logical_gbps=round(
            copies[0].numel() * copies[0].element_size() / (ms_per_step * 1e-3) / 1e9, 1),
            call_frac=round(copies[0].numel() * copies[0].element_size() / (ms_per_step * 1e-3) / 1e9
                            / stream["gbps"], 4) if stream["gbps"] and draft is None and not lazy
            else None),
        "accept_len_hist": np.bincount(accept, minlength=(K + 2) if mode != "tree" else 5).tolist(),
        "source_digest": source_digest(),
    }
    if pool is not None:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, pool, last_offset, gpu_out)
        pool.close()
        pool.join()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
