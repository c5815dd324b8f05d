"""Batched speculative-decoding verification on MI355X (gfx950).

A thin binding over ``libspecverify.so`` (C ABI in ``include/specverify.h``):
argument marshalling only. Every step of verification runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream. There is
no fallback: without the built library every call raises.

Entry points (same names as the C ABI):
  spec_verify_sample(target, draft, draft_tokens, temperature, seeds, offset)
  spec_verify_greedy(target, draft_tokens)
  spec_verify_tree(target, node_tokens, parents)           (parents: host [N], or device [B, N]
                                                          for a tree per request)
  spec_verify_sample_ragged / spec_verify_greedy_ragged   (per-request draft counts)
  spec_verify_sample_masked / spec_verify_greedy_masked   (grammar bitmasks)
  spec_verify_sample_lazy                                 (early exit at the first rejection)
  spec_verify_sample_filtered                             (top-k / top-p filtered p and q)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "LIB_PATH", "SpecVerifyError", "load_library", "spec_verify_sample", "spec_verify_greedy",
    "spec_verify_tree", "spec_verify_sample_ragged", "spec_verify_greedy_ragged",
    "spec_verify_sample_masked", "spec_verify_greedy_masked", "spec_verify_sample_lazy",
    "spec_verify_sample_filtered",
    "spec_verify_workspace_size", "spec_verify_workspace_init", "spec_verify_workspace_errors",
    "spec_verify_errors",
    "spec_verify_status_string", "SV_OK", "SV_ERR_NULL", "SV_ERR_SHAPE", "SV_ERR_DTYPE",
    "SV_ERR_STRIDE", "SV_ERR_WORKSPACE", "SV_ERR_TREE", "SV_ERR_HIP", "SV_ERR_NO_DEVICE",
    "SV_ERR_SCRATCH", "spec_verify_sample_noalloc", "SV_OP_SAMPLE",
    "SV_OP_GREEDY", "SV_OP_TREE", "SVLogits",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE = 0, -1, -2, -3
SV_ERR_STRIDE, SV_ERR_WORKSPACE, SV_ERR_TREE, SV_ERR_HIP, SV_ERR_NO_DEVICE = -4, -5, -6, -7, -8
SV_ERR_SCRATCH = -9
SV_DTYPE_F32, SV_DTYPE_BF16 = 0, 1
SV_OP_SAMPLE, SV_OP_GREEDY, SV_OP_TREE = 0, 1, 2

_c_i32, _c_i64, _c_u64, _c_size, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_size_t, ctypes.c_void_p)


class SVLogits(ctypes.Structure):
    _fields_ = [("data", _vp), ("dtype", _c_i32), ("reserved", _c_i32),
                ("stride_b", _c_i64), ("stride_k", _c_i64)]


_PSV = ctypes.POINTER(SVLogits)

_SIGNATURES = {
    "spec_verify_workspace_size": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "spec_verify_workspace_init": (ctypes.c_int, [_vp, _c_size, _vp]),
    "spec_verify_workspace_errors": (ctypes.c_int, [_vp, _c_size, _vp, _c_i32, _vp]),
    "spec_verify_sample": (ctypes.c_int, [_PSV, _PSV, _vp, _vp, _vp, _c_u64, _c_i32, _c_i32,
                                          _c_i32, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "spec_verify_sample_lazy": (ctypes.c_int, [_PSV, _PSV, _vp, _vp, _vp, _c_u64, _c_i32, _c_i32,
                                               _c_i32, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "spec_verify_sample_noalloc": (ctypes.c_int, [_PSV, _PSV, _vp, _vp, _vp, _c_u64, _c_i32, _c_i32,
                                                  _c_i32, _vp, _vp, _vp, _vp, _vp]),
    "spec_verify_sample_filtered": (ctypes.c_int, [_PSV, _PSV, _vp, _vp, _vp, _vp, _vp, _c_u64,
                                                   _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp,
                                                   _c_size, _vp]),
    "spec_verify_greedy": (ctypes.c_int, [_PSV, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp,
                                          _vp, _c_size, _vp]),
    "spec_verify_tree": (ctypes.c_int, [_PSV, _vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp,
                                        _vp, _c_size, _vp]),
    "spec_verify_tree_dynamic": (ctypes.c_int, [_PSV, _vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp,
                                                _vp, _c_size, _vp]),
    "spec_verify_sample_ragged": (ctypes.c_int, [_PSV, _PSV, _vp, _c_i32, _vp, _vp, _vp, _c_u64,
                                                 _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp,
                                                 _c_size, _vp]),
    "spec_verify_greedy_ragged": (ctypes.c_int, [_PSV, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32,
                                                 _vp, _vp, _vp, _vp, _c_size, _vp]),
    "spec_verify_sample_masked": (ctypes.c_int, [_PSV, _PSV, _vp, _vp, _vp, _vp, _c_u64, _c_i32,
                                                 _c_i32, _c_i32, _vp, _vp, _vp, _vp, _vp, _c_size,
                                                 _vp]),
    "spec_verify_greedy_masked": (ctypes.c_int, [_PSV, _vp, _vp, _c_i32, _c_i32, _c_i32, _vp, _vp,
                                                 _vp, _vp, _c_size, _vp]),
    "spec_verify_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None
_lock = threading.Lock()


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = spec_verify_status_string(status) if _lib is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle; raises if the library was not built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def spec_verify_status_string(status: int) -> str:
    return load_library().spec_verify_status_string(int(status)).decode()


def spec_verify_workspace_size(op: int, B: int, K_or_N: int, V: int, has_draft: bool = False) -> int:
    return int(load_library().spec_verify_workspace_size(op, B, K_or_N, V, int(bool(has_draft))))


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def spec_verify_workspace_init(ws: torch.Tensor) -> None:
    rc = load_library().spec_verify_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(),
                                                   _stream_ptr(ws.device))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_workspace_init")


def spec_verify_workspace_errors(ws: torch.Tensor, reset: bool = True) -> int:
    """Number of requests whose one-launch rule gave up waiting (and refused
    the request) since `ws` was zero-filled or last reset. Synchronises with
    the workspace's device. A working device always returns 0."""
    out = torch.zeros(1, dtype=torch.int32, device=ws.device)
    rc = load_library().spec_verify_workspace_errors(ws.data_ptr(), ws.numel() * ws.element_size(),
                                                     out.data_ptr(), int(bool(reset)),
                                                     _stream_ptr(ws.device))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_workspace_errors")
    return int(out.item())


def spec_verify_errors(device=None, reset: bool = True) -> int:
    """spec_verify_workspace_errors of the workspace this module keeps for
    the current stream of `device` (0 when it has none yet)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    ws = _workspaces.get((dev.index, _stream_ptr(dev)))
    return 0 if ws is None else spec_verify_workspace_errors(ws, reset)


# One zero-initialised workspace per (device, stream): the library leaves its
# counter and tagged words zero after every call, so reuse on the same stream
# is safe.
_workspaces: dict = {}


def _workspace(device, nbytes: int) -> torch.Tensor:
    key = (device.index, _stream_ptr(device))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        spec_verify_workspace_init(ws)
        _workspaces[key] = ws
    return ws


def _desc(t: torch.Tensor, name: str) -> SVLogits:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 3:
        raise ValueError(f"{name} must be [B, rows, V]")
    if t.dtype == torch.float32:
        dt = SV_DTYPE_F32
    elif t.dtype == torch.bfloat16:
        dt = SV_DTYPE_BF16
    else:
        raise ValueError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError(f"{name} must have a contiguous vocabulary dimension")
    return SVLogits(t.data_ptr(), dt, 0, t.stride(0), t.stride(1))


def _rows_desc(t: torch.Tensor, name: str) -> SVLogits:
    """Descriptor of packed rows [rows, V] (ragged calls: rows stride(0) apart)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be [rows, V]")
    if t.dtype == torch.float32:
        dt = SV_DTYPE_F32
    elif t.dtype == torch.bfloat16:
        dt = SV_DTYPE_BF16
    else:
        raise ValueError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a contiguous vocabulary dimension")
    return SVLogits(t.data_ptr(), dt, 0, 0, t.stride(0))


def _check(t: torch.Tensor, name: str, dtype, shape, device):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}, got {t.dtype} {tuple(t.shape)} on {t.device}")


def _seeds_u64(seeds: torch.Tensor) -> torch.Tensor:
    # uint64 seeds travel as their int64 bit pattern
    if seeds.dtype == torch.int64:
        return seeds
    if seeds.dtype == torch.uint64:
        return seeds.view(torch.int64)
    raise ValueError("seeds must be int64 or uint64")


def _ptr(t):
    return None if t is None else t.data_ptr()


def spec_verify_sample(target: torch.Tensor, draft: torch.Tensor | None, draft_tokens: torch.Tensor,
                       temperature: torch.Tensor, seeds: torch.Tensor, offset: int = 0,
                       *, want_probs: bool = True):
    """Stochastic verification. Returns (tokens [B,K+1], accept_len [B], p_draft [B,K], q_draft [B,K])."""
    return _sample("spec_verify_sample", target, draft, draft_tokens, temperature, seeds, offset,
                   want_probs)


def spec_verify_sample_noalloc(target: torch.Tensor, draft: torch.Tensor | None,
                               draft_tokens: torch.Tensor, temperature: torch.Tensor,
                               seeds: torch.Tensor, offset: int = 0, *, want_probs: bool = True):
    """spec_verify_sample through the entry point that allocates nothing: its
    workspace is the library's static per-device scratch (16 MiB; larger calls
    raise SV_ERR_SCRATCH). Calls that may overlap on one device race on that
    scratch. The outputs here are allocated by torch; the C entry point itself
    allocates nothing."""
    lib = load_library()
    B, R, V = target.shape
    K = R - 1
    dev = target.device
    tdesc = _desc(target, "target")
    ddesc = None
    if draft is not None:
        ddesc = _desc(draft, "draft")
        if draft.shape[0] != B or draft.shape[1] < K or draft.shape[2] != V or draft.device != dev:
            raise ValueError("draft must be [B, >=K, V] on the target's device")
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    seeds = _seeds_u64(seeds)
    _check(seeds, "seeds", torch.int64, (B,), dev)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    p = torch.empty((B, K), dtype=torch.float32, device=dev) if want_probs else None
    q = torch.empty((B, K), dtype=torch.float32, device=dev) if want_probs else None
    with torch.cuda.device(dev):
        rc = lib.spec_verify_sample_noalloc(ctypes.byref(tdesc), ctypes.byref(ddesc) if ddesc else None,
                                            draft_tokens.data_ptr() if K else None,
                                            temperature.data_ptr(), seeds.data_ptr(),
                                            int(offset) & (2**64 - 1), B, K, V, tokens.data_ptr(),
                                            alen.data_ptr(), _ptr(p), _ptr(q), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_sample_noalloc")
    return tokens, alen, p, q


def spec_verify_sample_lazy(target: torch.Tensor, draft: torch.Tensor | None,
                            draft_tokens: torch.Tensor, temperature: torch.Tensor,
                            seeds: torch.Tensor, offset: int = 0, *, want_probs: bool = True):
    """Early-exit stochastic verification: rows after a request's first rejection are not read.

    Same results as spec_verify_sample (tokens, accept_len); p_draft / q_draft are 0 after
    the position where the request stopped."""
    return _sample("spec_verify_sample_lazy", target, draft, draft_tokens, temperature, seeds,
                   offset, want_probs)


def spec_verify_sample_filtered(target: torch.Tensor, draft: torch.Tensor | None,
                                draft_tokens: torch.Tensor, temperature: torch.Tensor,
                                top_k: torch.Tensor | None, top_p: torch.Tensor | None,
                                seeds: torch.Tensor, offset: int = 0, *, want_probs: bool = True):
    """Stochastic verification on top-k / top-p filtered p (and q): top_k int32 [B] and
    top_p float32 [B] device tensors, either may be None. Returns as spec_verify_sample."""
    B = target.shape[0]
    if top_k is not None:
        _check(top_k, "top_k", torch.int32, (B,), target.device)
    if top_p is not None:
        _check(top_p, "top_p", torch.float32, (B,), target.device)
    return _sample("spec_verify_sample_filtered", target, draft, draft_tokens, temperature, seeds,
                   offset, want_probs, filters=(_ptr(top_k), _ptr(top_p)))


def _sample(entry, target, draft, draft_tokens, temperature, seeds, offset, want_probs,
            filters=None):
    lib = load_library()
    B, R, V = target.shape
    K = R - 1
    dev = target.device
    tdesc = _desc(target, "target")
    ddesc = None
    if draft is not None:
        ddesc = _desc(draft, "draft")
        if draft.shape[0] != B or draft.shape[1] < K or draft.shape[2] != V or draft.device != dev:
            raise ValueError("draft must be [B, >=K, V] on the target's device")
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    seeds = _seeds_u64(seeds)
    _check(seeds, "seeds", torch.int64, (B,), dev)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    p = torch.empty((B, K), dtype=torch.float32, device=dev) if want_probs else None
    q = torch.empty((B, K), dtype=torch.float32, device=dev) if want_probs else None
    nbytes = spec_verify_workspace_size(SV_OP_SAMPLE, B, K, V, draft is not None)
    ws = _workspace(dev, nbytes)
    head = [ctypes.byref(tdesc), ctypes.byref(ddesc) if ddesc else None,
            draft_tokens.data_ptr() if K else None, temperature.data_ptr()]
    if filters is not None:
        head += list(filters)
    rc = getattr(lib, entry)(*head, seeds.data_ptr(), int(offset) & (2**64 - 1), B, K, V,
                             tokens.data_ptr(), alen.data_ptr(), _ptr(p), _ptr(q),
                             ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, entry)
    return tokens, alen, p, q


def spec_verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor, *, want_argmax: bool = True):
    """Greedy verification. Returns (tokens [B,K+1], accept_len [B], argmax [B,K+1])."""
    lib = load_library()
    B, R, V = target.shape
    K = R - 1
    dev = target.device
    tdesc = _desc(target, "target")
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    g = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if want_argmax else None
    ws = _workspace(dev, spec_verify_workspace_size(SV_OP_GREEDY, B, K, V))
    rc = lib.spec_verify_greedy(ctypes.byref(tdesc), draft_tokens.data_ptr() if K else None,
                                B, K, V, tokens.data_ptr(), alen.data_ptr(), _ptr(g),
                                ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_greedy")
    return tokens, alen, g


def spec_verify_sample_ragged(target_rows: torch.Tensor, draft_rows: torch.Tensor | None,
                              cu_draft: torch.Tensor, draft_tokens: torch.Tensor,
                              temperature: torch.Tensor, seeds: torch.Tensor, offset: int = 0,
                              *, k_max: int, want_probs: bool = True):
    """Ragged batch: request b has K_b = cu_draft[b+1] - cu_draft[b] drafts.

    target_rows [total_k + B, V] (request b's rows from cu_draft[b] + b),
    draft_rows [total_k, V] or None, cu_draft int32 [B + 1], draft_tokens
    int32 [total_k]. Returns (tokens [B, k_max+1], accept_len [B],
    p_draft [total_k], q_draft [total_k]).
    """
    lib = load_library()
    dev = target_rows.device
    B = cu_draft.numel() - 1
    total_k = draft_tokens.numel()
    V = target_rows.shape[-1]
    tdesc = _rows_desc(target_rows, "target_rows")
    if target_rows.shape[0] != total_k + B:
        raise ValueError("target_rows must hold total_k + B rows")
    ddesc = None
    if draft_rows is not None:
        ddesc = _rows_desc(draft_rows, "draft_rows")
        if draft_rows.shape != (total_k, V) or draft_rows.device != dev:
            raise ValueError("draft_rows must be [total_k, V] on the target's device")
    _check(cu_draft, "cu_draft", torch.int32, (B + 1,), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (total_k,), dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    seeds = _seeds_u64(seeds)
    _check(seeds, "seeds", torch.int64, (B,), dev)
    tokens = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    p = torch.empty((total_k,), dtype=torch.float32, device=dev) if want_probs else None
    q = torch.empty((total_k,), dtype=torch.float32, device=dev) if want_probs else None
    ws = _workspace(dev, spec_verify_workspace_size(SV_OP_SAMPLE, B, k_max, V, draft_rows is not None))
    rc = lib.spec_verify_sample_ragged(ctypes.byref(tdesc), ctypes.byref(ddesc) if ddesc else None,
                                       cu_draft.data_ptr(), total_k,
                                       draft_tokens.data_ptr() if total_k else None,
                                       temperature.data_ptr(), seeds.data_ptr(),
                                       int(offset) & (2**64 - 1), B, int(k_max), V,
                                       tokens.data_ptr(), alen.data_ptr(), _ptr(p), _ptr(q),
                                       ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_sample_ragged")
    return tokens, alen, p, q


def spec_verify_greedy_ragged(target_rows: torch.Tensor, cu_draft: torch.Tensor,
                              draft_tokens: torch.Tensor, *, k_max: int, want_argmax: bool = True):
    """Ragged greedy verification. Returns (tokens [B, k_max+1], accept_len [B], argmax [total_k + B])."""
    lib = load_library()
    dev = target_rows.device
    B = cu_draft.numel() - 1
    total_k = draft_tokens.numel()
    V = target_rows.shape[-1]
    tdesc = _rows_desc(target_rows, "target_rows")
    if target_rows.shape[0] != total_k + B:
        raise ValueError("target_rows must hold total_k + B rows")
    _check(cu_draft, "cu_draft", torch.int32, (B + 1,), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (total_k,), dev)
    tokens = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    g = torch.full((total_k + B,), -1, dtype=torch.int32, device=dev) if want_argmax else None
    ws = _workspace(dev, spec_verify_workspace_size(SV_OP_GREEDY, B, k_max, V))
    rc = lib.spec_verify_greedy_ragged(ctypes.byref(tdesc), cu_draft.data_ptr(), total_k,
                                       draft_tokens.data_ptr() if total_k else None, B,
                                       int(k_max), V, tokens.data_ptr(), alen.data_ptr(), _ptr(g),
                                       ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_greedy_ragged")
    return tokens, alen, g


def _bitmask(bitmask: torch.Tensor, B: int, R: int, V: int, dev) -> torch.Tensor:
    if bitmask.dtype == torch.uint32:
        bitmask = bitmask.view(torch.int32)
    _check(bitmask, "bitmask", torch.int32, (B, R, (V + 31) // 32), dev)
    return bitmask


def spec_verify_sample_masked(target: torch.Tensor, draft: torch.Tensor | None,
                              draft_tokens: torch.Tensor, bitmask: torch.Tensor,
                              temperature: torch.Tensor, seeds: torch.Tensor, offset: int = 0,
                              *, want_probs: bool = True):
    """Grammar-masked stochastic verification; bitmask [B, K+1, ceil(V/32)] int32/uint32
    (bit v % 32 of word v // 32 set = token v allowed). Returns as spec_verify_sample."""
    lib = load_library()
    B, R, V = target.shape
    K = R - 1
    dev = target.device
    tdesc = _desc(target, "target")
    ddesc = None
    if draft is not None:
        ddesc = _desc(draft, "draft")
        if draft.shape[0] != B or draft.shape[1] < K or draft.shape[2] != V or draft.device != dev:
            raise ValueError("draft must be [B, >=K, V] on the target's device")
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    bitmask = _bitmask(bitmask, B, R, V, dev)
    _check(temperature, "temperature", torch.float32, (B,), dev)
    seeds = _seeds_u64(seeds)
    _check(seeds, "seeds", torch.int64, (B,), dev)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    p = torch.empty((B, K), dtype=torch.float32, device=dev) if want_probs else None
    q = torch.empty((B, K), dtype=torch.float32, device=dev) if want_probs else None
    ws = _workspace(dev, spec_verify_workspace_size(SV_OP_SAMPLE, B, K, V, draft is not None))
    rc = lib.spec_verify_sample_masked(ctypes.byref(tdesc), ctypes.byref(ddesc) if ddesc else None,
                                       draft_tokens.data_ptr() if K else None, bitmask.data_ptr(),
                                       temperature.data_ptr(), seeds.data_ptr(),
                                       int(offset) & (2**64 - 1), B, K, V, tokens.data_ptr(),
                                       alen.data_ptr(), _ptr(p), _ptr(q), ws.data_ptr(), ws.numel(),
                                       _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_sample_masked")
    return tokens, alen, p, q


def spec_verify_greedy_masked(target: torch.Tensor, draft_tokens: torch.Tensor, bitmask: torch.Tensor,
                              *, want_argmax: bool = True):
    """Grammar-masked greedy verification. Returns as spec_verify_greedy."""
    lib = load_library()
    B, R, V = target.shape
    K = R - 1
    dev = target.device
    tdesc = _desc(target, "target")
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    bitmask = _bitmask(bitmask, B, R, V, dev)
    tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    g = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if want_argmax else None
    ws = _workspace(dev, spec_verify_workspace_size(SV_OP_GREEDY, B, K, V))
    rc = lib.spec_verify_greedy_masked(ctypes.byref(tdesc), draft_tokens.data_ptr() if K else None,
                                       bitmask.data_ptr(), B, K, V, tokens.data_ptr(), alen.data_ptr(),
                                       _ptr(g), ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, "spec_verify_greedy_masked")
    return tokens, alen, g


def spec_verify_tree(target: torch.Tensor, node_tokens: torch.Tensor, parents):
    """Tree verification. ``parents`` is a host sequence of N entries (one tree for the
    batch), or an int32 tensor [B, N] on the target's device (a tree per request:
    spec_verify_tree_dynamic). Returns (tokens [B,N], accept_len [B], best [B])."""
    lib = load_library()
    B, N, V = target.shape
    dev = target.device
    tdesc = _desc(target, "target")
    _check(node_tokens, "node_tokens", torch.int32, (B, N), dev)
    dynamic = isinstance(parents, torch.Tensor) and parents.dim() == 2
    if dynamic:
        _check(parents, "parents", torch.int32, (B, N), dev)
        par_ptr, fn, name = ctypes.c_void_p(parents.data_ptr()), lib.spec_verify_tree_dynamic, \
            "spec_verify_tree_dynamic"
    else:
        if len(parents) != N:
            raise ValueError("parents must have one entry per node")
        par = (ctypes.c_int32 * N)(*[int(v) for v in parents])
        par_ptr, fn, name = ctypes.cast(par, ctypes.c_void_p), lib.spec_verify_tree, "spec_verify_tree"
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    best = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = _workspace(dev, spec_verify_workspace_size(SV_OP_TREE, B, N, V))
    rc = fn(ctypes.byref(tdesc), node_tokens.data_ptr(), par_ptr, N, B, V, tokens.data_ptr(),
            alen.data_ptr(), best.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(dev))
    if rc:
        raise SpecVerifyError(rc, name)
    return tokens, alen, best
