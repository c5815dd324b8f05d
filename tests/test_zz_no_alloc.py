"""The no-allocation entry point (spec_verify_sample_noalloc, for callers
that cannot allocate) against spec_verify_sample, through the C ABI: two
calls in a row, the second smaller, each equal to the workspace call."""
import ctypes

import numpy as np
import pytest
import torch

import draft_verification_05_amd as sv
from parity import to_device
from workloads import make

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def call(lib, wl, noalloc):
    d = to_device(wl, DEV)
    B, K, V = wl["B"], wl["K"], wl["V"]
    t = sv._desc(d["target"], "target")
    dd = sv._desc(d["draft"], "draft") if d["draft"] is not None else None
    tok = torch.full((B, K + 1), -7, dtype=torch.int32, device=DEV)
    alen = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    p = torch.full((B, K), -7.0, dtype=torch.float32, device=DEV)
    q = torch.full((B, K), -7.0, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    head = (ctypes.byref(t), ctypes.byref(dd) if dd is not None else None, d["tokens"].data_ptr(),
            d["temperature"].data_ptr(), d["seeds"].data_ptr(), wl["offset"], B, K, V,
            tok.data_ptr(), alen.data_ptr(), p.data_ptr(), q.data_ptr())
    if noalloc:
        rc = lib.spec_verify_sample_noalloc(*head, stream)
    else:
        nbytes = sv.spec_verify_workspace_size(sv.SV_OP_SAMPLE, B, K, V, dd is not None)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        sv.spec_verify_workspace_init(ws)
        rc = lib.spec_verify_sample(*head, ws.data_ptr(), nbytes, stream)
    assert rc == 0, sv.spec_verify_status_string(rc)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (tok, alen, p, q)]


def test_noalloc_equals_workspace_call_twice_second_smaller():
    lib = sv.load_library()
    cases = [make("c3_onehot", data_seed=900, B=64, V=3 * 8192 + 1232, offset=5),
             make("c2_stoch", data_seed=901, B=12, V=9001, offset=6)]
    for i, wl in enumerate(cases):
        print(f"[case] no-alloc call {i}: B={wl['B']} K={wl['K']} V={wl['V']} {wl['dtype']}", flush=True)
        a = call(lib, wl, True)
        b = call(lib, wl, False)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        assert np.all((a[1] >= 1) & (a[1] <= wl["K"] + 1))


def test_noalloc_rejects_calls_beyond_its_scratch():
    lib = sv.load_library()
    t = sv.SVLogits(0x10000, 1, 0, 6 * 128256, 128256)
    fake = ctypes.c_void_p(0x10000)
    rc = lib.spec_verify_sample_noalloc(ctypes.byref(t), None, fake, fake, fake, 0, 1024, 5, 128256,
                                        fake, fake, None, None, None)
    assert rc == sv.SV_ERR_SCRATCH
