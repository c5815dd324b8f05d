"""The library's device Philox4x64-10 against the oracle's, word for word.

A test-only kernel built beside the library (probe/philox_probe.hip) runs the
device generator of sv_device.hpp on 10^6 counter/key pairs: the verifier's
own layout (position, request, offset, 0) with keys (seed, 0), and full
64-bit random words in every counter and key position. Every output word
must equal oracle.philox's (Salmon et al., SC'11, the generator both sides
implement from its published definition).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle.philox import philox4x64_10

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N = 1_000_000


def test_device_philox_matches_oracle_on_1e6_counters():
    lib = ctypes.CDLL(os.path.join(ROOT, "draft_verification_05_amd", "libsvphilox.so"))
    lib.sv_philox_words.restype = ctypes.c_int
    lib.sv_philox_words.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_void_p]
    rng = np.random.default_rng(20261203)
    half = N // 2
    ctr = np.zeros((N, 4), np.uint64)
    key = np.zeros((N, 2), np.uint64)
    # the verifier's counters: position, request, offset; key = the request's seed
    ctr[:half, 0] = rng.integers(0, 33, half)
    ctr[:half, 1] = rng.integers(0, 1 << 16, half)
    ctr[:half, 2] = rng.integers(0, 1 << 40, half)
    key[:half, 0] = rng.integers(0, 2**64, half, dtype=np.uint64)
    # arbitrary 64-bit words everywhere
    ctr[half:] = rng.integers(0, 2**64, (N - half, 4), dtype=np.uint64)
    key[half:] = rng.integers(0, 2**64, (N - half, 2), dtype=np.uint64)
    dev = torch.device("cuda:0")
    d_ctr = torch.from_numpy(ctr.view(np.int64)).to(dev)
    d_key = torch.from_numpy(key.view(np.int64)).to(dev)
    d_out = torch.zeros((N, 4), dtype=torch.int64, device=dev)
    print(f"[case] device Philox on {N} counters", flush=True)
    rc = lib.sv_philox_words(d_ctr.data_ptr(), d_key.data_ptr(), d_out.data_ptr(), N,
                             torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = d_out.cpu().numpy().view(np.uint64)
    bad = 0
    for i in range(N):
        if i % 200_000 == 0:
            print(f"[philox] compared {i} of {N}", flush=True)
        want = philox4x64_10(tuple(int(v) for v in ctr[i]), (int(key[i, 0]), int(key[i, 1])))
        bad += tuple(int(v) for v in got[i]) != want
    assert bad == 0, f"{bad} of {N} counters differ"
