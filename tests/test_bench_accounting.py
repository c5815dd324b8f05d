"""The benchmark's byte accounting: the algorithmic bytes a call must read,
written out by hand for small shapes (host logic only, no GPU)."""
import numpy as np

import bench
from workloads import make


def test_dense_bytes():
    # one-hot bf16: every target row once, plus the draw's one 4 KiB chunk per request
    wl = make("c3_onehot", data_seed=0, B=4, V=5000)
    assert bench.algorithmic_bytes(wl) == 4 * 6 * 5000 * 2 + 4 * 4096
    # explicit fp32 drafts: target and draft rows, the draw chunk, and the stop
    # rows of target and draft again for each rejected request
    wl = make("c2_stoch", data_seed=0, B=3, V=3000)
    rows = 3 * (4 + 3) * 3000 * 4
    assert bench.algorithmic_bytes(wl, rejected=2) == rows + 3 * 4096 + 2 * 2 * 3000 * 4
    # greedy and tree draw nothing
    wl = make("c4_greedy", data_seed=0, B=2, V=1000)
    assert bench.algorithmic_bytes(wl) == 2 * 4 * 1000 * 4
    wl = make("c5_tree", data_seed=0, B=2, V=1000)
    assert bench.algorithmic_bytes(wl) == 2 * 31 * 1000 * 4
    # a row shorter than one chunk: the draw reads the row, not 4 KiB
    wl = make("c1_tiny", data_seed=0)
    assert bench.algorithmic_bytes(wl, rejected=1) == (2 + 1) * 1000 * 4 + 1000 * 4 + 2 * 1000 * 4


def test_early_exit_bytes_follow_the_two_windows():
    # windows [0] and [1, K]: a request that stops at position 0 (accept
    # length 1) read its first row only; any other read all K + 1
    wl = make("c3_onehot", data_seed=0, B=3, V=5000)
    accept = np.array([1, 2, 6], np.int32)
    row = 5000 * 2
    assert bench.lazy_bytes(wl, accept) == (1 + 6 + 6) * row + 3 * 4096
    # explicit drafts: draft rows up to min(e, K - 1), and the residual's two
    # stop rows for requests that rejected (accept length <= K)
    wl = make("c2_stoch", data_seed=0, B=2, V=3000)
    row = 3000 * 4
    accept = np.array([1, 4], np.int32)         # stop at 0 (rejected), all 3 accepted (bonus)
    expect = (1 + 1) * row + (4 + 3) * row + 2 * 4096 + 1 * 2 * row
    assert bench.lazy_bytes(wl, accept) == expect
