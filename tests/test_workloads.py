"""The synthetic generators produce what their recipes say (shapes, seeds, planted structure)."""
import numpy as np
import pytest

from workloads import CONFIGS, bf16_bits_to_f32, make


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_shapes_and_determinism(name):
    kw = dict(B=3, V=700)
    a = make(name, data_seed=9, **kw)
    b = make(name, data_seed=9, **kw)
    for k in ("target", "draft_tokens", "seeds"):
        np.testing.assert_array_equal(a[k], b[k])
    R = a["K"] + 1 if a["mode"] != "tree" else len(a["parents"])
    assert a["target"].shape == (3, R, 700)
    assert a["target"].dtype == (np.uint16 if a["dtype"] == "bf16" else np.float32)
    assert a["seeds"].dtype == np.uint64


def test_match_rates_and_peak():
    c3 = make("c3_onehot", data_seed=1, B=400, V=2000)
    am = bf16_bits_to_f32(c3["target"][:, :5]).argmax(-1)
    rate = (c3["draft_tokens"] == am).mean()
    assert abs(rate - 0.6) < 0.03
    c4 = make("c4_greedy", data_seed=1, B=400, V=2000)
    rate = (c4["draft_tokens"] == c4["target"][:, :3].argmax(-1)).mean()
    assert abs(rate - 0.85) < 0.03
    c2 = make("c2_stoch", data_seed=1, B=50, V=4000)
    t = c2["target"].astype(np.float64)
    assert abs((c2["draft"] - t[:, :3]).std() - 0.7) < 0.01
    assert abs(np.median(t.std(axis=-1)) - 2.0) < 0.05
    # exactly one planted +6 per row lifts the row mean by 6/V
    assert abs(t.mean() - 6.0 / 4000) < 0.003
