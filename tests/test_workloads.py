"""The seeded generator: determinism and the workloads' stated distributions."""
import numpy as np

from moe_routed_expert_amd.workloads import WORKLOADS, custom
from tests.numerics import bf16_bits_to_f32


def test_same_seed_same_inputs_and_prefix_property():
    w = WORKLOADS["swiglu_100003x1536"]
    a = w.generate(rows=5000)
    b = w.generate(rows=5000)
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = w.generate(rows=4096)
    for k in a:
        assert np.array_equal(a[k][:4096], c[k])


def test_shapes_and_dtypes():
    for w in WORKLOADS.values():
        d = w.generate(rows=min(w.rows, 300))
        n = d["probs"].shape[0]
        assert d["x"].dtype == np.uint16 and d["x"].shape == (n, w.x_cols)
        assert d["grad_out"].dtype == np.uint16 and d["grad_out"].shape == (n, w.cols)
        assert d["probs"].dtype == np.float32


def test_special_values_and_probability_zeros():
    w = WORKLOADS["swiglu_100003x1536"]
    d = w.generate(rows=8192)
    x = bf16_bits_to_f32(d["x"])
    special = np.isin(x, [-7.0, 7.0, 0.0])
    assert 0.095 < special.mean() < 0.105
    assert 0.18 < (d["probs"] == 0).mean() < 0.22
    s = np.std(x[~special])
    assert 4.7 < s < 5.3
    w1 = WORKLOADS["swiglu_256x128"]
    x1 = bf16_bits_to_f32(w1.generate()["x"])
    assert 0.04 < np.isin(x1, [-7.0, 7.0]).mean() < 0.07


def test_top8_renormalisation():
    w = WORKLOADS["swiglu_8192x2048"]
    p = w.generate(rows=512)["probs"].astype(np.float64)
    sums = p.reshape(-1, 8).sum(axis=1)
    assert np.all(np.abs(sums - 1.0) < 1e-6)


def test_byte_model():
    w = WORKLOADS["swiglu_131072x2048"]
    assert w.fwd_bytes() == 1_611_137_024
    assert w.bwd_bytes() == 2_685_403_136
    r = WORKLOADS["router_65536x7168"]
    assert r.fwd_bytes() == 1_879_310_336
    assert r.bwd_bytes() == 2_819_096_576
    assert custom("router", 10, 8).bwd_bytes(with_grad_probs=False) == 10 * (4 * 8 + 4)
