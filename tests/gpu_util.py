"""Helpers for the GPU parity tests: host <-> device copies of bf16 bit
patterns and the parity bar.

The bar (clamped SwiGLU and router multiply):
  - bf16 outputs: within 1 bf16 ulp of the oracle's fp32-then-round value;
    every position where the oracle has a zero (+0 or -0, masked or not) is
    bit-identical; NaN exactly where the oracle has NaN;
  - router forward and router grad_x: bit-exact (one fp32 multiply, one
    rounding);
  - probability gradients: |gpu - oracle| <= 2e-5 * sum_j |term_j| per row
    (the sum of absolute terms is the scale any summation order's error is
    proportional to; a plain relative error cannot hold on rows whose sum
    cancels, for any order).
"""
import numpy as np
import torch

from tests.numerics import bf16_is_nan, bf16_ulp_diff

DPROBS_REL = 2e-5


def to_dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_parity(got: np.ndarray, want: np.ndarray, what: str, exact: bool = False) -> dict:
    assert got.shape == want.shape, (what, got.shape, want.shape)
    nan_w, nan_g = bf16_is_nan(want), bf16_is_nan(got)
    assert np.array_equal(nan_w, nan_g), f"{what}: NaN positions differ ({int((nan_w != nan_g).sum())})"
    ok = ~nan_w
    g, w = got[ok], want[ok]
    if exact:
        bad = g != w
        assert not bad.any(), f"{what}: {int(bad.sum())} of {g.size} differ (bit-exact bar); first at {np.argmax(bad)}"
        return {"n": int(g.size), "exact": 1.0}
    zero_w = (w & 0x7FFF) == 0
    zero_g = (g & 0x7FFF) == 0
    assert np.array_equal(zero_w, zero_g), f"{what}: zero positions differ ({int((zero_w != zero_g).sum())})"
    assert np.array_equal(g[zero_w], w[zero_w]), f"{what}: sign of a zero differs"
    d = bf16_ulp_diff(g, w)
    assert d.max(initial=0) <= 1, f"{what}: max ulp diff {d.max()} (at {np.argmax(d)})"
    return {"n": int(g.size), "exact": float((d == 0).mean()) if d.size else 1.0}


def assert_dprobs(got: np.ndarray, want: np.ndarray, abs_sum: np.ndarray, what: str) -> dict:
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bound = DPROBS_REL * abs_sum + 1e-30
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows beyond 2e-5*sum|term|; worst ratio "
                           f"{float((err / bound).max()):.3g}")
    rel = err / np.maximum(np.abs(want.astype(np.float64)), 1e-30)
    return {"max_err_over_scale": float((err / np.maximum(abs_sum, 1e-30)).max(initial=0)),
            "plain_rel_p50": float(np.median(rel)) if rel.size else 0.0,
            "plain_rel_max": float(rel.max(initial=0))}
