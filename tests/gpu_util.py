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

from tests.numerics import bf16_is_nan, bf16_ulp_diff, f16_is_nan

DPROBS_REL = 2e-5


def to_dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def to_dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bf16_parity(got: np.ndarray, want: np.ndarray, what: str, exact: bool = False,
                       is_nan=bf16_is_nan) -> dict:
    assert got.shape == want.shape, (what, got.shape, want.shape)
    nan_w, nan_g = is_nan(want), is_nan(got)
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


# ---- float16 / float32 storage -------------------------------------------------
#
# float16 outputs: the bfloat16 bar with float16 ulps (1 ulp, zeros bit-exact).
# float32 outputs: no rounding hides the difference between the kernels'
# exp (v_exp_f32 of -z*log2(e), whose argument rounding is worth up to |z|
# ulps of e^-z and so of sigma) and reciprocal (v_rcp_f32) and the oracle's
# expf and division; every other step is the same binary32 operation in the
# same order. The oracle is within 8 ulps (y, d_up) or (|gc| + 8) ulps of the
# scale M = |t*uc|*s*(1 + |gc|*(1-s)) (d_gate) of the exact value, the kernels
# add |gc| + 8 ulps of sigma's error, carried through (1-s)*gc once more for
# d_gate. Bar: y, d_up within (|gc| + 16) * 2^-24 * |oracle|; d_gate within
# (3*|gc| + 16) * 2^-24 * M; zeros bit-exact.

def f16_bits(a) -> np.ndarray:
    return np.asarray(a).view(np.uint16)


def assert_f16_parity(got: np.ndarray, want: np.ndarray, what: str) -> dict:
    # Same sign-magnitude ulp order as bfloat16; only the NaN encoding differs.
    return assert_bf16_parity(f16_bits(got), f16_bits(want), what, is_nan=f16_is_nan)


def f32_swiglu_bounds(x: np.ndarray, probs: np.ndarray, grad_y: np.ndarray, L: float):
    """Per-element allowed |gpu - oracle| for y, d_gate and d_up (float32 storage)."""
    inter = x.shape[1] // 2
    g = x[:, :inter].astype(np.float64)
    u = x[:, inter:].astype(np.float64)
    gc = np.minimum(g, L)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-gc))
    uc = np.clip(u, -L, L)
    p = probs.astype(np.float64)[:, None]
    a = np.abs(gc * s)
    eps = 2.0 ** -24
    y_abs = a * np.abs(uc) * np.abs(p)
    t = np.abs(grad_y.astype(np.float64) * p)
    m = t * np.abs(uc) * s * (1 + np.abs(gc) * (1 - s))
    b_y = (np.abs(gc) + 16) * eps * y_abs + 1e-37
    b_dg = (3 * np.abs(gc) + 16) * eps * m + 1e-37
    b_du = (np.abs(gc) + 16) * eps * t * a + 1e-37
    return b_y, b_dg, b_du


def assert_f32_within(got: np.ndarray, want: np.ndarray, bound: np.ndarray, what: str) -> dict:
    nan_w, nan_g = np.isnan(want), np.isnan(got)
    assert np.array_equal(nan_w, nan_g), f"{what}: NaN positions differ"
    ok = ~nan_w
    zero = ok & (want == 0)
    assert np.array_equal(got[zero].view(np.uint32), want[zero].view(np.uint32)), f"{what}: zeros differ"
    err = np.abs(got[ok].astype(np.float64) - want[ok].astype(np.float64))
    bad = err > bound[ok]
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond the float32 bound"
    return {"max_err_over_bound": float((err / bound[ok]).max(initial=0)), "exact": float((err == 0).mean())}


# ---- grouped GEMM output (bf16 of an fp32-accumulated sum) ---------------------
#
# The kernel accumulates the K = hidden exact bf16 products in fp32 (in the MFMA
# units' order) and rounds the sum once to bf16. Against the exact sum S, an fp32
# accumulation of K terms in any order errs by at most gamma_K * sum|a*w| with
# gamma_K = K u / (1 - K u), u = 2^-24; the bar doubles that (an accumulator that
# truncated instead of rounding would still pass) and adds half a bf16 ulp for
# the final rounding.

def bf16_spacing(v: np.ndarray) -> np.ndarray:
    """bfloat16 ulp at |v| (subnormal spacing 2^-133 below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def assert_gemm_bf16_within(got_bits: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray, k: int, what: str) -> dict:
    from tests.numerics import bf16_bits_to_f32
    got = bf16_bits_to_f32(got_bits).astype(np.float64)
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    bound = 2 * gamma * abs_sum + 0.5 * bf16_spacing(np.maximum(np.abs(got), np.abs(exact)))
    err = np.abs(got - exact)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {got.size} beyond the fp32-accumulation bound"
    from tests.numerics import f64_to_bf16_exact
    return {"n": int(got.size), "equal_to_exact_rounding": float((got_bits == f64_to_bf16_exact(exact)).mean()),
            "max_err_over_bound": float((err / bound).max(initial=0))}


# ---- down projection + router multiply ------------------------------------------
#
# out = round_out(fp32(c) * p) where c is the kernel's bf16 GEMM output. c itself
# is not an output, so the bar asks that some bf16 value c that passes the GEMM
# bound above (|c - S| <= 2 gamma_K sum|h*w| + half a bf16 ulp) gives exactly
# `got` through the router multiply's definition: one binary32 product, rounded
# once to the output dtype. For float32 output c is the bf16 value nearest to
# got / p (the product's own rounding, 2^-24 relative, is far below bf16's
# spacing); for bf16 output the candidates are the bf16 values within 3 ulps of
# got / p, and -0. The bf16 rounding of the exact sum is tried first in both.

def _bf16_from_order(o: np.ndarray) -> np.ndarray:
    o = np.asarray(o, dtype=np.int64)
    return np.where(o >= 0, o, 0x8000 | (-o)).astype(np.uint16)


def assert_down_router_within(got: np.ndarray, out_is_f32: bool, exact: np.ndarray, abs_sum: np.ndarray,
                              probs: np.ndarray, k: int, what: str) -> dict:
    from tests.numerics import bf16_bits_to_f32, bf16_order, f64_to_bf16_exact
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    p = np.broadcast_to(np.asarray(probs, np.float32).reshape(-1, 1), exact.shape)
    got_f = got.astype(np.float64) if out_is_f32 else bf16_to_f64(got)
    zero_p = p == 0
    assert (got_f[zero_p] == 0).all(), f"{what}: nonzero output where the probability is 0"
    nz = ~zero_p
    ratio = np.where(nz, got_f / np.where(nz, p, 1).astype(np.float64), 0.0)
    center = bf16_order(f64_to_bf16_exact(ratio))

    def bound_ok(c_bits):
        c = bf16_bits_to_f32(c_bits).astype(np.float64)
        bound = 2 * gamma * abs_sum + 0.5 * bf16_spacing(np.maximum(np.abs(c), np.abs(exact)))
        return np.abs(c - exact) <= bound

    def through_router(c_bits):
        prod = bf16_bits_to_f32(c_bits) * p                     # one binary32 product
        return prod if out_is_f32 else f64_to_bf16_exact(prod.astype(np.float64))

    ok = zero_p.copy()
    chosen = np.zeros(exact.shape, np.uint16)
    steps = [0] if out_is_f32 else [0, -1, 1, -2, 2, -3, 3]
    # the exact sum's own rounding first, so the statistic below counts the outputs it explains
    cands = [f64_to_bf16_exact(exact)] + [_bf16_from_order(center + s) for s in steps] + \
        [np.full(exact.shape, 0x8000, np.uint16)]
    for c in cands:
        r = through_router(c)
        same = (r.view(np.uint32) == got.view(np.uint32)) if out_is_f32 else (r == got)
        hit = ~ok & same & bound_ok(c)
        chosen[hit] = c[hit]
        ok |= hit
    bad = ~ok
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {got.size} outputs are not the router multiply of a bf16 "
                           f"value within the fp32-accumulation bound (first at {np.argmax(bad.ravel())})")
    eq = chosen[nz] == f64_to_bf16_exact(exact[nz])
    return {"n": int(got.size), "c_equal_to_exact_rounding": float(eq.mean()) if eq.size else 1.0}


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    from tests.numerics import bf16_bits_to_f32
    return bf16_bits_to_f32(bits).astype(np.float64)
