"""Pins of the oracle's float16 / float32 storage paths.

Pages: nemo_automodel.components.moe.swiglu_triton (_SUPPORTED_DTYPES: bf16,
fp16, fp32 for x) and nemo_automodel.components.moe.optimized_ops
(_RouterWeightMulFunction.forward: out_dtype may be the activation dtype, or
float32 where expert outputs are combined by scatter-add).

Anchors: numpy's float16 conversions (library routines), float64 torch.clamp /
F.silu / autograd, torch eager fp32 multiplies, exact rational sums.

float32 outputs are compared with bounds derived from the arithmetic: each of
the oracle's binary32 steps (expf, one division, a few multiplies and adds)
errs by at most about half an ulp, so y and d_up are within 8 ulps of the
float64 value. d_gate = (t*uc) * s*(1 + gc*(1-s)) is judged against the
magnitude of its two parts, M = |t*uc| * s*(1 + |gc|*(1-s)): the rounding of
s (half an ulp of 1 when s is near 1) enters 1-s as an absolute error and is
multiplied by gc, and the factor cancels near gc = -1.28, so the bound is
(|gc| + 8) ulps of M.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as oracle_module
from oracle import BF16, F16, F32
from tests.numerics import bf16_bits_to_f32, f64_to_bf16_exact, fraction_to_f32
from tests.test_oracle_pins import torch_bf16_bits, torch_swiglu_f64

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.fixture
def o():
    return oracle_module


def f16_order(h):
    h = np.asarray(h).view(np.uint16).astype(np.int64)
    mag = h & 0x7FFF
    return np.where(h & 0x8000, -mag, mag)


def f16_ulp_diff(a, b):
    return np.abs(f16_order(a) - f16_order(b))


# ---- float16 conversions --------------------------------------------------

def test_f16_widening_every_pattern_matches_numpy(o):
    got = np.array([o.f16_to_f32(int(h)) for h in ALL16], dtype=np.float32)
    ref = ALL16.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_rounding_matches_numpy_via_router_forward(o):
    # router forward with x = 1.0 (float32) and a float16 output returns f16(p)
    rng = np.random.default_rng(41)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    small = (rng.integers(0x33000000, 0x38800000, size=1 << 16, dtype=np.uint64)).astype(np.uint32)  # subnormal band
    ties = ((rng.integers(0x3880, 0x4780, size=1 << 15).astype(np.uint32) << 16) | 0x1000)             # half-ulp ties
    edge = np.array([0x477FEFFF, 0x477FF000, 0x477FF001, 0x477FE000, 0x33000000, 0x33000001, 0x33800000,
                     0x387FE000, 0x387FF000, 0x38800000, 0xC77FF000, 0x7F800000, 0x00000001], dtype=np.uint32)
    p = np.concatenate([bits, small, ties, edge]).view(np.float32)
    x = np.ones((p.size, 1), np.float32)
    out = o.router_weight_mul_fwd_typed(x, F32, p, F16, p.size, 1)[:, 0]
    with np.errstate(over="ignore", invalid="ignore"):
        ref = p.astype(np.float16)
    nan = np.isnan(p)
    assert np.array_equal(out[~nan].view(np.uint16), ref[~nan].view(np.uint16))
    assert np.isnan(out[nan]).all()


# ---- the typed functions with bfloat16 equal the bfloat16 ones -------------

def test_typed_bf16_equals_untyped(o):
    from moe_routed_expert_amd.workloads import WORKLOADS, custom
    w = WORKLOADS["swiglu_256x128"]
    d = w.generate()
    a = o.swiglu_clamped_fwd(d["x"], d["probs"], w.rows, w.cols, w.limit)
    b = o.swiglu_clamped_fwd_typed(d["x"], BF16, d["probs"], w.rows, w.cols, w.limit)
    assert np.array_equal(a, b)
    ga, pa = o.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], w.rows, w.cols, w.limit)
    gb, pb = o.swiglu_clamped_bwd_typed(d["x"], BF16, d["probs"], d["grad_out"], w.rows, w.cols, w.limit)
    assert np.array_equal(ga, gb) and np.array_equal(pa, pb)
    r = custom("router", 8, 256, x_sigma=1.0, seed=4).generate()
    assert np.array_equal(o.router_weight_mul_fwd(r["x"], r["probs"], 8, 256),
                          o.router_weight_mul_fwd_typed(r["x"], BF16, r["probs"], BF16, 8, 256))
    ga, pa = o.router_weight_mul_bwd(r["grad_out"], r["x"], r["probs"], 8, 256)
    gb, pb = o.router_weight_mul_bwd_typed(r["grad_out"], BF16, r["x"], BF16, r["probs"], 8, 256)
    assert np.array_equal(ga, gb) and np.array_equal(pa, pb)


# ---- clamped SwiGLU with float16 storage ------------------------------------

def _sweep_f16(o, gates, ups, p, gy, L):
    n = gates.size
    inter = 256
    rows = n // inter
    x = np.concatenate([gates.reshape(rows, inter), ups.reshape(rows, inter)], axis=1)
    probs = np.full(rows, p, np.float32)
    y = o.swiglu_clamped_fwd_typed(x, F16, probs, rows, inter, L).ravel()
    gx, _ = o.swiglu_clamped_bwd_typed(x, F16, probs, gy.reshape(rows, inter), rows, inter, L)
    return y, gx[:, :inter].ravel(), gx[:, inter:].ravel()


@pytest.mark.parametrize("which", ["gate", "up"])
def test_f16_every_pattern_vs_float64_autograd(which, o):
    L = 7.0
    allf = ALL16.view(np.float16)
    fixed = np.full(65536, 1.5, np.float16)
    gates, ups = (allf, fixed) if which == "gate" else (fixed, allf)
    gy = np.full(65536, -0.75, np.float16)
    y, dg, du = _sweep_f16(o, gates, ups, 0.5, gy, L)
    g64, u64 = gates.astype(np.float64)[None, :], ups.astype(np.float64)[None, :]
    ref_y, g_grad, u_grad, _ = torch_swiglu_f64(g64, u64, np.array([0.5]), L, gy=np.full((1, 65536), -0.75))
    ok = np.isfinite(allf.astype(np.float64))
    if which == "gate":
        ok &= allf.astype(np.float64) >= -87.0
    for got, ref in ((y, ref_y[0]), (dg, g_grad[0]), (du, u_grad[0])):
        want = ref.astype(np.float16)  # numpy: float64 -> float16 rounded directly
        d = f16_ulp_diff(got[ok], want[ok])
        assert d.max() <= 1, which
        assert (d == 0).mean() > 0.999
    v = allf.astype(np.float64)
    if which == "gate":
        assert np.all(dg.view(np.uint16)[~(v <= L)] == 0)
    else:
        assert np.all(du.view(np.uint16)[~(np.abs(v) <= L)] == 0)


# ---- clamped SwiGLU with float32 storage ------------------------------------

def test_f32_random_inputs_within_derived_bounds(o):
    rng = np.random.default_rng(42)
    rows, inter, L = 64, 512, 10.0
    g = (rng.standard_normal((rows, inter)) * 6).astype(np.float32)
    u = (rng.standard_normal((rows, inter)) * 6).astype(np.float32)
    g[:, :8] = [L, -L, np.nextafter(np.float32(L), np.float32(20)), 0.0, -0.0, -1.2785, 30.0, -30.0]
    u[:, :8] = [L, -L, np.nextafter(np.float32(-L), np.float32(-20)), 0.0, 3.0, 2.0, -12.0, 12.0]
    p = rng.random(rows, dtype=np.float32)
    gy = rng.standard_normal((rows, inter)).astype(np.float32)
    x = np.concatenate([g, u], axis=1)
    y = o.swiglu_clamped_fwd_typed(x, F32, p, rows, inter, L)
    gx, gp = o.swiglu_clamped_bwd_typed(x, F32, p, gy, rows, inter, L)
    ref_y, g_grad, u_grad, p_grad = torch_swiglu_f64(g.astype(np.float64), u.astype(np.float64),
                                                     p.astype(np.float64), L, gy=gy.astype(np.float64))
    eps = 2.0 ** -24
    assert np.all(np.abs(y - ref_y) <= 8 * eps * np.abs(ref_y) + 1e-37)
    assert np.all(np.abs(gx[:, inter:] - u_grad) <= 8 * eps * np.abs(u_grad) + 1e-37)
    gc = np.minimum(g.astype(np.float64), L)
    s = 1.0 / (1.0 + np.exp(-gc))
    uc = np.clip(u.astype(np.float64), -L, L)
    t = gy.astype(np.float64) * p[:, None]
    scale = np.abs(t * uc) * s * (1 + np.abs(gc) * (1 - s))
    assert np.all(np.abs(gx[:, :inter] - g_grad) <= (np.abs(gc) + 8) * eps * scale + 1e-37)
    # masks exact
    assert np.all(gx[:, :inter][g > L] == 0) and not np.signbit(gx[:, :inter][g > L]).any()
    assert np.all(gx[:, inter:][np.abs(u) > L] == 0)
    terms = np.abs(gy.astype(np.float64) * F_silu_uc(g, u, L)).sum(axis=1)
    assert np.all(np.abs(gp - p_grad) <= 1e-6 * terms)


def F_silu_uc(g, u, L):
    gc = np.minimum(g.astype(np.float64), L)
    return gc / (1.0 + np.exp(-gc)) * np.clip(u.astype(np.float64), -L, L)


# ---- router multiply with other dtypes --------------------------------------

@pytest.mark.parametrize("x_dtype,out_dtype", [(BF16, F32), (F16, F16), (F16, F32), (F32, F32), (BF16, BF16)])
def test_router_typed_forward_bitwise_equals_eager(x_dtype, out_dtype, o):
    rng = np.random.default_rng(43)
    rows, hidden = 24, 1000
    xf = rng.standard_normal((rows, hidden)).astype(np.float32)
    p = rng.random(rows, dtype=np.float32)
    if x_dtype == BF16:
        x = torch_bf16_bits(xf)
        xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    elif x_dtype == F16:
        x = xf.astype(np.float16)
        xt = torch.from_numpy(x)
    else:
        x = xf
        xt = torch.from_numpy(x)
    out = o.router_weight_mul_fwd_typed(x, x_dtype, p, out_dtype, rows, hidden)
    tdt = {BF16: torch.bfloat16, F16: torch.float16, F32: torch.float32}[out_dtype]
    ref = (xt.float() * torch.from_numpy(p)[:, None]).to(tdt)
    if out_dtype == BF16:
        assert np.array_equal(out, ref.view(torch.int16).numpy().view(np.uint16))
    else:
        assert np.array_equal(out.view(np.uint16 if out_dtype == F16 else np.uint32),
                              ref.numpy().view(np.uint16 if out_dtype == F16 else np.uint32))


def test_router_typed_backward_fp32_grad_out(o):
    # fp32 output (scatter-add path) -> fp32 grad_out; bf16 x
    rng = np.random.default_rng(44)
    rows, hidden = 6, 7168
    g = rng.standard_normal((rows, hidden)).astype(np.float32)
    x = torch_bf16_bits(rng.standard_normal((rows, hidden)).astype(np.float32))
    p = rng.random(rows, dtype=np.float32)
    gx, gp = o.router_weight_mul_bwd_typed(g, F32, x, BF16, p, rows, hidden)
    ref = (torch.from_numpy(g) * torch.from_numpy(p)[:, None]).to(torch.bfloat16)
    assert np.array_equal(gx, ref.view(torch.int16).numpy().view(np.uint16))
    x64 = bf16_bits_to_f32(x).astype(np.float64)
    for r in range(rows):
        # each fp32 x bf16 product is exact in float64; the oracle rounds each to
        # fp32 first, so it may differ from the exact sum by 2^-24 per term
        exact = sum((Fraction(float(v)) for v in g[r].astype(np.float64) * x64[r]), Fraction(0))
        bound = 2.0 ** -24 * float(np.abs(g[r].astype(np.float64) * x64[r]).sum()) + 1e-30
        assert abs(float(gp[r]) - float(fraction_to_f32(exact))) <= bound
