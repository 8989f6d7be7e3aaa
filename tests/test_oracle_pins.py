"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself or with a retyped copy of its
code. The anchors are:
  - library routines: torch's bfloat16 conversion, torch.nn.functional.silu and
    torch.clamp with torch.autograd (the pages name torch.clamp's inclusive
    masks as the clamp-gradient rule), evaluated in float64;
  - exhaustive sweeps over every bfloat16 pattern;
  - central and one-sided finite differences of the oracle's own unrounded
    forward (they check the backward against the forward, not against a
    formula);
  - exact rational sums for the router probability gradient;
  - hand-derived exact cases (tests/golden/swiglu_clamped_exact_cases.tsv);
  - structural brute force on a 4 x 8 input (which outputs depend on which
    inputs) and exact power-of-two scaling invariants.
Pages: nemo_automodel.components.moe.swiglu_triton (module description) and
nemo_automodel.components.moe.optimized_ops (_RouterWeightMulFunction and the
_rw_*_core entries).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as oracle_module
from moe_routed_expert_amd.workloads import WORKLOADS, custom
from tests.numerics import (bf16_bits_to_f32, bf16_is_nan, bf16_ulp_diff, f32_ulp,
                            f64_to_bf16_exact, fraction_to_f32)

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
ALL_F = bf16_bits_to_f32(ALL_BF16)
with np.errstate(invalid="ignore"):
    ALL_F64 = ALL_F.astype(np.float64)
FINITE_BF16 = ALL_BF16[np.isfinite(ALL_F)]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "swiglu_clamped_exact_cases.tsv")


def torch_bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_swiglu_f64(gate, up, p, L, gy=None):
    """The pages' expression with library routines in float64 (torch.clamp,
    F.silu; autograd for the gradients). gate/up: [rows, inter]; p: [rows]."""
    g = torch.tensor(np.asarray(gate, np.float64), requires_grad=gy is not None)
    u = torch.tensor(np.asarray(up, np.float64), requires_grad=gy is not None)
    pp = torch.tensor(np.asarray(p, np.float64)[:, None], requires_grad=gy is not None)
    y = F.silu(torch.clamp(g, max=L)) * torch.clamp(u, -L, L) * pp
    if gy is None:
        return y.detach().numpy(), None, None, None
    y.backward(torch.tensor(np.asarray(gy, np.float64)))
    return y.detach().numpy(), g.grad.numpy(), u.grad.numpy(), pp.grad.numpy()[:, 0]


@pytest.fixture
def o():
    """The oracle under test (tests/test_oracle_mutations.py passes planted-mistake builds)."""
    return oracle_module


def split_gate_up(x_bits, inter):
    xf = bf16_bits_to_f32(x_bits).astype(np.float64)
    return xf[:, :inter], xf[:, inter:]


# ---- the test helpers themselves, against torch's conversions -------------

def test_helper_exact_bf16_rounding_agrees_with_torch_on_f32_inputs(o):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    ties = ((rng.integers(0, 2**16, size=20_000).astype(np.uint32) << 16) | 0x8000).astype(np.uint32)
    f = np.concatenate([bits, ties]).view(np.float32)
    f = f[~np.isnan(f)]
    assert np.array_equal(f64_to_bf16_exact(f.astype(np.float64)), torch_bf16_bits(f))


def test_helper_fraction_rounding_agrees_with_hardware_conversion(o):
    rng = np.random.default_rng(12)
    d = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 39, 2000),
                        rng.standard_normal(200) * 1e-42])
    for v in d:
        assert fraction_to_f32(Fraction(float(v))) == np.float32(v)


# ---- bfloat16 conversion inside the oracle ---------------------------------

def test_oracle_widening_is_exact_for_every_pattern(o):
    got = np.array([o.bf16_to_f32(int(b)) for b in ALL_BF16], dtype=np.float32)
    nan = np.isnan(ALL_F)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ALL_F[~nan].view(np.uint32))


def test_oracle_rounding_matches_torch_via_router_forward(o):
    # router forward with x = 1.0 returns bf16(p): the oracle's rounding on
    # every p, including all tie patterns and values next to the overflow edge.
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    ties = ((np.arange(1 << 16, dtype=np.uint32) << 16) | 0x8000)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7E8000, 0x00008000, 0x00018000,
                     0x80008000, 0x00007FFF, 0xFF7F8000], dtype=np.uint32)
    p = np.concatenate([bits, ties, edge]).view(np.float32)
    x = np.full((p.size, 1), 0x3F80, dtype=np.uint16)
    out = o.router_weight_mul_fwd(x, p, p.size, 1)[:, 0]
    ref = torch_bf16_bits(p)
    nan = np.isnan(p)
    assert np.array_equal(out[~nan], ref[~nan])
    assert bf16_is_nan(out[nan]).all()


# ---- clamped SwiGLU forward -------------------------------------------------

def _sweep_fwd(o, gates, ups, p, L):
    n = gates.size
    inter = 256
    rows = n // inter
    x = np.concatenate([gates.reshape(rows, inter), ups.reshape(rows, inter)], axis=1)
    probs = np.full(rows, p, dtype=np.float32)
    return o.swiglu_clamped_fwd(x, probs, rows, inter, L).ravel()


@pytest.mark.parametrize("L", [7.0, 10.0])
def test_fwd_every_bf16_gate_vs_float64_library(L, o):
    gates = ALL_BF16
    ups = np.full_like(gates, 0x3F80)                       # up = 1
    y = _sweep_fwd(o, gates, ups, 1.0, L)
    gf = ALL_F64
    ref64, *_ = torch_swiglu_f64(gf[None, :], np.ones((1, gf.size)), np.ones(1), L)
    ref = f64_to_bf16_exact(ref64[0])
    nan = np.isnan(gf) | np.isnan(ref64[0])
    assert np.array_equal(bf16_is_nan(y), nan)
    ok = ~nan & (gf >= -87.0)
    d = bf16_ulp_diff(y[ok], ref[ok])
    assert d.max() <= 1
    assert (d == 0).mean() > 0.999
    deep = ~nan & (gf < -87.0)
    assert np.all(np.abs(bf16_bits_to_f32(y[deep]).astype(np.float64) - ref64[0][deep]) <= 1e-30)


def test_fwd_every_bf16_up_vs_float64_library(o):
    L = 7.0
    ups = ALL_BF16
    gates = np.full_like(ups, 0x3FC0)                       # gate = 1.5
    p = np.float32(0.75)
    y = _sweep_fwd(o, gates, ups, p, L)
    uf = ALL_F64
    ref64, *_ = torch_swiglu_f64(np.full((1, uf.size), 1.5), uf[None, :], np.array([0.75]), L)
    ref = f64_to_bf16_exact(ref64[0])
    nan = np.isnan(uf)
    assert np.array_equal(bf16_is_nan(y), nan)
    d = bf16_ulp_diff(y[~nan], ref[~nan])
    assert d.max() <= 1 and (d == 0).mean() > 0.999
    # saturation: every |up| >= L gives the same value as up = +-L
    big = ~nan & (np.abs(uf) >= L)
    pos = y[big & (uf > 0)]
    neg = y[big & (uf < 0)]
    assert np.all(pos == pos[0]) and np.all(neg == neg[0])


@pytest.mark.parametrize("name", ["swiglu_256x128"])
def test_fwd_workload_vs_float64_library(name, o):
    w = WORKLOADS[name]
    d = w.generate()
    y = o.swiglu_clamped_fwd(d["x"], d["probs"], w.rows, w.cols, w.limit)
    g, u = split_gate_up(d["x"], w.cols)
    ref64, *_ = torch_swiglu_f64(g, u, d["probs"].astype(np.float64), w.limit)
    diff = bf16_ulp_diff(y, f64_to_bf16_exact(ref64))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.995


def test_fwd_reduces_to_textbook_swiglu_without_clamp(o):
    # With L beyond every input and p = 1 the method is silu(gate) * up.
    rng = np.random.default_rng(14)
    rows, inter = 64, 96
    gf = (rng.standard_normal((rows, inter)) * 6).astype(np.float32)
    uf = (rng.standard_normal((rows, inter)) * 6).astype(np.float32)
    x = np.concatenate([torch_bf16_bits(gf), torch_bf16_bits(uf)], axis=1)
    y = o.swiglu_clamped_fwd(x, np.ones(rows, np.float32), rows, inter, 1e30)
    gt = torch.from_numpy(bf16_bits_to_f32(x[:, :inter]))
    ut = torch.from_numpy(bf16_bits_to_f32(x[:, inter:]))
    ref = (F.silu(gt) * ut).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert bf16_ulp_diff(y, ref).max() <= 1


# ---- clamped SwiGLU backward -----------------------------------------------

def _sweep_bwd(o, gates, ups, p, gy_bits, L):
    n = gates.size
    inter = 256
    rows = n // inter
    x = np.concatenate([gates.reshape(rows, inter), ups.reshape(rows, inter)], axis=1)
    probs = np.full(rows, p, dtype=np.float32)
    gx, gp = o.swiglu_clamped_bwd(x, probs, gy_bits.reshape(rows, inter), rows, inter, L)
    return gx[:, :inter].ravel(), gx[:, inter:].ravel(), gp


def test_bwd_every_bf16_gate_vs_autograd(o):
    L = 7.0
    gates = ALL_BF16
    ups = np.full_like(gates, 0x3FC0)                       # up = 1.5
    gy = np.full_like(gates, 0x3F80)                        # gy = 1
    dg, du, _ = _sweep_bwd(o, gates, ups, 1.0, gy, L)
    gf = ALL_F64
    _, g_grad, u_grad, _ = torch_swiglu_f64(gf[None, :], np.full((1, gf.size), 1.5), np.ones(1), L,
                                            gy=np.ones((1, gf.size)))
    ok = np.isfinite(gf) & (gf >= -87.0)
    assert bf16_ulp_diff(dg[ok], f64_to_bf16_exact(g_grad[0][ok])).max() <= 1
    assert bf16_ulp_diff(du[ok], f64_to_bf16_exact(u_grad[0][ok])).max() <= 1
    # the gate mask: +0 exactly where gate > L or gate is NaN, never elsewhere
    masked = ~(gf <= L)
    assert np.all(dg[masked] == 0x0000)
    assert np.all(dg[ok & ~masked] & 0x7FFF != 0)
    # gate has no lower clamp: far below -L the gradient is still there
    assert np.all(dg[ok & (gf < -L)] != 0)


def test_bwd_every_bf16_up_vs_autograd(o):
    L = 7.0
    ups = ALL_BF16
    gates = np.full_like(ups, 0x3FC0)                       # gate = 1.5
    gy = np.full_like(ups, 0xBF40)                          # gy = -0.75
    dg, du, _ = _sweep_bwd(o, gates, ups, 0.5, gy, L)
    uf = ALL_F64
    _, g_grad, u_grad, _ = torch_swiglu_f64(np.full((1, uf.size), 1.5), uf[None, :], np.array([0.5]), L,
                                            gy=np.full((1, uf.size), -0.75))
    ok = ~np.isnan(uf)
    assert bf16_ulp_diff(dg[ok], f64_to_bf16_exact(g_grad[0][ok])).max() <= 1
    assert bf16_ulp_diff(du[ok], f64_to_bf16_exact(u_grad[0][ok])).max() <= 1
    inside = np.abs(uf) <= L
    assert np.all(du[~inside] == 0x0000)                 # masked: +0, also for NaN
    nonzero_u = inside & (uf != 0)
    assert np.all(du[nonzero_u] & 0x7FFF != 0)
    assert np.all(du[inside & (uf == 0)] & 0x7FFF != 0)  # d_up = t*silu(gate) does not depend on up


@pytest.mark.parametrize("wl", [
    WORKLOADS["swiglu_256x128"],
    custom("swiglu", 48, 200, limit=7.0, x_sigma=5.0, seed=21, x_special_frac=0.3,
           x_special_values=(-7.0, 7.0, 0.0, -7.03125, 7.03125, -6.96875, 6.96875),
           probs_kind="uniform_zeros", probs_zero_frac=0.2),
])
def test_bwd_workload_vs_autograd(wl, o):
    d = wl.generate()
    gx, gp = o.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], wl.rows, wl.cols, wl.limit)
    g, u = split_gate_up(d["x"], wl.cols)
    gy = bf16_bits_to_f32(d["grad_out"]).astype(np.float64)
    _, g_grad, u_grad, p_grad = torch_swiglu_f64(g, u, d["probs"].astype(np.float64), wl.limit, gy=gy)
    I = wl.cols
    assert bf16_ulp_diff(gx[:, :I], f64_to_bf16_exact(g_grad)).max() <= 1
    assert bf16_ulp_diff(gx[:, I:], f64_to_bf16_exact(u_grad)).max() <= 1
    # masked positions are +0 bits; torch.clamp's mask is inclusive
    L = wl.limit
    assert np.all(gx[:, :I][g > L] == 0)
    assert np.all(gx[:, I:][np.abs(u) > L] == 0)
    # probability gradient: float64 autograd sums float64 terms; the oracle sums
    # float32 terms in float64. Scale = sum of |terms|.
    h = F.silu(torch.clamp(torch.tensor(g), max=L)).numpy() * np.clip(u, -L, L)
    scale = np.abs(gy * h).sum(axis=1)
    assert np.all(np.abs(gp.astype(np.float64) - p_grad) <= 1e-6 * scale + 1e-30)


def test_bwd_zero_probability_rows(o):
    wl = WORKLOADS["swiglu_100003x1536"]
    d = wl.generate(rows=4096)
    rows = 4096
    zero = d["probs"] == 0
    assert 0.1 < zero.mean() < 0.3
    y = o.swiglu_clamped_fwd(d["x"], d["probs"], rows, wl.cols, wl.limit)
    gx, gp = o.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], rows, wl.cols, wl.limit)
    assert np.all(y[zero] & 0x7FFF == 0)                 # +-0
    assert np.all(gx[zero] & 0x7FFF == 0)
    assert np.all(gp[zero] != 0)                         # d_probs does not vanish with p


def _golden_rows():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            f = line.rstrip("\n").split("\t")
            rows.append(f)
    return rows


def _closed(expr):
    return float(eval(expr[1:], {"__builtins__": {}}, {"s": lambda z: 1.0 / (1.0 + math.exp(-z)),
                                                         "exp": math.exp}))


@pytest.mark.parametrize("case", _golden_rows(), ids=lambda f: f[0])
def test_bwd_hand_derived_cases(case, o):
    name, L, g, u, p, gy = case[0], *map(float, case[1:6])
    expects = case[6:10]
    q = o.swiglu_point(g, u, p, gy, L)
    x = np.array([[o.f32_to_bf16(g), o.f32_to_bf16(u)]], dtype=np.uint16)
    assert bf16_bits_to_f32(x)[0, 0] == np.float32(g) and bf16_bits_to_f32(x)[0, 1] == np.float32(u)
    y = o.swiglu_clamped_fwd(x, np.array([p], np.float32), 1, 1, L)[0, 0]
    gx, gp = o.swiglu_clamped_bwd(x, np.array([p], np.float32),
                                       np.array([[o.f32_to_bf16(gy)]], np.uint16), 1, 1, L)
    got = [int(y), int(gx[0, 0]), int(gx[0, 1])]
    for want, have in zip(expects[:3], got):
        if want.startswith("0x"):
            assert have == int(want, 16), (name, hex(have), want)
        else:
            ref = f64_to_bf16_exact(np.array([_closed(want)]))[0]
            assert bf16_ulp_diff(np.array([have], np.uint16), np.array([ref]))[0] <= 1, (name, hex(have), hex(ref))
    term = _closed(expects[3])
    assert abs(q[3] - term) <= 4 * f32_ulp(term) + 1e-30
    assert abs(float(gp[0]) - term) <= 4 * f32_ulp(term) + 1e-30


def test_bwd_matches_central_finite_differences(o):
    # d/dg, d/du and d/dp of the oracle's own unrounded forward (gy = 1), at
    # random points away from the clamp kinks.
    rng = np.random.default_rng(15)
    L = 7.0
    checked = 0
    for _ in range(400):
        g, u = rng.uniform(-12, 12, 2)
        p = rng.uniform(0.05, 1.0)
        if abs(g - L) < 0.05 or abs(abs(u) - L) < 0.05:
            continue
        _, dg, du, term = o.swiglu_point(g, u, p, 1.0, L)
        f = lambda gg, uu, pp: o.swiglu_point(gg, uu, pp, 1.0, L)[0]
        hg = hu = 1e-2
        fd_g = (f(g + hg, u, p) - f(g - hg, u, p)) / (2 * hg)
        fd_u = (f(g, u + hu, p) - f(g, u - hu, p)) / (2 * hu)
        fd_p = (f(g, u, p + 1e-3) - f(g, u, p - 1e-3)) / 2e-3
        assert abs(fd_g - dg) <= 2e-3 * abs(dg) + 2e-3, (g, u, p, fd_g, dg)
        assert abs(fd_u - du) <= 2e-3 * abs(du) + 2e-3, (g, u, p, fd_u, du)
        assert abs(fd_p - term) <= 2e-3 * abs(term) + 2e-3, (g, u, p, fd_p, term)
        checked += 1
    assert checked > 300


def test_bwd_one_sided_differences_at_the_limits(o):
    # At exactly +-L the inclusive masks keep the derivative from inside the
    # interval; one step outside, the function is flat and the gradient is +0.
    L, p, h = 7.0, 0.5, 1e-3
    f = lambda g, u: o.swiglu_point(g, u, p, 1.0, L)[0]
    for u in (-3.0, 2.0, L, -L):
        dg = o.swiglu_point(L, u, p, 1.0, L)[1]
        inside = (f(L, u) - f(L - h, u)) / h
        assert abs(inside - dg) <= 5e-3 * abs(dg) + 1e-3
        assert (f(L + h, u) - f(L, u)) == 0.0
        assert o.swiglu_point(7.03125, u, p, 1.0, L)[1] == 0.0
    for g in (-2.0, 0.5, 3.0, L):
        du_hi = o.swiglu_point(g, L, p, 1.0, L)[2]
        assert abs((f(g, L) - f(g, L - h)) / h - du_hi) <= 5e-3 * abs(du_hi) + 1e-3
        du_lo = o.swiglu_point(g, -L, p, 1.0, L)[2]
        assert abs((f(g, -L + h) - f(g, -L)) / h - du_lo) <= 5e-3 * abs(du_lo) + 1e-3
        assert o.swiglu_point(g, 7.03125, p, 1.0, L)[2] == 0.0
        assert o.swiglu_point(g, -7.03125, p, 1.0, L)[2] == 0.0
    # below -L the gate is not clamped: the central difference is the gradient
    g = -8.0
    dg = o.swiglu_point(g, 1.0, p, 1.0, L)[1]
    fd = (f(g + h, 1.0) - f(g - h, 1.0)) / (2 * h)
    assert dg != 0.0 and abs(fd - dg) <= 5e-3 * abs(dg) + 1e-4


def test_grad_probs_keep_small_terms_next_to_cancelling_large_ones(o):
    # One row: gate = up = L = 8192 gives the term +2^26 (exact), then 126
    # elements with gate = up = 1 (term silu(1)), then up = -8192 gives -2^26.
    # The large terms cancel exactly; a sum carried at float64 keeps the small
    # ones (a float32 running sum would lose every one of them next to 2^26).
    L, inter = 8192.0, 128
    g = np.ones(inter, np.float32)
    u = np.ones(inter, np.float32)
    g[0] = g[-1] = 8192.0
    u[0], u[-1] = 8192.0, -8192.0
    x = np.concatenate([torch_bf16_bits(g), torch_bf16_bits(u)])[None, :]
    gy = np.full((1, inter), 0x3F80, np.uint16)
    _, gp = o.swiglu_clamped_bwd(x, np.ones(1, np.float32), gy, 1, inter, L)
    _, _, _, p_grad = torch_swiglu_f64(g[None, :].astype(np.float64), u[None, :].astype(np.float64),
                                       np.ones(1), L, gy=np.ones((1, inter)))
    assert abs(p_grad[0] - 126 * (1.0 / (1.0 + math.exp(-1.0)))) < 1e-6
    assert abs(float(gp[0]) - p_grad[0]) <= 1e-4, (gp[0], p_grad[0])


def test_bruteforce_4x8_dependency_structure(o):
    # rows = 4, inter = 4 (x is 4 x 8). Change one input at a time to a very
    # different value and record which outputs move: y[r, j], d_gate[r, j] and
    # d_up[r, j] may depend only on x[r, j], x[r, 4 + j], p[r] (and gy[r, j]);
    # d_probs[r] only on row r. Values sit at L, one bf16 step either side of
    # +-L, at 0 and in between, so every mask pattern occurs.
    L = 7.0
    vals = [7.0, 7.03125, 6.96875, -7.0, -7.03125, -6.96875, 0.0, 2.5, -9.0, 11.0, -0.5, 7.0]
    rng = np.random.default_rng(16)
    rows, inter = 4, 4
    xf = rng.choice(vals, size=(rows, 2 * inter)).astype(np.float32)
    x = torch_bf16_bits(xf)
    p = np.array([0.5, 0.25, 1.0, 0.75], np.float32)
    gy = torch_bf16_bits(rng.choice([1.0, -0.5, 2.0], size=(rows, inter)).astype(np.float32))

    def run(x_, p_, gy_):
        y = o.swiglu_clamped_fwd(x_, p_, rows, inter, L)
        gx, gp = o.swiglu_clamped_bwd(x_, p_, gy_, rows, inter, L)
        return y, gx, gp

    y0, gx0, gp0 = run(x, p, gy)
    for r in range(rows):
        for c in range(2 * inter):
            x1 = x.copy()
            x1[r, c] = torch_bf16_bits(np.array([3.25 if xf[r, c] != 3.25 else -1.5], np.float32))[0]
            y1, gx1, gp1 = run(x1, p, gy)
            j = c % inter
            allowed = np.zeros((rows, inter), bool)
            allowed[r, j] = True
            assert np.all((y1 != y0) <= allowed)
            assert np.all((gx1[:, :inter] != gx0[:, :inter]) <= allowed)
            assert np.all((gx1[:, inter:] != gx0[:, inter:]) <= allowed)
            assert np.all((gp1 != gp0) <= (np.arange(rows) == r))
            new = float(bf16_bits_to_f32(x1[r:r + 1, c])[0])
            if c < inter and xf[r, inter + j] != 0 and not (xf[r, c] > L and new > L):
                # the gate slot feeds d_gate through silu'; unless the gate stays
                # masked or up is 0 (a zero factor), d_gate must change
                assert gx1[r, j] != gx0[r, j]
    # mask pattern at every position: a masked gradient is +0 bits; otherwise
    # it is zero only through a zero factor (up = 0 for d_gate, gate = 0 for d_up)
    gate, up = xf[:, :inter], xf[:, inter:]
    assert np.all(gx0[:, :inter][gate > L] == 0x0000)
    assert np.all(gx0[:, inter:][np.abs(up) > L] == 0x0000)
    assert np.array_equal(gx0[:, :inter] & 0x7FFF == 0, (gate > L) | (up == 0))
    assert np.array_equal(gx0[:, inter:] & 0x7FFF == 0, (np.abs(up) > L) | (gate == 0))


def test_power_of_two_scaling_is_exact(o):
    wl = WORKLOADS["swiglu_256x128"]
    d = wl.generate()
    rows, I, L = wl.rows, wl.cols, wl.limit
    gy2 = torch_bf16_bits(bf16_bits_to_f32(d["grad_out"]) * 2)
    gx1, gp1 = o.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], rows, I, L)
    gx2, gp2 = o.swiglu_clamped_bwd(d["x"], d["probs"], gy2, rows, I, L)
    assert np.array_equal(bf16_bits_to_f32(gx2), bf16_bits_to_f32(gx1) * 2)
    assert np.array_equal(gp2, gp1 * 2)
    y1 = o.swiglu_clamped_fwd(d["x"], d["probs"], rows, I, L)
    y2 = o.swiglu_clamped_fwd(d["x"], d["probs"] * 2, rows, I, L)
    assert np.array_equal(bf16_bits_to_f32(y2), bf16_bits_to_f32(y1) * 2)


# ---- router-weight multiply -------------------------------------------------

def _router_inputs(rows, hidden, seed):
    w = custom("router", rows, hidden, x_sigma=1.0, seed=seed)
    return w.generate()


def test_router_fwd_bitwise_equals_eager_fp32_multiply(o):
    # The page states that this forward equals the eager (x.float() * probs.float()).to(dtype) bit for bit.
    d = _router_inputs(96, 7168, 31)
    out = o.router_weight_mul_fwd(d["x"], d["probs"], 96, 7168)
    xt = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16)
    ref = (xt.float() * torch.from_numpy(d["probs"])[:, None]).to(torch.bfloat16)
    assert np.array_equal(out, ref.view(torch.int16).numpy().view(np.uint16))


def test_router_bwd_grad_x_bitwise_equals_eager_and_grad_probs_exact(o):
    rows, hidden = 12, 7168
    d = _router_inputs(rows, hidden, 32)
    gx, gp = o.router_weight_mul_bwd(d["grad_out"], d["x"], d["probs"], rows, hidden)
    gt = torch.from_numpy(d["grad_out"].view(np.int16)).view(torch.bfloat16)
    ref = (gt.float() * torch.from_numpy(d["probs"])[:, None]).to(torch.bfloat16)
    assert np.array_equal(gx, ref.view(torch.int16).numpy().view(np.uint16))
    # every product of two bf16 values is exact in float64; their exact rational
    # sum, rounded once, is the correctly rounded gradient
    g64 = bf16_bits_to_f32(d["grad_out"]).astype(np.float64)
    x64 = bf16_bits_to_f32(d["x"]).astype(np.float64)
    exact_hits = 0
    for r in range(rows):
        s = sum((Fraction(float(v)) for v in g64[r] * x64[r]), Fraction(0))
        want = fraction_to_f32(s)
        assert abs(float(gp[r]) - float(want)) <= f32_ulp(want), (r, gp[r], want)
        exact_hits += int(gp[r] == want)
    assert exact_hits >= rows - 1
    # and it agrees with torch autograd's float32 chain within a float32 sum's error
    xt = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16)
    pt = torch.from_numpy(d["probs"])[:, None].clone().requires_grad_(True)
    (xt.float() * pt).to(torch.bfloat16).float().backward(gt.float())
    scale = np.abs(g64 * x64).sum(axis=1)
    assert np.all(np.abs(pt.grad.numpy()[:, 0] - gp) <= 1e-5 * scale)


def test_router_bwd_without_probability_gradient_skips_x(o):
    rows, hidden = 8, 512
    d = _router_inputs(rows, hidden, 33)
    gx_a, gp_a = o.router_weight_mul_bwd(d["grad_out"], d["x"], d["probs"], rows, hidden)
    gx_b, gp_b = o.router_weight_mul_bwd(d["grad_out"], None, d["probs"], rows, hidden,
                                              want_grad_probs=False)
    assert gp_b is None and np.array_equal(gx_a, gx_b)


def test_oracle_threads_do_not_change_results(o):
    wl = WORKLOADS["swiglu_256x128"]
    d = wl.generate()
    a = o.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], wl.rows, wl.cols, wl.limit, threads=1)
    b = o.swiglu_clamped_bwd(d["x"], d["probs"], d["grad_out"], wl.rows, wl.cols, wl.limit, threads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
