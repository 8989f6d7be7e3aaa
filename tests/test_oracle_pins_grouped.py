"""Pins of the oracle's gate_up grouped GEMM with the clamped SwiGLU epilogue.

Pages: nemo_automodel.components.moe.mok_experts (routed gate / up weights,
bf16 [local_experts, expert_intermediate, hidden]);
nemo_automodel.components.moe.quantized_experts, _mxfp4_base_mm (activations
[tokens, in_dim] grouped contiguously by local expert, offs int32 cumulative
token counts, result [tokens, out_dim] in the activation dtype);
nemo_automodel.components.moe.swiglu_triton (the epilogue on that output).

Anchors: integer matrix products (numpy int64), float64 numpy matmuls, exact
rational sums, a nearest-value search over every finite bfloat16 and the
exact-rounding helper of tests/numerics.py (itself pinned to torch).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as oracle_module
from tests.numerics import bf16_bits_to_f32, f64_to_bf16_exact


@pytest.fixture
def o():
    return oracle_module


def bf16_bits(v):
    """float values that are exact in bfloat16 -> their bit patterns."""
    f = np.asarray(v, dtype=np.float32)
    assert np.array_equal(bf16_bits_to_f32((f.view(np.uint32) >> 16).astype(np.uint16)), f), "not exact in bf16"
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def ranges(offs, tokens):
    """[start, end) of each expert under the oracle's reading of offs."""
    out, start = [], 0
    for c in offs:
        end = min(max(int(c), start), tokens)
        out.append((start, end))
        start = end
    return out


# ---- binary64 -> bfloat16 --------------------------------------------------

FINITE_BF16 = np.unique(bf16_bits_to_f32(np.arange(0x7F80, dtype=np.uint16)).astype(np.float64))  # +0 .. max


def nearest_bf16(v: float) -> int:
    """Round |v| to bfloat16 by searching the sorted finite values; ties to the even pattern."""
    a = abs(v)
    hi_i = int(np.searchsorted(FINITE_BF16, a, side="left"))
    if hi_i < len(FINITE_BF16) and FINITE_BF16[hi_i] == a:
        bits = hi_i
    elif hi_i == len(FINITE_BF16):               # above the largest finite value
        mid = FINITE_BF16[-1] + (2.0 ** 128 - FINITE_BF16[-1]) / 2
        bits = 0x7F80 if a >= mid else 0x7F7F    # the tie goes to the even pattern 0x7F80 (inf)
    else:
        lo, hi = FINITE_BF16[hi_i - 1], FINITE_BF16[hi_i]
        mid = lo + (hi - lo) / 2                 # exact: lo, hi have 8 significant bits
        bits = hi_i - 1 if a < mid else (hi_i if a > mid else (hi_i - 1 if (hi_i - 1) % 2 == 0 else hi_i))
    return bits | (0x8000 if np.signbit(v) else 0)


def test_f64_rounding_matches_nearest_search_and_the_exact_helper(o):
    rng = np.random.default_rng(50)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    # exact ties, and one binary64 step either side, across the range (normal and subnormal)
    for b in rng.integers(1, 0x7F7F, 400):
        lo = float(bf16_bits_to_f32(np.uint16(b)))
        hi = float(bf16_bits_to_f32(np.uint16(b + 1)))
        mid = lo + (hi - lo) / 2
        vals += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid]
    top = float(bf16_bits_to_f32(np.uint16(0x7F7F)))
    mid_top = top + (2.0 ** 128 - top) / 2
    vals += [mid_top, np.nextafter(mid_top, 0.0), 2.0 ** -133, 2.0 ** -134, np.nextafter(2.0 ** -134, 1.0),
             3 * 2.0 ** -134, 0.0, -0.0, 1e-300, -1e-300, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40]
    got = np.array([o.f64_to_bf16(v) for v in vals], dtype=np.uint16)
    want = np.array([nearest_bf16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want), np.nonzero(got != want)[0][:5]
    assert np.array_equal(got, f64_to_bf16_exact(np.array(vals)))
    assert o.f64_to_bf16(float("inf")) == 0x7F80 and o.f64_to_bf16(float("-inf")) == 0xFF80
    assert (o.f64_to_bf16(float("nan")) & 0x7FC0) == 0x7FC0


# ---- the grouped sums -------------------------------------------------------

def int_case(rng, tokens, hidden, inter, experts, offs):
    a = rng.integers(-8, 9, (tokens, hidden))
    wg = rng.integers(-8, 9, (experts, inter, hidden))
    wu = rng.integers(-8, 9, (experts, inter, hidden))
    return a, wg, wu, np.asarray(offs, dtype=np.int32)


@pytest.mark.parametrize("offs", [[3, 3, 9, 14], [0, 14, 14, 14], [5, 2, 20, 14], [-4, 6, 9, 11], [14, 0, 0, 0]])
def test_integer_products_per_expert_are_exact(offs, o):
    """Small integers make every sum exact in any order: the oracle must equal numpy's
    int64 products of each expert's rows with that expert's weights, and leave rows
    of no expert untouched."""
    rng = np.random.default_rng(51)
    tokens, hidden, inter, experts = 14, 24, 5, 4
    a, wg, wu, offs = int_case(rng, tokens, hidden, inter, experts, offs)
    s, s_abs = o.grouped_gate_up(bf16_bits(a), bf16_bits(wg), bf16_bits(wu), offs, tokens, hidden, inter, experts,
                                 with_abs_sum=True)
    covered = np.zeros(tokens, bool)
    for e, (lo, hi) in enumerate(ranges(offs, tokens)):
        covered[lo:hi] = True
        want = np.concatenate([a[lo:hi] @ wg[e].T, a[lo:hi] @ wu[e].T], axis=1)
        assert np.array_equal(s[lo:hi], want.astype(np.float64))
        want_abs = np.concatenate([np.abs(a[lo:hi]) @ np.abs(wg[e]).T, np.abs(a[lo:hi]) @ np.abs(wu[e]).T], axis=1)
        assert np.array_equal(s_abs[lo:hi], want_abs.astype(np.float64))
    assert np.isnan(s[~covered]).all()


def test_float64_matmul_on_normal_data(o):
    rng = np.random.default_rng(52)
    tokens, hidden, inter, experts = 40, 256, 24, 3
    offs = np.array([11, 11, 40], np.int32)
    a = f64_to_bf16_exact(rng.standard_normal((tokens, hidden)))
    wg = f64_to_bf16_exact(rng.standard_normal((experts, inter, hidden)) * 0.06)
    wu = f64_to_bf16_exact(rng.standard_normal((experts, inter, hidden)) * 0.06)
    s, s_abs = o.grouped_gate_up(a, wg, wu, offs, tokens, hidden, inter, experts, with_abs_sum=True)
    A = bf16_bits_to_f32(a).astype(np.float64)
    for e, (lo, hi) in enumerate(ranges(offs, tokens)):
        Wg, Wu = bf16_bits_to_f32(wg[e]).astype(np.float64), bf16_bits_to_f32(wu[e]).astype(np.float64)
        want = np.concatenate([A[lo:hi] @ Wg.T, A[lo:hi] @ Wu.T], axis=1)
        assert np.all(np.abs(s[lo:hi] - want) <= 1e-13 * s_abs[lo:hi])


def test_tiny_case_exact_rational_sums_and_rounding(o):
    """5 tokens, 3 experts (one empty), hidden 3, inter 2, values with many significant bits:
    the oracle's bfloat16 output equals the exact rational sum rounded to nearest even."""
    rng = np.random.default_rng(53)
    tokens, hidden, inter, experts = 5, 3, 2, 3
    offs = np.array([2, 2, 5], np.int32)
    a = f64_to_bf16_exact(rng.standard_normal((tokens, hidden)) * 3)
    wg = f64_to_bf16_exact(rng.standard_normal((experts, inter, hidden)))
    wu = f64_to_bf16_exact(rng.standard_normal((experts, inter, hidden)))
    probs = np.array([0.5, 1.0, 0.25, 0.75, 1.5], np.float32)
    y, x = o.grouped_swiglu_fwd(a, wg, wu, offs, probs, tokens, hidden, inter, experts, 10.0)
    fa = [[Fraction(float(v)) for v in row] for row in bf16_bits_to_f32(a)]
    for e, (lo, hi) in enumerate(ranges(offs, tokens)):
        for t in range(lo, hi):
            for half, w in enumerate((wg, wu)):
                fw = bf16_bits_to_f32(w[e])
                for j in range(inter):
                    exact = sum(fa[t][h] * Fraction(float(fw[j, h])) for h in range(hidden))
                    # the sum of three products is exact in binary64 here: round that
                    assert Fraction(float(exact)) == exact
                    assert x[t, half * inter + j] == nearest_bf16(float(exact))


def test_per_expert_power_of_two_weights_select_the_expert(o):
    """W_e = 2**e * W_0: expert e's rows get exactly 2**e times what expert 0 would give."""
    rng = np.random.default_rng(54)
    tokens, hidden, inter, experts = 30, 64, 8, 4
    offs = np.array([7, 13, 13, 30], np.int32)
    a = f64_to_bf16_exact(rng.standard_normal((tokens, hidden)))
    w0g = rng.standard_normal((inter, hidden)) * 0.1
    w0u = rng.standard_normal((inter, hidden)) * 0.1
    wg = f64_to_bf16_exact(np.stack([w0g * 2.0 ** e for e in range(experts)]))
    wu = f64_to_bf16_exact(np.stack([w0u * 2.0 ** e for e in range(experts)]))
    s = o.grouped_gate_up(a, wg, wu, offs, tokens, hidden, inter, experts)
    base = o.grouped_gate_up(a, np.stack([wg[0]] * experts), np.stack([wu[0]] * experts), offs, tokens, hidden,
                             inter, experts)
    for e, (lo, hi) in enumerate(ranges(offs, tokens)):
        assert np.array_equal(s[lo:hi], base[lo:hi] * 2.0 ** e)


def test_forward_is_the_epilogue_of_the_rounded_sums(o):
    """x = bf16(exact sums) and y = the clamped SwiGLU forward of that x, row by row;
    rows of no expert keep their initial contents."""
    rng = np.random.default_rng(55)
    tokens, hidden, inter, experts, L = 50, 128, 16, 5, 7.0
    offs = np.array([9, 9, 31, 20, 45], np.int32)    # expert 3 empty (decreasing count); rows 45.. uncovered
    a = f64_to_bf16_exact(rng.standard_normal((tokens, hidden)))
    wg = f64_to_bf16_exact(rng.standard_normal((experts, inter, hidden)) * 0.5)
    wu = f64_to_bf16_exact(rng.standard_normal((experts, inter, hidden)) * 0.5)
    probs = rng.random(tokens, dtype=np.float32)
    y, x = o.grouped_swiglu_fwd(a, wg, wu, offs, probs, tokens, hidden, inter, experts, L)
    s = o.grouped_gate_up(a, wg, wu, offs, tokens, hidden, inter, experts)
    covered = ~np.isnan(s[:, 0])
    assert covered.sum() == 45 and not covered[45:].any()
    assert np.array_equal(x[covered], f64_to_bf16_exact(s[covered]))
    assert (x[~covered] == 0xFFFF).all() and (y[~covered] == 0xFFFF).all()
    assert np.array_equal(y[covered], o.swiglu_clamped_fwd(x[covered], probs[covered], int(covered.sum()), inter, L))
    # a clamp is reached: some gate and up values beyond the limit
    xf = bf16_bits_to_f32(x[covered])
    assert (xf[:, :inter] > L).any() and (np.abs(xf[:, inter:]) > L).any()


def test_sums_next_to_a_bf16_tie_are_rounded_once(o):
    """1 + 2^-8 is halfway between two bfloat16 values. A sum just above it must round up and
    one just below must round down; rounding it through binary32 first would land on the tie
    and round to even (down) in both cases."""
    tokens, hidden, inter, experts = 4, 3, 1, 1
    a = bf16_bits(np.ones((tokens, hidden)))
    w_rows = [[1.0, 2.0 ** -8, 2.0 ** -30], [1.0, 2.0 ** -8, -2.0 ** -30], [1.0, 2.0 ** -8, 0.0],
              [1.0, 3 * 2.0 ** -8, -2.0 ** -30]]
    for k, w in enumerate(w_rows):
        wg = bf16_bits(np.array(w).reshape(1, 1, hidden))
        y, x = o.grouped_swiglu_fwd(a, wg, wg, np.array([tokens], np.int32), np.ones(tokens, np.float32), tokens,
                                    hidden, inter, experts, 10.0)
        exact = sum(w)
        assert x[0, 0] == nearest_bf16(exact) == f64_to_bf16_exact(exact), (k, hex(x[0, 0]))
    assert nearest_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81 and nearest_bf16(1.0 + 2.0 ** -8 - 2.0 ** -30) == 0x3F80


def test_epilogue_reads_the_bf16_rounded_sums_not_the_accumulators(o):
    """On the designed inputs of tests/grouped_designed.py, every grouped sum is exact in binary32
    and not a bf16 value, and each row's probability puts, in one column, the clamped SwiGLU of
    the bf16-rounded gate and up and that of the unrounded sums on different bf16 values (both
    computed here in float64, away from any rounding midpoint). The oracle must give x = the
    bf16 roundings of the sums and, in every target column, the first of the two."""
    from tests import grouped_designed as gd
    d = gd.build()
    y, x = o.grouped_swiglu_fwd(d["a"], d["w_gate"], d["w_up"], d["offs"], d["probs"], gd.TOKENS, gd.HIDDEN,
                                gd.INTER, gd.EXPERTS, gd.LIMIT)
    assert np.array_equal(x, d["x_bits"])
    yt = y[np.arange(gd.TOKENS), d["target"]]
    assert np.array_equal(yt, d["want_bits"])
    assert (yt != d["other_bits"]).all()
    # the gate side and the up side are both exercised, with both signs of the result
    assert (d["target"] < gd.INTER // 2).any() and (d["target"] >= gd.INTER // 2).any()
    assert ((d["want_bits"] & 0x8000) != 0).any() and ((d["want_bits"] & 0x8000) == 0).any()
