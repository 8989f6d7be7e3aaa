"""Pins of the oracle's down projection with the router-weight multiply, and of
the combine of the routed rows back into tokens.

Pages: nemo_automodel.components.moe.mok_experts (routed down weights, bf16
[local_experts, hidden, expert_intermediate]); nemo_automodel.components.moe
.optimized_ops, _apply_router_weight_fp32 (expert outputs times the permuted
probabilities in fp32, cast to the output dtype; fp32 for the scatter-add
combine); nemo_automodel.components.moe.quantized_experts,
GroupedExpertsMXFP4.forward (the local experts' fp32 [tokens, hidden]
contribution from each token's top-k slots).

Anchors: numpy int64 products, exact rational sums, the exact-rounding helper
of tests/numerics.py, the (pinned) router-multiply oracle, hand-worked sums
where binary32 order matters.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as oracle_module
from oracle import BF16, F32
from tests.numerics import bf16_bits_to_f32, f64_to_bf16_exact


@pytest.fixture
def o():
    return oracle_module


def bits(v):
    f = np.asarray(v, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f32(b), f), "not exact in bf16"
    return b


def ranges(offs, tokens):
    out, start = [], 0
    for c in offs:
        end = min(max(int(c), start), tokens)
        out.append((start, end))
        start = end
    return out


# ---- down projection + router-weight multiply --------------------------------

@pytest.mark.parametrize("out_dtype", [BF16, F32])
@pytest.mark.parametrize("offs", [[4, 4, 11], [11, 3, 20], [0, 0, 7]])
def test_down_integer_products_and_power_of_two_probs(out_dtype, offs, o):
    """Integer data and power-of-two probabilities: out = bf16(exact integer sum) * p exactly,
    per expert; rows of no expert untouched."""
    rng = np.random.default_rng(60)
    tokens, inter, hidden, experts = 11, 24, 9, 3
    h = rng.integers(-8, 9, (tokens, inter))
    w = rng.integers(-8, 9, (experts, hidden, inter))
    p = np.float32(2.0) ** rng.integers(-3, 3, tokens).astype(np.float32)
    offs = np.array(offs, np.int32)
    out = o.grouped_down_router_fwd(bits(h), bits(w), offs, p, tokens, inter, hidden, experts, out_dtype=out_dtype)
    covered = np.zeros(tokens, bool)
    for e, (lo, hi) in enumerate(ranges(offs, tokens)):
        covered[lo:hi] = True
        s = (h[lo:hi] @ w[e].T).astype(np.float64)
        want = bf16_bits_to_f32(f64_to_bf16_exact(s)) * p[lo:hi, None]
        got = bf16_bits_to_f32(out[lo:hi]) if out_dtype == BF16 else out[lo:hi]
        assert np.array_equal(got, want.astype(np.float32))
    if out_dtype == BF16:
        assert (out[~covered] == 0xFFFF).all()
    else:
        assert np.isnan(out[~covered]).all()


def test_down_exact_rational_sums_then_the_router_multiply(o):
    """Values with many significant bits: out2 is the exact rational sum rounded once to bf16,
    and out is the (pinned) router-multiply oracle of out2."""
    rng = np.random.default_rng(61)
    tokens, inter, hidden, experts = 6, 16, 5, 2
    offs = np.array([2, 6], np.int32)
    h = f64_to_bf16_exact(rng.standard_normal((tokens, inter)))
    w = f64_to_bf16_exact(rng.standard_normal((experts, hidden, inter)) * 0.3)
    p = rng.random(tokens, dtype=np.float32)
    out = o.grouped_down_router_fwd(h, w, offs, p, tokens, inter, hidden, experts, out_dtype=BF16)
    hf = bf16_bits_to_f32(h)
    out2 = np.zeros((tokens, hidden), np.uint16)
    for e, (lo, hi) in enumerate(ranges(offs, tokens)):
        wf = bf16_bits_to_f32(w[e])
        for t in range(lo, hi):
            for n in range(hidden):
                exact = sum(Fraction(float(hf[t, i])) * Fraction(float(wf[n, i])) for i in range(inter))
                assert Fraction(float(exact)) == exact          # exact in binary64 here
                out2[t, n] = f64_to_bf16_exact(float(exact))
    want = o.router_weight_mul_fwd_typed(out2, BF16, p, BF16, tokens, hidden)
    assert np.array_equal(out, want)


def test_down_weights_are_rows_of_hidden(o):
    """w_down[e] is [hidden, inter]: a one-hot weight row n picks h's column i into out's column n."""
    tokens, inter, hidden, experts = 4, 8, 3, 1
    h = bits(np.arange(tokens * inter, dtype=np.float32).reshape(tokens, inter))
    w = np.zeros((experts, hidden, inter), np.float32)
    w[0, 0, 5] = w[0, 1, 0] = w[0, 2, 7] = 1.0
    out = o.grouped_down_router_fwd(h, bits(w), np.array([4], np.int32), np.ones(tokens, np.float32), tokens, inter,
                                    hidden, experts, out_dtype=F32)
    hf = bf16_bits_to_f32(h)
    assert np.array_equal(out, hf[:, [5, 0, 7]])


# ---- combine --------------------------------------------------------------------

def test_combine_adds_slots_in_ascending_order_in_binary32(o):
    eo = np.array([[1e8], [1.0], [-1e8], [3.0], [-0.0]], np.float32)
    ro = np.array([[0, 1, 2], [2, 1, 0], [1, 0, 2], [-1, 3, 7], [-1, -1, -1], [4, -1, -1]], np.int32)
    out = o.moe_combine(eo, F32, ro, 5, 6, 3, 1)[:, 0]
    # 1e8 + 1 rounds back to 1e8 in binary32, so these orders cancel to 0
    assert out[0] == 0.0 and out[1] == 0.0
    assert out[3] == 3.0                                   # absent and out-of-range slots skipped
    assert out[4] == 0.0 and not np.signbit(out[4])        # no local slot: +0
    assert out[5] == 0.0 and not np.signbit(out[5])        # +0 + (-0) is +0
    # an order-sensitive case: 2^24 + 1 + 1 in ascending order is 2^24 (each 1 is lost), reversed it is 2^24 + 2
    eo2 = np.array([[2.0 ** 24], [1.0], [1.0]], np.float32)
    fwd = o.moe_combine(eo2, F32, np.array([[0, 1, 2]], np.int32), 3, 1, 3, 1)[0, 0]
    rev = o.moe_combine(eo2, F32, np.array([[1, 2, 0]], np.int32), 3, 1, 3, 1)[0, 0]
    assert fwd == 2.0 ** 24 and rev == 2.0 ** 24 + 2


@pytest.mark.parametrize("eo_dtype", [BF16, F32])
def test_combine_integer_rows_match_numpy(eo_dtype, o):
    rng = np.random.default_rng(62)
    rows, tokens, top_k, hidden = 40, 25, 4, 12
    vals = rng.integers(-100, 101, (rows, hidden)).astype(np.float32)
    eo = bits(vals) if eo_dtype == BF16 else vals
    ro = rng.integers(-1, rows + 3, (tokens, top_k)).astype(np.int32)   # some absent, some out of range
    out = o.moe_combine(eo, eo_dtype, ro, rows, tokens, top_k, hidden)
    want = np.zeros((tokens, hidden), np.float64)
    for t in range(tokens):
        for j in range(top_k):
            r = ro[t, j]
            if 0 <= r < rows:
                want[t] += vals[r]
    assert np.array_equal(out, want.astype(np.float32))
