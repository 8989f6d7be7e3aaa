"""The parity bars' own helpers, checked on the CPU (they decide every GPU verdict)."""
import numpy as np
import pytest

from tests.gpu_util import assert_bf16_parity, assert_f16_parity
from tests.numerics import bf16_is_nan, f16_is_nan

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_f16_is_nan_matches_numpy_on_every_pattern():
    assert np.array_equal(f16_is_nan(ALL16), np.isnan(ALL16.view(np.float16)))


def test_bf16_is_nan_matches_float32_widening_on_every_pattern():
    f32 = (ALL16.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(bf16_is_nan(ALL16), np.isnan(f32))


def f16(*v):
    return np.array(v, dtype=np.float16)


def test_f16_bar_ignores_nan_sign_and_payload():
    got = f16(np.nan, 1.0, -0.0)
    want = got.copy()
    want.view(np.uint16)[0] = 0xFE01  # a negative NaN with another payload
    assert_f16_parity(got, want, "nan")


def test_f16_bar_rejects_nan_against_a_number_and_inf():
    with pytest.raises(AssertionError, match="NaN positions"):
        assert_f16_parity(f16(np.nan), f16(np.inf), "nan vs inf")


@pytest.mark.parametrize("got,want,ok", [
    (f16(1.0), f16(np.nextafter(np.float16(1.0), np.float16(2.0))), True),    # 1 ulp
    (f16(1.0), f16(1.001953125), False),                                       # 2 ulps
    (f16(0.0), f16(-0.0), False),                                              # zero sign
    (f16(6e-8), f16(0.0), False),                                              # zero position
    (f16(-6e-8), f16(6e-8), False),                                            # across zero: 2 ulps
    (f16(np.inf), f16(65504.0), True),                                         # 1 ulp: max finite -> inf
])
def test_f16_bar_on_hand_pairs(got, want, ok):
    if ok:
        assert_f16_parity(got, want, "pair")
    else:
        with pytest.raises(AssertionError):
            assert_f16_parity(got, want, "pair")


def test_bf16_bar_exact_mode_and_zero_sign():
    one, next_one = np.uint16(0x3F80), np.uint16(0x3F81)
    assert_bf16_parity(np.array([one]), np.array([next_one]), "1 ulp")
    with pytest.raises(AssertionError):
        assert_bf16_parity(np.array([one]), np.array([next_one]), "exact", exact=True)
    with pytest.raises(AssertionError, match="sign of a zero"):
        assert_bf16_parity(np.array([0x0000], np.uint16), np.array([0x8000], np.uint16), "zero")


# ---- the down-projection bar -----------------------------------------------------

def _down_case(out_dtype):
    import oracle
    from moe_routed_expert_amd.workloads import DownWorkload
    w = DownWorkload("helper", 300, 64, 40, 3, seed=50, out_dtype="f32" if out_dtype == oracle.F32 else "bf16")
    d = w.generate()
    d["probs"][::9] = 0.0
    out = oracle.grouped_down_router_fwd(d["h"], d["w_down"], d["offs"], d["probs"], w.tokens, w.inter, w.hidden,
                                         w.experts, out_dtype=out_dtype)
    s, s_abs = oracle.grouped_gate_up(d["h"], d["w_down"], d["w_down"], d["offs"], w.tokens, w.inter, w.hidden,
                                      w.experts, with_abs_sum=True)
    return out, s[:, :w.hidden], s_abs[:, :w.hidden], d["probs"], w.inter


@pytest.mark.parametrize("f32", [True, False])
def test_down_bar_accepts_the_oracle_and_finds_its_rounding(f32):
    import oracle
    from tests.gpu_util import assert_down_router_within
    out, s, s_abs, p, k = _down_case(oracle.F32 if f32 else oracle.BF16)
    st = assert_down_router_within(out, f32, s, s_abs, p, k, "oracle")
    assert st["c_equal_to_exact_rounding"] == 1.0


def test_down_bar_rejects_one_float32_ulp():
    import oracle
    from tests.gpu_util import assert_down_router_within
    out, s, s_abs, p, k = _down_case(oracle.F32)
    bad = out.copy()
    i = np.flatnonzero((p != 0) & (np.abs(out[:, 0]) > 0))[3]
    bad[i, 0] = np.nextafter(bad[i, 0], np.float32(np.inf))
    with pytest.raises(AssertionError, match="not the router multiply"):
        assert_down_router_within(bad, True, s, s_abs, p, k, "planted")


@pytest.mark.parametrize("f32", [True, False])
def test_down_bar_rejects_a_value_off_by_a_few_bf16_ulps(f32):
    import oracle
    from tests.gpu_util import assert_down_router_within
    out, s, s_abs, p, k = _down_case(oracle.F32 if f32 else oracle.BF16)
    bad = out.copy()
    i = np.flatnonzero((p != 0) & (np.abs(s[:, 1]) > 0.5))[2]
    if f32:
        bad[i, 1] = np.float32(bad[i, 1] * np.float32(1 + 2.0 ** -5))
    else:
        bad[i, 1] = bad[i, 1] + 6                      # 6 bf16 ulps up (same sign, no binade edge near 0.5)
    with pytest.raises(AssertionError, match="not the router multiply"):
        assert_down_router_within(bad, f32, s, s_abs, p, k, "planted")


def test_down_bar_rejects_a_nonzero_output_where_the_probability_is_zero():
    import oracle
    from tests.gpu_util import assert_down_router_within
    out, s, s_abs, p, k = _down_case(oracle.F32)
    bad = out.copy()
    bad[0, 0] = 1e-30                                  # p[0] == 0
    with pytest.raises(AssertionError, match="probability is 0"):
        assert_down_router_within(bad, True, s, s_abs, p, k, "planted")
