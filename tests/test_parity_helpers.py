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
