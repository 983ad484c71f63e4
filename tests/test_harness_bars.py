"""The comparison bars of the GPU parity tests, checked on hand-made arrays
(CPU only): what passes and what fails each bar, so that a loosened bar
shows here before it can let a GPU result through."""
import numpy as np
import pytest

import harness as H
from synth.workloads import BF16, F16


def _f32(bits):
    return np.array(bits, np.uint32).view(np.float32)


def _step(x, k):
    """x moved k fp32 ulps up (x > 0)."""
    return (np.asarray(x, np.float32).view(np.uint32) + np.uint32(k)).view(np.float32)


def test_f32_equal_bits_pass():
    x = np.array([0.02, -3.5e-4, 1.25e-10, 0.0], np.float32)
    st = H.assert_f32_close("x", x.copy(), x)
    assert st["bit_exact_frac"] == 1.0 and st["max_ulps"] == 0


def test_f32_ulps_without_floor():
    """v-sized values (about 1e-10, far below the 1e-9 floor of the graded
    bar): 4 ulps pass when bits need not match, 5 fail."""
    ref = np.array([1.25e-10, 3.0e-11], np.float32)
    H.assert_f32_close("v", _step(ref, 4), ref, exact=False)
    with pytest.raises(AssertionError, match="ulps apart"):
        H.assert_f32_close("v", _step(ref, 5), ref, exact=False)
    # a several-fold error at this size is inside the floor, but not the ulp bar
    with pytest.raises(AssertionError):
        H.assert_f32_close("v", ref * 3, ref, exact=False)


def test_f32_graded_bar_above_the_floor():
    ref = np.array([1.0], np.float32)
    with pytest.raises(AssertionError, match="outside the bar"):
        H.assert_f32_close("p", ref + np.float32(2e-6), ref, exact=False)


def test_f32_exact_asks_for_equal_bits():
    ref = np.array([0.02, 0.5], np.float32)
    got = ref.copy()
    got[1] = _step(ref[1], 1)
    H.assert_f32_close("m", got, ref, exact=False)
    with pytest.raises(AssertionError, match="differ in their bits"):
        H.assert_f32_close("m", got, ref, exact=True)


def test_f32_nan_where_and_only_where_the_oracle_has_it():
    ref = _f32([0x7FC00000, 0x3F800000])
    H.assert_f32_close("p", _f32([0xFFC00000, 0x3F800000]), ref)    # any NaN sign or payload
    with pytest.raises(AssertionError, match="one side only"):
        H.assert_f32_close("p", _f32([0x3F800000, 0x3F800000]), ref)
    with pytest.raises(AssertionError, match="one side only"):
        H.assert_f32_close("p", _f32([0x7FC00000, 0x7FC00001]), ref)


@pytest.mark.parametrize("dtype,one,inf,nan,neg_nan", [(F16, 0x3C00, 0x7C00, 0x7E00, 0xFE00),
                                                      (BF16, 0x3F80, 0x7F80, 0x7FC0, 0xFFC0)])
def test_16bit_bar(dtype, one, inf, nan, neg_nan):
    ref = np.array([one, inf, nan, 0x0000], np.uint16)
    H.assert_16bit_within_ulp("slot", ref.copy(), ref, dtype)
    up = ref.copy()
    up[0] += 1
    H.assert_16bit_within_ulp("slot", up, ref, dtype, exact=False)          # 1 ulp: graded bar
    with pytest.raises(AssertionError, match="differ in their bits"):
        H.assert_16bit_within_ulp("slot", up, ref, dtype, exact=True)
    up[0] += 1
    with pytest.raises(AssertionError, match="more than 1 ulp"):
        H.assert_16bit_within_ulp("slot", up, ref, dtype, exact=False)
    # -0 and +0 share an ordinal: within the bar, though not equal bits
    z = ref.copy()
    z[3] = 0x8000
    H.assert_16bit_within_ulp("slot", z, ref, dtype, exact=False)
    # NaN of either sign matches NaN; NaN never matches inf or a number
    n = ref.copy()
    n[2] = neg_nan
    H.assert_16bit_within_ulp("slot", n, ref, dtype, exact=True)
    for other in (inf, one):
        bad = ref.copy()
        bad[2] = other
        with pytest.raises(AssertionError, match="one side only"):
            H.assert_16bit_within_ulp("slot", bad, ref, dtype)


def test_same_clips_ignores_skipped_steps():
    ref = [{"skip": 0, "clip": 0.5}, {"skip": 1, "clip": 1.0}]
    assert H.same_clips([{"skip": 0, "clip": 0.5}, {"skip": 1, "clip": 0.25}], ref)
    assert not H.same_clips([{"skip": 0, "clip": float(np.nextafter(np.float32(0.5), 1))},
                             {"skip": 1, "clip": 1.0}], ref)
