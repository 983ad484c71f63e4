"""Pins of the oracle's 16-bit formats against independent library conversions.

NumPy's float16 casts and torch's bfloat16 casts both round to nearest even;
the oracle's conversions are written from the IEEE definitions.  The fp32 ->
16-bit direction is checked over every binary32 bit pattern.
"""
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

CHUNK = 1 << 24
NCHUNK = (1 << 32) // CHUNK


def test_f16_to_f32_all_patterns(O):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.to_f32(h, O.F16)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_all_patterns(O):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.to_f32(h, O.BF16)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


_local = threading.local()


def _check_chunk(O, dtype, c):
    b0 = c * CHUNK
    if not hasattr(_local, "bufs"):
        _local.bufs = (np.empty(CHUNK, np.uint32), np.empty(CHUNK, np.uint16),
                       torch.empty(CHUNK, dtype=torch.float16), torch.empty(CHUNK, dtype=torch.bfloat16))
    u32, ours, h16, b16 = _local.bufs
    np.add(np.arange(CHUNK, dtype=np.uint32), np.uint32(b0), out=u32)
    f = u32.view(np.float32)
    O.from_f32_bits_range(b0, CHUNK, dtype, out=ours)
    tgt = h16 if dtype == O.F16 else b16
    tgt.copy_(torch.from_numpy(f))
    ref = tgt.view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    bad = (ours != ref) & ~nan
    exp_mask = 0x7C00 if dtype == O.F16 else 0x7F80
    frac_mask = 0x03FF if dtype == O.F16 else 0x007F
    on = ours[nan]
    nan_ok = bool(np.all((on & exp_mask) == exp_mask) and np.all((on & frac_mask) != 0))
    return int(bad.sum()), nan_ok, (int(np.flatnonzero(bad)[0]) + b0 if bad.any() else None)


@pytest.mark.parametrize("dtype_name", ["f16", "bf16"])
def test_f32_to_16bit_every_binary32(O, dtype_name):
    """Every binary32 pattern against torch's round-to-nearest-even casts."""
    dtype = O.F16 if dtype_name == "f16" else O.BF16
    torch.set_num_threads(1)
    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(lambda c: _check_chunk(O, dtype, c), range(NCHUNK)))
    bad = sum(r[0] for r in res)
    first = next((r[2] for r in res if r[2] is not None), None)
    assert bad == 0, f"{bad} mismatches, first at bit pattern {first:#010x}"
    assert all(r[1] for r in res), "NaN inputs must give NaN"


def test_f32_to_f16_against_numpy(O):
    """NumPy's float16 cast as a second reference, on every pattern of the
    binades around the subnormal range (2^-26 .. 2^-13) and the overflow
    boundary (2^14 .. 2^17), both signs."""
    for sign in (0, 0x80000000):
        for e_lo, e_hi in ((-26, -13), (14, 17)):
            lo, hi = sign | (127 + e_lo) << 23, sign | (127 + e_hi) << 23
            f = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32).view(np.float32)
            with np.errstate(over="ignore"):
                ref = f.astype(np.float16).view(np.uint16)
            assert np.array_equal(O.from_f32_bits_range(lo, hi - lo, O.F16), ref)


@pytest.mark.parametrize("dtype_name", ["f16", "bf16"])
def test_round_trip_and_boundaries(O, dtype_name):
    dtype = O.F16 if dtype_name == "f16" else O.BF16
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.to_f32(h, dtype)
    back = O.from_f32(f, dtype)
    ok = ~np.isnan(f)
    assert np.array_equal(back[ok], h[ok])
    if dtype == O.F16:
        # 65504 is the largest half; 65520 is the tie with 65536 and rounds to inf
        vals = np.array([65504.0, 65519.996, 65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
                         3 * 2.0 ** -25], np.float32)
        assert [int(x) for x in O.from_f32(vals, dtype)] == [0x7BFF, 0x7BFF, 0x7C00, 0x0001, 0x0000,
                                                             0x0001, 0x0002]
