"""Pins of the oracle's block quantisation (ZeRO++ quantised communication,
"CMU 11-868 L18", Other memory optimizations: parameters quantised block-wise
from 16 bits to INT8 with a zero point, gradients to INT8 or INT4).

The page gives neither block size nor rounding; the oracle's reading is the
affine zero-point map over 2048-element blocks whose range contains 0, with
round-half-even: PyTorch's per-tensor affine quantisation applied block by
block.  The pins: PyTorch's own quantiser on the CPU, bit for bit, and what
the definition and arithmetic fix: hand-worked examples, the error bound of
rounding to a grid, exact zero, the end points of the range, monotonicity,
exactness on grid values, block independence and size, non-finite blocks,
and the quantised reduce against the plain reduce on exactly representable
rows (including an order-sensitive case).
"""
import numpy as np
import pytest

import oracle as O

F16, BF16 = 1, 2


def bits16(x, dtype):
    return O.from_f32(np.asarray(x, np.float32), dtype)


def values(src, dtype):
    return O.to_f32(src, dtype)


def test_int4_worked_example():
    # 0, 0.5, ..., 7.5: lo = 0, hi = 7.5, S = 7.5 / 15 = 0.5 exactly, Z = 0,
    # codes 0..15; element 2j in the low nibble of byte j.
    x = np.arange(16, dtype=np.float32) * 0.5
    q = O.quantize(bits16(x, F16), F16, 4)
    assert q.codes.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert q.scale.tolist() == [0.5] and q.zero.tolist() == [0]
    assert np.array_equal(O.dequantize(q), x)


def test_int8_worked_example():
    # -1, 0, 0.5, 2: S = fl(3/255); -lo/S = 85.000... -> Z = 85; 0.5/S = 42.5 (to
    # within rounding) -> 42 (half to even) + 85 = 127; 2/S = 170 -> 255.
    q = O.quantize(bits16([-1.0, 0.0, 0.5, 2.0], F16), F16, 8)
    assert q.scale[0] == np.float32(3.0) / np.float32(255.0)
    assert q.zero.tolist() == [85]
    assert q.codes.tolist() == [0, 85, 127, 255]
    d = O.dequantize(q)
    assert d[1] == 0.0                                    # zero is exact
    assert np.all(np.abs(d - np.array([-1, 0, 0.5, 2])) <= q.scale[0] / 2 * (1 + 2 ** -20))


def _random_blocks(rng, dtype, n):
    kinds = [rng.normal(0, 1e-3, n), rng.normal(5, 1, n), -np.abs(rng.normal(0, 30, n)),
             rng.uniform(-1e4, 1e4, n), rng.normal(0, 1e-6, n),
             np.where(rng.random(n) < 0.01, rng.normal(0, 100, n), rng.normal(0, 0.01, n))]
    return [bits16(k.astype(np.float32), dtype) for k in kinds]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_error_bound_and_code_range(bits, dtype):
    rng = np.random.default_rng(bits * 10 + dtype)
    Q = (1 << bits) - 1
    for src in _random_blocks(rng, dtype, 3 * O.QBLOCK + 77):
        q = O.quantize(src, dtype, bits)
        x = values(src, dtype).astype(np.float64)
        d = O.dequantize(q).astype(np.float64)
        assert np.all((q.zero >= 0) & (q.zero <= Q))
        for b in range(q.scale.size):
            sl = slice(b * O.QBLOCK, min((b + 1) * O.QBLOCK, src.size))
            S = float(q.scale[b])
            lo, hi = min(0.0, x[sl].min()), max(0.0, x[sl].max())
            assert S >= (hi - lo) / Q * (1 - 2 ** -22)
            err = np.abs(x[sl] - d[sl])
            assert np.all(err <= S * (0.5 + 2 ** -16) + 2 ** -23 * np.abs(x[sl])), (b, err.max(), S)


@pytest.mark.parametrize("bits", [8, 4])
def test_zero_exact_endpoints_monotone(bits):
    Q = (1 << bits) - 1
    rng = np.random.default_rng(7 + bits)
    x = np.sort(rng.normal(0.3, 2.0, O.QBLOCK).astype(np.float32))
    x[100] = 0.0
    x = np.sort(x)
    src = bits16(x, BF16)
    q = O.quantize(src, BF16, bits)
    codes = _unpack(q)
    xv = values(src, BF16)
    z = int(q.zero[0])
    assert np.all(codes[xv == 0.0] == z)                 # real zero -> the zero point
    assert np.all(O.dequantize(q)[xv == 0.0] == 0.0)     # ... and back to exactly 0
    assert codes[0] == 0 and codes[-1] >= Q - 1           # lo -> 0, hi -> Q (or Q - 1)
    assert np.all(np.diff(codes.astype(int)) >= 0)        # monotone in x
    assert codes.max() <= Q


def _unpack(q):
    if q.bits == 8:
        return q.codes.astype(np.int64)[:q.length]
    lo, hi = q.codes & 15, q.codes >> 4
    return np.stack([lo, hi], 1).reshape(-1)[:q.length].astype(np.int64)


@pytest.mark.parametrize("bits,S0,Z0", [(8, 2.0 ** -10, 100), (4, 2.0 ** -3, 6)])
def test_grid_values_are_exact(bits, S0, Z0):
    Q = (1 << bits) - 1
    j = np.concatenate([np.arange(Q + 1), np.random.default_rng(1).integers(0, Q + 1, 500)])
    x = (S0 * (j - Z0)).astype(np.float32)
    q = O.quantize(bits16(x, F16), F16, bits)
    assert q.scale[0] == S0 and q.zero[0] == Z0
    assert np.array_equal(_unpack(q), j)
    assert np.array_equal(O.dequantize(q), x)


def test_one_sided_and_zero_blocks():
    Q = 255
    pos = O.quantize(bits16(np.linspace(1, 2, 300), F16), F16, 8)
    assert pos.zero[0] == 0 and _unpack(pos)[-1] == Q
    neg = O.quantize(bits16(-np.linspace(1, 2, 300), F16), F16, 8)
    assert neg.zero[0] == Q and _unpack(neg)[-1] == 0      # -2 is lo: code 0
    zer = O.quantize(np.zeros(70, np.uint16), F16, 8)
    assert zer.scale[0] == 1.0 and zer.zero[0] == 0
    assert not zer.codes.any() and not O.dequantize(zer).any()


@pytest.mark.parametrize("bits", [8, 4])
def test_blocks_are_independent_and_2048_long(bits):
    rng = np.random.default_rng(3)
    n = 2 * O.QBLOCK + 5
    x = rng.normal(0, 1, n).astype(np.float32)
    x[O.QBLOCK:2 * O.QBLOCK] *= 50          # a different range in block 1
    src = bits16(x, F16)
    whole = O.quantize(src, F16, bits)
    assert O.qblock() == 2048 and whole.scale.size == 3
    for b in range(3):
        part = O.quantize(src[b * O.QBLOCK:(b + 1) * O.QBLOCK], F16, bits)
        assert part.scale[0] == whole.scale[b] and part.zero[0] == whole.zero[b]
        assert np.array_equal(_unpack(part), _unpack(whole)[b * O.QBLOCK:(b + 1) * O.QBLOCK])
    # a block boundary one element off would mix the ranges of blocks 0 and 1
    shifted = O.quantize(src[1:O.QBLOCK + 1], F16, bits)
    assert shifted.scale[0] != whole.scale[0]


@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("bits", [8, 4])
def test_non_finite_block(bad, bits):
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, 3 * O.QBLOCK).astype(np.float32)
    x[O.QBLOCK + 17] = bad
    src = bits16(x, F16)
    q = O.quantize(src, F16, bits)
    assert np.isnan(q.scale[1]) and q.zero[1] == 0
    assert not _unpack(q)[O.QBLOCK:2 * O.QBLOCK].any()
    d = O.dequantize(q)
    assert np.all(np.isnan(d[O.QBLOCK:2 * O.QBLOCK]))
    assert np.all(np.isfinite(d[:O.QBLOCK])) and np.all(np.isfinite(d[2 * O.QBLOCK:]))
    alone = O.quantize(src[:O.QBLOCK], F16, bits)
    assert alone.scale[0] == q.scale[0]


def test_reduce_q_equals_reduce_on_grid_rows():
    """Rows whose values lie on their blocks' grids (each block holds both
    ends of its grid, so S and Z come out exact) dequantise exactly, so the
    quantised reduce must equal the plain reduce of the 16-bit rows.  Element 0
    is order-sensitive: 255*2^-10, +255*2^16, -255*2^16 sums to 0 in rank
    order (the small value is absorbed) and to 255*2^-10 last-to-first."""
    length = O.QBLOCK + 9
    rng = np.random.default_rng(9)
    grids = [(2.0 ** -10, 0), (2.0 ** 16, 0), (2.0 ** 16, 255)]   # (S, Z) per row
    rows = []
    for S0, Z0 in grids:
        j = rng.integers(0, 256, length)
        for b0 in (0, O.QBLOCK):
            j[b0 + 1], j[b0 + 2] = 0, 255
        j[0] = 255 if Z0 == 0 else 0
        rows.append((S0 * (j - Z0)).astype(np.float32))
    assert rows[0][0] == 255 * 2.0 ** -10 and rows[1][0] == -rows[2][0] == 255 * 2.0 ** 16
    C = np.stack([bits16(r, BF16) for r in rows])
    n = len(rows)
    qs = [O.quantize(C[k], BF16, 8) for k in range(n)]
    for k in range(n):
        assert np.array_equal(O.dequantize(qs[k]), values(C[k], BF16)), k
    inv = O.inv_scale(n, 1.0)
    g_ref, f_ref = O.reduce(C, BF16, length, inv)
    g, f = O.reduce_q(qs, length, inv)
    assert np.array_equal(g.view(np.uint32), g_ref.view(np.uint32)) and f == f_ref == 0
    assert g[0] == 0.0   # the small value is absorbed by the large one in rank order


def test_reduce_q_flags_non_finite_block():
    x = np.random.default_rng(2).normal(0, 1, O.QBLOCK + 3).astype(np.float32)
    clean = O.quantize(bits16(x, F16), F16, 4)
    x[O.QBLOCK + 1] = np.inf
    dirty = O.quantize(bits16(x, F16), F16, 4)
    g, f = O.reduce_q([clean, dirty], x.size, O.inv_scale(2, 1.0))
    assert f == 1 and np.all(np.isnan(g[O.QBLOCK:])) and np.all(np.isfinite(g[:O.QBLOCK]))


def test_reduce_q_flags_fp32_overflow_of_finite_rows():
    """Two finite bf16 rows of 1.5 * 2^127 each dequantise to finite values
    whose fp32 sum exceeds the largest binary32 (about 3.4e38): the sum is
    +inf and must raise the overflow flag."""
    x = np.zeros(64, np.float32)
    x[3] = np.float32(1.5 * 2.0 ** 127)
    q = O.quantize(bits16(x, BF16), BF16, 8)
    d = O.dequantize(q)
    assert np.all(np.isfinite(d)) and d[3] > 2.0 ** 127
    g, f = O.reduce_q([q, q], x.size, 1.0)
    assert f == 1 and np.isinf(g[3]) and np.all(np.isfinite(np.delete(g, 3)))


# --------------------------------------------------------------------------- against torch
def _torch_block(x32: np.ndarray, bits: int):
    """torch's per-tensor affine quantisation of one block: MinMaxObserver's
    scale and zero point (range widened to contain 0, fp32 arithmetic, zero
    point rounded half to even and clamped), quantize_per_tensor's codes
    (quint8, or quint4x2 packed two per byte) and dequantize's fp32 values."""
    import torch
    from torch.ao.quantization.observer import MinMaxObserver
    qmax = (1 << bits) - 1
    qdt = torch.quint8 if bits == 8 else torch.quint4x2
    x = torch.from_numpy(x32)
    ob = MinMaxObserver(dtype=qdt, qscheme=torch.per_tensor_affine, quant_min=0, quant_max=qmax)
    ob(x)
    scale, zp = ob.calculate_qparams()
    q = torch.quantize_per_tensor(x, float(scale), int(zp), qdt)
    return (np.float32(scale.item()), int(zp.item()), q.int_repr().numpy().astype(np.uint8),
            torch.dequantize(q).numpy())


def _torch_cases():
    rng = np.random.default_rng(41)
    for dtype in (F16, BF16):
        for kind in ("normal", "positive", "negative", "wide", "zeros_in", "few_levels"):
            for _ in range(12):
                if kind == "normal":
                    x = rng.normal(0, 10.0 ** rng.uniform(-4, 1), 2048)
                elif kind == "positive":
                    x = np.abs(rng.normal(0, 1e-2, 2048)) + 1e-3
                elif kind == "negative":
                    x = -np.abs(rng.normal(0, 1e-2, 2048)) - 1e-3
                elif kind == "wide":
                    x = rng.normal(0, 1e-3, 2048) * rng.choice([1, 100], 2048, p=[0.99, 0.01])
                elif kind == "zeros_in":
                    x = rng.normal(0, 1e-1, 2048) * (rng.random(2048) < 0.5)
                else:
                    x = rng.integers(-3, 5, 2048) * 0.25
                yield dtype, kind, bits16(x, dtype)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_matches_torch_affine_quantization(bits):
    """Each block's scale and zero point equal MinMaxObserver's, its codes (and
    INT4 packing) equal quantize_per_tensor's, and its values equal
    dequantize's, bit for bit, on 144 blocks of fp16 and bf16 data: normal
    at scales 1e-4..10, one-sided positive and negative, outliers, half
    zeros, values on a coarse grid.  torch floors the scale at fp32's
    epsilon, which these blocks' ranges all exceed."""
    checked = 0
    for dtype, kind, src in _torch_cases():
        q = O.quantize(src, dtype, bits)
        x32 = values(src, dtype)
        scale, zp, codes, deq = _torch_block(x32, bits)
        assert scale > np.finfo(np.float32).eps  # torch's floor on the scale does not bind
        assert q.scale.view(np.uint32)[0] == scale.view(np.uint32), (kind, q.scale[0], scale)
        assert int(q.zero[0]) == zp, (kind, q.zero[0], zp)
        assert np.array_equal(q.codes[:O.qcode_bytes(2048, bits)], codes), kind
        assert np.array_equal(O.dequantize(q).view(np.uint32), deq.view(np.uint32)), kind
        checked += 1
    assert checked == 144
