"""Pins of the oracle's gradient reduce, overflow flag and squared norm.

Independent references: NumPy binary64 sums (exact for these sums of 16-bit
values), the recursive-summation error bound, special values, closed forms
of the norm, NumPy's binary64 norm, and order independence.
"""
import numpy as np
import pytest

rng = np.random.default_rng(1234)


def _bits(O, values, dtype):
    return O.from_f32(np.asarray(values, np.float32), dtype)


def test_single_contribution_is_scaled_copy(O):
    x = rng.normal(0, 1e-3, size=(1, 1000)).astype(np.float32)
    C = _bits(O, x, O.F16).reshape(1, -1)
    inv = O.inv_scale(1, 4.0)
    g, flag = O.reduce(C, O.F16, 1000, inv)
    ref = C.view(np.float16).astype(np.float32)[0] * np.float32(0.25)
    assert flag == 0 and np.array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n,scale", [(2, 1.0), (8, 2.0 ** 16), (32, 1.0), (64, 1.0), (8, 2.0 ** 15)])
def test_equal_contributions_average_to_value(O, n, scale):
    c = (rng.normal(0, 1e-3, 777) * scale).astype(np.float32)
    row = _bits(O, c, O.F16)
    C = np.tile(row, (n, 1))
    g, flag = O.reduce(C, O.F16, 777, O.inv_scale(n, scale))
    expect = row.view(np.float16).astype(np.float32) / np.float32(scale)
    assert flag == 0 and np.array_equal(g, expect)


@pytest.mark.parametrize("dtype_name,n", [("f16", 3), ("f16", 8), ("bf16", 7), ("bf16", 64)])
def test_reduce_within_summation_bound(O, dtype_name, n):
    # Recursive fp32 summation of n terms: |acc - exact| <= gamma_{n-1} * sum|x_k|,
    # gamma_m = m u / (1 - m u), u = 2^-24.  With inv = 1 the oracle returns acc.
    dtype = O.F16 if dtype_name == "f16" else O.BF16
    # magnitudes spread over 2^-12 .. 2^12 so that fp32 sums must round
    vals = (rng.normal(0, 1.0, size=(n, 4096)) * 2.0 ** rng.integers(-12, 13, size=(n, 4096)))
    C = _bits(O, vals.astype(np.float32), dtype).reshape(n, 4096)
    x = O.to_f32(C, dtype).astype(np.float64)
    exact = x.sum(axis=0)  # exact in binary64 for these 16-bit values
    gamma = (n - 1) * 2.0 ** -24 / (1 - (n - 1) * 2.0 ** -24)
    acc, _ = O.reduce(C, dtype, 4096, 1.0)
    err = np.abs(acc.astype(np.float64) - exact)
    assert np.all(err <= gamma * np.abs(x).sum(axis=0))
    assert np.any(err > 0)  # the sum really is rounded in fp32, not wider


def test_reduce_order_is_rank_sequential_fp32(O):
    # bf16 holds 2^24 and 1 exactly; sequential fp32 addition loses each +1
    # (2^24 + 1 ties to even 2^24), a pairwise or wider sum would not.
    C = _bits(O, [[2.0 ** 24], [1.0], [1.0], [1.0]], O.BF16).reshape(4, 1)
    g, _ = O.reduce(C, O.BF16, 1, O.inv_scale(1, 1.0))  # inv = 1: raw sum
    assert g[0] == np.float32(2.0 ** 24)
    # 1 + 1 = 2; 2 + 2^24 is exact; 2^24 + 2 + 1 ties between 2^24 + 2 (odd
    # significand) and 2^24 + 4 (even), so the order-dependent result is 2^24 + 4.
    C2 = _bits(O, [[1.0], [1.0], [2.0 ** 24], [1.0]], O.BF16).reshape(4, 1)
    g2, _ = O.reduce(C2, O.BF16, 1, O.inv_scale(1, 1.0))
    assert g2[0] == np.float32(2.0 ** 24 + 4)


@pytest.mark.parametrize("pos", [0, 500, 999])
@pytest.mark.parametrize("special", ["inf", "-inf", "nan", "inf_and_neg_inf"])
def test_overflow_flag(O, pos, special):
    vals = rng.normal(0, 1e-3, size=(4, 1000)).astype(np.float32)
    if special == "inf_and_neg_inf":
        vals[1, pos], vals[2, pos] = np.inf, -np.inf
    else:
        vals[3, pos] = {"inf": np.inf, "-inf": -np.inf, "nan": np.nan}[special]
    C = _bits(O, vals, O.F16).reshape(4, 1000)
    g, flag = O.reduce(C, O.F16, 1000, O.inv_scale(4, 1.0))
    assert flag == 1
    if special in ("nan", "inf_and_neg_inf"):
        assert np.isnan(g[pos])
    else:
        assert np.isinf(g[pos]) and np.sign(g[pos]) == (1 if special == "inf" else -1)
    assert np.all(np.isfinite(np.delete(g, pos)))


def test_overflow_in_padding_is_ignored(O):
    C = _bits(O, rng.normal(0, 1e-3, size=(4, 64)), O.F16).reshape(4, 64)
    C[2, 60] = 0x7C00  # +inf beyond the valid length 50
    g, flag = O.reduce(C, O.F16, 50, O.inv_scale(4, 1.0))
    assert flag == 0 and g.size == 50


def test_fp32_overflow_of_finite_bf16_sum(O):
    C = _bits(O, [[3.0e38], [3.0e38]], O.BF16).reshape(2, 1)
    g, flag = O.reduce(C, O.BF16, 1, O.inv_scale(2, 1.0))
    assert flag == 1 and np.isinf(g[0])


def test_all_reduce_equals_reduce_scatter_slices(O, S):
    # "CMU 11-868 L18", Try it yourself, exercise 3: all-reduce == reduce-scatter + all-gather
    psi, n = 10_000, 8
    C = S.contrib_rows(0, 1, n, O.F16, 1e-3, 1.0, 0.0, 100.0, 0, psi)
    full, _ = O.reduce(C, O.F16, psi, O.inv_scale(n, 1.0))
    parts = []
    for r in range(n):
        _, off, valid = O.partition(psi, n, r)
        g, _ = O.reduce(np.ascontiguousarray(C[:, off:off + valid]), O.F16, valid,
                        O.inv_scale(n, 1.0))
        parts.append(g)
    assert np.array_equal(np.concatenate(parts).view(np.uint32), full.view(np.uint32))


# ------------------------------------------------------------------------- norm
def test_norm_constant_vector_closed_form(O):
    for c in (1e-3, -0.37, 3.0e-20, 1.5e18):
        g = np.full(4096, c, np.float32)
        ss = O.SumSq().add(g).value()
        assert ss == float(np.float32(c)) ** 2 * 4096
        assert np.sqrt(ss) == abs(float(np.float32(c))) * 64


def test_norm_extremes_exact(O):
    tiny = np.full(1000, 2.0 ** -149, np.float32)
    assert O.SumSq().add(tiny).value() == 1000 * 2.0 ** -298
    big = np.array([np.finfo(np.float32).max] * 3, np.float32)
    assert O.SumSq().add(big).value() == 3 * float(np.finfo(np.float32).max) ** 2


def test_norm_matches_numpy_binary64(O):
    g = (rng.normal(0, 1e-3, 1_000_003) * rng.choice([1, 100], 1_000_003, p=[0.999, 0.001])).astype(np.float32)
    ours = O.SumSq().add(g).value()
    ref = float(np.linalg.norm(g.astype(np.float64))) ** 2
    assert abs(ours - ref) <= 1e-12 * ref


def test_norm_independent_of_order_and_grouping(O):
    g = rng.normal(0, 1, 100_000).astype(np.float32) * np.float32(1e-3)
    whole = O.SumSq().add(g)
    perm = O.SumSq().add(g[rng.permutation(g.size)])
    pieces = [O.SumSq().add(c) for c in np.array_split(g, 37)]
    merged = O.SumSq()
    for p in pieces[::-1]:
        merged.merge(p)
    assert whole.limbs() == perm.limbs() == merged.limbs()
    assert whole.value() == perm.value() == merged.value()


def test_norm_nonfinite(O):
    assert np.isinf(O.SumSq().add(np.array([1, np.inf, -np.inf], np.float32)).value())
    assert np.isnan(O.SumSq().add(np.array([1, np.inf, np.nan], np.float32)).value())
    assert O.SumSq().add(np.zeros(10, np.float32)).value() == 0.0
