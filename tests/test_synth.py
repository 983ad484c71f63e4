"""The seeded input generator: determinism, addressing and distributions.

The generator is shared infrastructure, not part of the method: these tests
only check that it draws what the workloads ask for (zero-mean draws of the
requested spread, a Bernoulli outlier mask of the requested rate, values
addressable element by element).
"""
import numpy as np
import pytest

from synth import workloads


def test_normal_moments_and_bounds(S):
    z = S.normal_range(0, 1, 1, 0, 0, 1 << 22)
    assert abs(z.mean()) < 3 * 1 / np.sqrt(z.size)
    assert abs(z.std() - 1.0) < 2e-3
    assert np.abs(z).max() <= 2 * np.sqrt(3)
    # four-uniform sum: excess kurtosis -1.2/4 = -0.3
    k = np.mean(z ** 4) / np.mean(z ** 2) ** 2 - 3
    assert abs(k + 0.3) < 0.02


def test_streams_are_distinct_and_deterministic(S):
    a = S.bits_range(0, 1, 1, 0, 0, 1000)
    assert np.array_equal(a, S.bits_range(0, 1, 1, 0, 0, 1000))
    for other in [(1, 1, 1, 0), (0, 2, 1, 0), (0, 1, 2, 0), (0, 1, 1, 1)]:
        b = S.bits_range(*other, 0, 1000)
        assert np.mean(a == b) < 0.01


def test_elements_are_addressable(S):
    idx = np.array([0, 1, 17, 999_999, 123_456_789_012], np.int64)
    rows = S.contrib_rows(5, 3, 4, workloads.F16, 1e-3, 2.0 ** 15, 1e-3, 100.0, 999_990, 16)
    at = S.contrib_at(5, 3, 4, workloads.F16, 1e-3, 2.0 ** 15, 1e-3, 100.0,
                      np.arange(999_990, 1_000_006))
    assert np.array_equal(rows, at)
    m = S.master_at(0, 0.02, idx)
    for j, i in enumerate(idx):
        assert m[j] == S.master_range(0, 0.02, int(i), 1)[0]
    p = S.param_range(0, 0.02, workloads.BF16, 100, 50)
    mr = S.master_range(0, 0.02, 100, 50)
    import torch
    assert np.array_equal(p, torch.from_numpy(mr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_padding_columns_are_zero(S):
    C = S.contrib_rows(0, 1, 3, workloads.F16, 1e-3, 1.0, 0.0, 100.0, 0, 50, stride=64)
    assert np.all(C[:, 50:] == 0) and np.all(C[:, :50].view(np.int16) != 0x7C00)


@pytest.mark.parametrize("dtype", [workloads.F16, workloads.BF16])
def test_contribution_spread_and_outliers(S, dtype):
    n = 1 << 20
    import torch
    C = S.contrib_rows(0, 1, 2, dtype, 1e-3, 2.0 ** 15, 1e-3, 100.0, 0, n)
    tdt = torch.float16 if dtype == workloads.F16 else torch.bfloat16
    x = torch.from_numpy(C.view(np.int16)).view(tdt).float().numpy().astype(np.float64)
    big = np.abs(x) > 4 * 1e-3 * 2.0 ** 15  # beyond the +-2 sqrt(3) sigma support: outliers only
    rate = big.mean()
    # P(outlier and |z| * 100 > 4) ~ 1e-3 * P(|z| > 0.04) ~ 0.98e-3
    assert 0.8e-3 < rate < 1.15e-3
    core = x[~big] / 2.0 ** 15
    assert abs(core.std() - 1e-3) < 2e-5


def test_workload_table():
    w = workloads.BY_NAME
    assert workloads.TOY.shard == 19_932 and workloads.TOY.bytes_per_elem == 90
    assert workloads.GPT2.shard == 15_554_976 and workloads.GPT2.bytes_per_elem == 42
    assert workloads.P1_5B.bytes_per_elem == 154 and workloads.P1_5B.stride % 64 == 0
    assert workloads.P7B.variant == "two_pass" and workloads.P7B.bytes_per_elem == 50
    assert workloads.P13B.variant == "fused" and workloads.P13B.inject_inf[0][2] == 812_500_000
    assert len(w) == 5
