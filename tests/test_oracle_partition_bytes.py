"""Pins of the oracle's partition and of the per-rank model-state byte accounting.

The partition is checked by brute force (every element owned exactly once,
contiguous chunks in rank order).  Byte counts are the sums of what the
oracle's own layouts allocate per rank, compared with the values the pages
print (tests/golden/byte_accounting.json) and with the pages' closed forms.
"""
import json
import os

import numpy as np
import pytest

from oracle import layouts

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "byte_accounting.json")


def test_partition_brute_force(O):
    for psi in range(1, 301):
        for n in range(1, 18):
            owner = np.full(psi, -1)
            shard0 = None
            prev_end = 0
            for r in range(n):
                shard, off, valid = O.partition(psi, n, r)
                shard0 = shard if shard0 is None else shard0
                assert shard == shard0 == -(-psi // n)
                assert 0 <= valid <= shard
                if valid:
                    assert off == prev_end  # contiguous, in rank order
                    assert np.all(owner[off:off + valid] == -1)
                    owner[off:off + valid] = r
                    prev_end = off + valid
                else:
                    assert off >= psi
            assert prev_end == psi and np.all(owner >= 0)


@pytest.mark.parametrize("psi,n,r,shard", [
    (637_824, 32, 31, 19_932),          # toy: 19,932 elements per shard
    (124_439_808, 8, 7, 15_554_976),    # GPT-2-sized: 15.55M
    (1_500_000_000, 64, 63, 23_437_500),  # 1.5B over 64: 23.4M
    (7_000_000_000, 8, 7, 875_000_000),
    (13_000_000_000, 8, 7, 1_625_000_000),
])
def test_partition_workload_shards(O, psi, n, r, shard):
    s, off, valid = O.partition(psi, n, r)
    assert (s, off, valid) == (shard, r * shard, shard)


def test_partition_ragged_and_empty(O):
    assert O.partition(637_825, 32, 31) == (19_933, 31 * 19_933, 637_825 - 31 * 19_933)
    assert O.partition(10, 7, 4) == (2, 8, 2)
    assert O.partition(10, 7, 5) == (2, 10, 0)
    assert O.partition(10, 7, 6) == (2, 12, 0)
    for bad in [(0, 4, 0), (10, 0, 0), (10, 4, 4), (10, 4, -1)]:
        with pytest.raises(ValueError):
            O.partition(*bad)


def test_toy_allocations_match_page_table():
    g = json.load(open(GOLDEN))
    case = g["cases"][0]
    psi, n = case["psi"], case["nranks"]
    for stage in layouts.STAGES:
        per_rank = {layouts.allocate_rank(stage, psi, n, r).nbytes for r in range(n)}
        assert len(per_rank) == 1  # every rank holds the same bytes
        measured = per_rank.pop()
        value, tol = case["values"][str(stage)]
        assert abs(measured / case["unit"] - value) <= tol, (stage, measured)


def test_toy_allocations_equal_closed_forms():
    psi, n = 637_824, 32
    expect = {0: 16 * psi, 1: 4 * psi + 12 * psi // n, 2: 2 * psi + 14 * psi // n,
              3: 16 * psi // n}
    for stage, b in expect.items():
        assert layouts.allocate_rank(stage, psi, n, 0).nbytes == b
    assert expect == {0: 10_205_184, 1: 2_790_480, 2: 1_554_696, 3: 318_912}


def test_printed_sizes_at_scale():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        for stage, (value, tol) in case["values"].items():
            b = layouts.planned_bytes(int(stage), case["psi"], case["nranks"], 0)
            assert abs(b / case["unit"] - value) <= tol, (case["cite"], stage, b)
    ratios = g["ratios"]
    for stage, value in ratios["values"].items():
        b = layouts.planned_bytes(int(stage), ratios["psi"], ratios["nranks"], 0)
        assert round(b / ratios["psi"], ratios["digits"]) == value
