"""Shards longer than one launch of a streaming pass.

The library issues each streaming pass (reduce, fused step, Adam) as
consecutive launches of at most 2^26 elements (32,768 tiles) with its
pointers advanced per launch; a pass that reads N > 8 contribution rows
launches 2^17 / N tiles at a time (at least 2,048).  These shards cross those
boundaries, with a ragged last launch, and are checked in full against the
oracle: every step's decisions and every element of master, m, v, slot and
quantised payload.  An overflow is injected right after a boundary.
"""
import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth.workloads import BF16, F16, Workload

pytestmark = pytest.mark.gpu

CHUNK = 32768 * 2048
SHARD = CHUNK + 3 * 2048 + 77  # a second, ragged launch


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import synth
    synth.gpu()
    import zero_partitioned_mixed_amd  # noqa: F401
    yield
    torch.cuda.empty_cache()


def two_chunk(dtype=F16, steps=3, **kw):
    return Workload(name="two_chunk", psi=2 * SHARD, nranks=2, ranks=(1,), dtype=dtype,
                    steps=steps, **kw)


DYN = dict(scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)

# name: (case, payload bits, 16-bit slot, contribution layout)
CASES = {
    "fused_skip_after_boundary": (Case(two_chunk(**DYN), 1, 3,
                                       extra=(Inject(2, 1, CHUNK + 5, np.inf),)), 0, True,
                                  "strided"),
    "two_pass_clip": (Case(two_chunk(dtype=BF16, max_grad_norm=0.5), 1, 3), 0, True, "strided"),
    "fused_int8_payload_no_slot": (Case(two_chunk(**DYN), 1, 3,
                                        extra=(Inject(2, 0, CHUNK + 2048, np.inf),)), 8, False,
                                   "strided"),
    "fused_int4_payload": (Case(two_chunk(steps=2), 1, 2), 4, True, "strided"),
    "two_pass_int4_payload": (Case(two_chunk(dtype=BF16, max_grad_norm=0.5), 1, 2), 4, True,
                              "strided"),
    "fused_int8_contributions": (Case(two_chunk(steps=2), 1, 2, qbits=8), 0, True, "strided"),
    "fused_int4_contributions": (Case(two_chunk(steps=2), 1, 2, qbits=4), 0, True, "strided"),
    "two_pass_int8_contributions": (Case(two_chunk(dtype=BF16, max_grad_norm=0.5, steps=2), 1, 2,
                                         qbits=8), 0, True, "strided"),
    "fused_row_table": (Case(two_chunk(steps=2), 1, 2), 0, True, "rows"),
    "two_pass_row_table_shifted": (Case(two_chunk(dtype=BF16, max_grad_norm=0.5, steps=2), 1, 2),
                                   0, True, "rows_shifted"),
    "fused_int8_contributions_int4_payload": (Case(two_chunk(steps=2), 1, 2, qbits=8), 4, True,
                                              "strided"),
    "fused_row_table_int8_payload_skip": (Case(two_chunk(**DYN), 1, 3,
                                               extra=(Inject(2, 1, CHUNK + 5, np.inf),)), 8,
                                          False, "rows"),
}


T64, T24 = 2048 * 2048, 5461 * 2048  # elements per launch over 64 and over 24 rows


def many_rows(n, shard, dtype=BF16, steps=2, **kw):
    return Workload(name=f"n{n}_launches", psi=n * shard, nranks=n, ranks=(n - 1,), dtype=dtype,
                    steps=steps, **kw)


# name: (case, payload bits, 16-bit slot, layout, expected launches of the row pass)
MANY_ROWS = {
    "n64_fused_three_launches_skip": (
        Case(many_rows(64, 2 * T64 + 2048 + 77, dtype=F16, steps=3, **DYN), 63, 3,
             extra=(Inject(2, 40, T64 + 3, np.inf),)), 0, True, "strided", 3),
    "n64_two_pass_clip": (Case(many_rows(64, T64 + 4099, max_grad_norm=0.5), 63, 2), 0, True,
                          "strided", 2),
    "n64_two_pass_int4_rows_int8_payload": (Case(many_rows(64, T64 + 2048 * 3 + 9,
                                                           max_grad_norm=0.5), 63, 2, qbits=4), 8,
                                            False, "strided", 2),
    "n24_fused_int8_rows_int4_payload": (Case(many_rows(24, T24 + 2048 + 5), 23, 2, qbits=8), 4,
                                         True, "strided", 2),
    "n24_fused_row_table": (Case(many_rows(24, 2 * T24 + 1, dtype=F16), 23, 2), 0, True, "rows",
                            3),
}


@pytest.mark.parametrize("name", list(MANY_ROWS))
def test_many_rows_over_several_launches(name):
    import zero_partitioned_mixed_amd as Z
    c, qbits, slot, layout, nlaunch = MANY_ROWS[name]
    assert Z.launches(c.part[2], c.w.nranks) == nlaunch
    H.run_and_compare(c, name, layout=layout, qgather=qbits, write_slot=slot)


@pytest.mark.parametrize("name", list(CASES))
def test_shard_over_two_launches(name):
    c, qbits, slot, layout = CASES[name]
    assert c.part[2] == SHARD
    H.run_and_compare(c, name, layout=layout, qgather=qbits, write_slot=slot)
