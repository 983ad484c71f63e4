"""The test harness's two oracle element paths agree: the whole-shard pass
and the sampled pass (the one the full-size tests use, which for quantised
contributions rebuilds each sampled column's whole quantisation block) give
the same master, m, v and slot at the sampled columns, bit for bit.  CPU only."""
import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth.workloads import BF16, F16, Workload


def small(psi, n, rank, dtype=F16, steps=3, **kw):
    return Workload(name="small", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)


CASES = [
    Case(small(100_003, 3, 2, steps=3, scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10),
         2, 3, extra=(Inject(2, 1, 17_001, np.inf),)),
    Case(small(60_016, 4, 1, dtype=BF16, max_grad_norm=0.01), 1, 2),
    Case(small(100_003, 3, 2), 2, 2, qbits=8),
    Case(small(64 * 1_000 + 37, 8, 7, dtype=BF16), 7, 2, qbits=4),
]


@pytest.mark.parametrize("c", CASES, ids=["skip", "clip", "int8", "int4"])
def test_sampled_elements_equal_whole_shard(c):
    reps = H.oracle_scalars(c)
    full = H.oracle_elements(c, reps)
    cols = H.sample_cols(c.part[2], 500, seed=3, extra=[0, 2047, 2048, c.part[2] - 1])
    sampled = H.oracle_elements(c, reps, cols)
    for name, a, b in zip(("master", "m", "v", "slot"), full, sampled):
        assert np.array_equal(np.asarray(a)[cols].view(np.uint8), np.asarray(b).view(np.uint8)), name
