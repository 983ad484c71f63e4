"""Seeded random cases of the whole shard step, GPU against the oracle.

Each seed draws one configuration from the space the C ABI accepts: Psi, N,
the rank (so every slot alignment class and ragged or empty tails occur),
the 16-bit format, the path (fused, or two-pass with a clip threshold that
may or may not bind), the loss scaler, the contribution hand-over (one
buffer, a row table, rows at 8-byte-aligned starts, INT8 or INT4 blocks), the
step count, the weight decay, outliers, and sometimes an inf or NaN in one
contribution.  A second draw per seed (its own generator, so the first draw
stays as it was) adds the quantised all-gather payload (INT8 or INT4, with
or without the 16-bit slot), bucketed steps (pieces of a few tiles) and the
slot's 16-bit format (the other one in about a quarter of the cases).  The
bars are those of the fixed cases.  The data come from the seeded input
generator as always.
"""
from dataclasses import replace

import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth.workloads import BF16, F16, Workload

pytestmark = pytest.mark.gpu

SEEDS = list(range(1, 257))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import synth
    synth.gpu()
    import zero_partitioned_mixed_amd  # noqa: F401
    yield


def draw(seed: int):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.choice([1, 2, 3, 5, 7, 8, 8, 8, 12, 16, 31, 64]))
    psi = int(rng.integers(n, 400_000))
    rank = int(rng.integers(0, n))
    dtype = int(rng.choice([F16, BF16]))
    steps = int(rng.integers(1, 5))
    two_pass = bool(rng.random() < 0.4)
    scaler = int(rng.choice([0, 1, 2])) if dtype == F16 else 0
    scale = float(2.0 ** int(rng.integers(4, 14))) if scaler else 1.0
    kw = dict(contrib_scale=scale, loss_scale=scale, scaler=scaler, min_scale=1.0,
              growth_interval=int(rng.integers(1, 4)),
              weight_decay=float(rng.choice([0.0, 0.01])),
              outlier_p=float(rng.choice([0.0, 1e-3])),
              lr=float(rng.choice([1e-3, 3e-4])))
    if two_pass:
        kw["max_grad_norm"] = float(rng.choice([1e-3, 0.05, 10.0]))
    w = Workload(name=f"random{seed}", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps,
                 seed=seed, **kw)
    qbits = int(rng.choice([0, 0, 0, 8, 4]))
    layout = "strided" if qbits else str(rng.choice(["strided", "rows", "rows_shifted"]))
    extra = ()
    _, _, valid = Case(w, rank, steps).part
    if valid and rng.random() < 0.3:
        bad = float(rng.choice([np.inf, -np.inf, np.nan]))
        extra = (Inject(int(rng.integers(1, steps + 1)), int(rng.integers(0, n)),
                        int(rng.integers(0, valid)), bad),)
    return Case(w, rank, steps, extra=extra, qbits=qbits), layout


def draw_options(seed: int, c: Case, layout: str):
    """(payload bits, write the 16-bit slot, bucket elements, slot format) for
    a case; the slot format is the other 16-bit format for about one case in
    four."""
    rng = np.random.default_rng(5000 + seed)
    qgather = int(rng.choice([0, 0, 0, 8, 4]))
    write_slot = not qgather or bool(rng.random() < 0.5)
    bucket = int(rng.choice([0, 0, 0, 1, 2, 5])) * 2048
    other = BF16 if c.w.dtype == F16 else F16
    gather_dtype = other if rng.random() < 0.25 else c.w.dtype
    return qgather, write_slot, bucket, gather_dtype


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(seed):
    c, layout = draw(seed)
    qgather, write_slot, bucket, gather_dtype = draw_options(seed, c, layout)
    c = replace(c, w=replace(c.w, gather_dtype=gather_dtype))
    H.run_and_compare(c, f"random{seed}", full=True, layout=layout, qgather=qgather,
                      write_slot=write_slot, bucket=bucket)
