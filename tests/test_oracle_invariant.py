"""The exactness invariant of ZeRO, on the oracle.

The simulation README reports that ZeRO-0/1/2/3 train identically: the
stages change where bytes live, not the arithmetic ("zero-stages-simulation"
README, opening summary and the loss/master-weight equality table).  With a
fixed per-element operation order and an order-independent norm, the oracle's
four layouts must agree bit for bit on master, m, v and the 16-bit
parameters, on the toy workload (Psi = 637,824, N = 32).  The small hand-sized
cases follow the lecture's two walkthroughs ("CMU 11-868 L18", Mechanism 1
with K = 2 GPUs and Mechanism 2 with K = 4).
"""
import numpy as np
import pytest

from oracle import layouts
from synth import workloads


def _toy_inputs(S, psi, n, dtype, scale, steps, inject=None):
    cache = {}

    def contrib(step):
        if step not in cache:
            C = S.contrib_rows(0, step, n, dtype, 1e-3, scale, 0.0, 100.0, 0, psi)
            if inject and step in inject:
                k, i = inject[step]
                C[k, i] = 0x7C00
            cache[step] = C
        return cache[step]

    return contrib, S.master_range(0, 0.02, 0, psi)


def _compare(results):
    ref = results[0]
    for res in results[1:]:
        for a, b in zip(ref[:4], res[:4]):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b)
        for ra, rb in zip(ref[4], res[4]):
            assert ra["skip"] == rb["skip"] and ra["nonfinite"] == rb["nonfinite"]
            assert ra["sumsq"] == rb["sumsq"] or (np.isnan(ra["sumsq"]) and np.isnan(rb["sumsq"]))


def test_toy_four_layouts_identical(O, S):
    w = workloads.TOY
    contrib, master0 = _toy_inputs(S, w.psi, w.nranks, w.dtype, 1.0, w.steps)
    hp = O.hparams(lr=w.lr)
    res = [layouts.run(st, w.psi, w.nranks, w.steps, contrib, master0, hp) for st in layouts.STAGES]
    _compare(res)
    # the step really moved the weights
    assert not np.array_equal(res[0][0], master0)


def test_toy_layouts_identical_with_clipping_and_skip(O, S):
    # clipping makes the update depend on the global norm, so any grouping of
    # the norm sum would break equality; a skipped step must be skipped by all.
    psi, n = 637_824, 32
    contrib, master0 = _toy_inputs(S, psi, n, O.F16, 2.0 ** 10, 4, inject={2: (5, 400_000)})
    hp = O.hparams(max_grad_norm=1e-4, scaler=2, min_scale=1.0)
    res = [layouts.run(st, psi, n, 4, contrib, master0, hp, loss_scale=2.0 ** 10)
           for st in layouts.STAGES]
    _compare(res)
    skips = [r["skip"] for r in res[0][4]]
    clips = [r["clip"] for r in res[0][4]]
    assert skips == [0, 1, 0, 0] and all(c < 1.0 for i, c in enumerate(clips) if not skips[i])


@pytest.mark.parametrize("psi,n", [(637_825, 32), (1000, 7), (10, 7)])
def test_ragged_partitions_identical(O, S, psi, n):
    contrib, master0 = _toy_inputs(S, psi, n, O.F16, 1.0, 2)
    hp = O.hparams(max_grad_norm=0.01)
    res = [layouts.run(st, psi, n, 2, contrib, master0, hp) for st in layouts.STAGES]
    _compare(res)


def test_two_gpu_walkthrough(O):
    """K = 2: each GPU holds a full fp16 gradient; the reduce-scatter gives each
    the average of its half in fp32; each updates its half and casts it back."""
    grads_gpu0 = np.array([0.5, -1.0, 2.0, 0.25], np.float32)
    grads_gpu1 = np.array([1.5, 1.0, -2.0, 0.75], np.float32)
    C = np.stack([O.from_f32(grads_gpu0, O.F16), O.from_f32(grads_gpu1, O.F16)])
    p0 = np.array([0.1, 0.2, 0.3, 0.4], np.float32)
    hp = O.hparams(lr=0.01)
    for r, expect_g in ((0, [1.0, 0.0]), (1, [0.0, 0.5])):
        _, off, valid = O.partition(4, 2, r)
        g, _ = O.reduce(np.ascontiguousarray(C[:, off:off + valid]), O.F16, valid,
                        O.inv_scale(2, 1.0))
        assert list(g) == expect_g
    st = O.new_scalars(1.0)
    states = []
    for r in range(2):
        _, off, valid = O.partition(4, 2, r)
        states.append(O.RankState.fresh(p0[off:off + valid]))
    gather = O.from_f32(p0, O.F16)
    contribs = [np.ascontiguousarray(C[:, 0:2]), np.ascontiguousarray(C[:, 2:4])]
    O.shard_step(contribs, O.F16, states, [0, 2], st, hp, gather, O.F16)
    # first Adam step moves each weight by lr * sign(g) (g = 0 stays put)
    expect = np.array([0.1 - 0.01, 0.2, 0.3, 0.4 - 0.01], np.float64)
    got = np.concatenate([s.master for s in states])
    assert np.allclose(got, expect, rtol=0, atol=2e-8)
    assert np.array_equal(gather, O.from_f32(got, O.F16))


def test_four_gpu_segments(O, S):
    """K = 4: GPU i owns segment M_i; its update depends only on the reduced
    gradients of M_i, whatever the other segments hold."""
    psi, n = 64, 4
    C = S.contrib_rows(3, 1, n, O.F16, 1e-2, 1.0, 0.0, 100.0, 0, psi)
    C2 = C.copy()
    C2[:, 16:32] = S.contrib_rows(4, 1, n, O.F16, 1e-2, 1.0, 0.0, 100.0, 0, 16)  # change M_1 only
    p0 = S.master_range(3, 0.02, 0, psi)
    hp = O.hparams()
    outs = []
    for CC in (C, C2):
        contrib = lambda s, CC=CC: CC
        outs.append(layouts.run(2, psi, n, 1, contrib, p0, hp)[0])
    same = np.r_[0:16, 32:64]
    assert not np.array_equal(outs[0][16:32], outs[1][16:32])
    # clipping is off and no overflow, so other owners are untouched
    assert np.array_equal(outs[0][same], outs[1][same])
