"""Shard steps of several ranks enqueued on separate HIP streams at once, as a
caller that runs independent shards (or buckets) side by side would: every
call keeps its state in the caller's buffers (ctrl block, workspace, state,
slot), so the steps may overlap on the GPU in any way and must end with the
bits of the same steps run one after another.  (The allocation-free entry
point shares one array per GPU and is left out: overlapping calls of it race,
as its header says.)"""
import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth.workloads import BF16, F16, Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import synth
    synth.gpu()
    import zero_partitioned_mixed_amd  # noqa: F401
    yield


def _small(psi, n, rank, dtype=F16, steps=3, **kw):
    return Workload(name="streams", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)


DYN = dict(scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)

# (case, quantised all-gather payload bits): a fused step with a skip and a
# halving at step 2, a two-pass step with clipping, a fused step over INT8
# rows, and a fused step that writes the INT8 payload instead of the slot
CASES = [
    (Case(_small(3 * 1_000_003, 3, 2, **DYN), 2, 3, extra=(Inject(2, 1, 170_001, np.inf),)), 0),
    (Case(_small(8 * 800_000, 8, 5, dtype=BF16, max_grad_norm=0.05), 5, 3), 0),
    (Case(_small(8 * 640_037, 8, 7), 7, 3, qbits=8), 0),
    (Case(_small(4 * 700_001, 4, 1, dtype=BF16, weight_decay=0.01), 1, 3), 8),
]


def _run(c: Case, qgather: int):
    return H.DeviceRun(c, full_gather=False, qgather=qgather, write_slot=not qgather)


def _enqueue_step(g, s):
    g.fill(s)
    src = g.qrows if g.qrows is not None else g.contrib
    g.step_obj.step(src, g.gather if g.write_slot else None, g.qg)


def _result(g):
    out = [np.ascontiguousarray(x).view(np.uint8) for x in g.fetch()]
    if g.qg is not None:
        out += [np.ascontiguousarray(x).view(np.uint8) for x in g.qpayload()]
    return repr(g.step_obj.ctrl_dict()), out


def test_ranks_on_separate_streams_equal_serial_steps():
    import torch
    serial = []
    for c, qg in CASES:
        g = _run(c, qg)
        for s in range(1, c.steps + 1):
            _enqueue_step(g, s)
        torch.cuda.synchronize()
        serial.append(_result(g))
        del g
    runs = [_run(c, qg) for c, qg in CASES]
    streams = [torch.cuda.Stream() for _ in runs]
    torch.cuda.synchronize()
    for s in range(1, 4):                        # step s of every rank, each on its own stream
        for g, st in zip(runs, streams):
            with torch.cuda.stream(st):
                _enqueue_step(g, s)
    torch.cuda.synchronize()
    for i, (g, (ctrl, bits)) in enumerate(zip(runs, serial)):
        got_ctrl, got_bits = _result(g)
        assert got_ctrl == ctrl, (i, got_ctrl, ctrl)
        for k, (a, b) in enumerate(zip(got_bits, bits)):
            assert np.array_equal(a, b), (i, k)
    assert "'skip': 0" in serial[0][0]           # the last step applied, after the skip at step 2
    H.log(f"streams: {len(CASES)} ranks on separate streams equal their serial steps")
