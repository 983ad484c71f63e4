"""Contribution rows that live in another process, mapped through IPC.

"ZeRO: Memory Optimizations Toward Training Trillion Parameter Models" (paper
summary), 3.4 Stage 2: each rank receives the reduce-scatter's share of the
gradients it owns.  On a node, a rank can read its N slices where the other
ranks wrote them: peer memory mapped into its own address space, one pointer
per row (the *_rows calls).  With one GPU the peers are two processes on it:
a producer allocates each step's N rows (one allocation per row) and hands
them over as CUDA IPC handles (torch's tensor sharing); the test process maps
them and steps its shard from the mapped rows.  Decisions, master, m, v and
slot must meet the oracle's bars, as for rows in the test's own memory.
"""
import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth.workloads import F16, Workload

pytestmark = pytest.mark.gpu

W = Workload(name="ipc_rows", psi=8 * 200_003, nranks=8, ranks=(3,), dtype=F16, steps=3,
             scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)
CASE = Case(W, 3, 3, extra=(Inject(2, 5, 150_001, np.inf),))


def _checksum(rows):
    """Sum of the rows' 16-bit patterns (as int64), one per row."""
    import torch
    return [int(r.view(torch.int16).to(torch.int64).sum()) for r in rows]


def _check_mapped(rows, sums):
    for s, (rs, want) in enumerate(zip(rows, sums), 1):
        assert all(r.is_cuda and r.data_ptr() % 8 == 0 for r in rs)
        assert _checksum(rs) == want, f"step {s}: mapped rows differ from the producer's"


def producer(q, done, steps):
    """Allocates and fills every step's rows, sends them, and keeps them alive
    until the consumer is done."""
    import torch
    import synth
    c = CASE
    shard, off, valid = c.part
    dev = torch.device("cuda", 0)
    C = torch.empty((W.nranks, c.stride), dtype=torch.float16, device=dev)
    out = []
    for s in range(1, steps + 1):
        synth.gpu_contrib_rows(C, W.seed, s, W.dtype, W.contrib_sigma, W.contrib_scale,
                               W.outlier_p, W.outlier_mult, off, valid)
        for inj in c.injections:
            if inj.step == s:
                C[inj.k, inj.col] = inj.value
        out.append([C[k, :valid].clone() for k in range(W.nranks)])  # one allocation per row
    torch.cuda.synchronize()
    q.put((out, [_checksum(rows) for rows in out]))
    done.wait(300)


def test_fused_step_over_ipc_mapped_rows():
    import torch
    import torch.multiprocessing as mp
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ctx = mp.get_context("spawn")
    q, done = ctx.Queue(), ctx.Event()
    p = ctx.Process(target=producer, args=(q, done, CASE.steps))
    p.start()
    rows = None
    try:
        rows, sums = q.get(timeout=240)
        _, off, valid = CASE.part
        H.log(f"ipc rows: {len(rows)} steps x {len(rows[0])} rows of {valid} elements mapped from "
              f"pid {p.pid}")
        _check_mapped(rows, sums)
        g = H.DeviceRun(CASE, full_gather=True, layout="rows")
        for s in range(1, CASE.steps + 1):
            g.step_obj.step(rows[s - 1], g.gather)
            g.reports.append(g.step_obj.ctrl_dict())
        torch.cuda.synchronize()
        reps = H.oracle_scalars(CASE)
        stats = H.assert_reports(g.reports, reps)
        p_, m, v, slot = g.fetch()
        rp, rm, rv, rslot = H.oracle_elements(CASE, reps)
        stats["master"] = H.assert_f32_close("master", p_, rp)
        stats["m"] = H.assert_f32_close("m", m, rm)
        stats["v"] = H.assert_f32_close("v", v, rv)
        stats["slot"] = H.assert_16bit_within_ulp("slot", slot, rslot, W.dtype)
        assert [r["skip"] for r in g.reports] == [0, 1, 0]
        H.log(f"ipc rows: ok {stats}")
    finally:
        rows = None  # the mapped rows go before the producer frees them
        done.set()
        p.join(60)
        if p.is_alive():
            p.terminate()
            p.join(10)
    assert p.exitcode == 0
