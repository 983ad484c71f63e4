"""Contribution rows that live in another process, mapped through IPC.

"ZeRO: Memory Optimizations Toward Training Trillion Parameter Models" (paper
summary), 3.4 Stage 2: each rank receives the reduce-scatter's share of the
gradients it owns.  On a node, a rank can read its N slices where the other
ranks wrote them: peer memory mapped into its own address space, one pointer
per row (the *_rows calls).  With one GPU the peers are two processes on it:
a producer allocates each step's N rows (one allocation per row) and hands
them over as CUDA IPC handles (torch's tensor sharing); the test process maps
them and steps its shard from the mapped rows: the fused step, the two-pass
step (reduce from the mapped rows, then Adam), and the fused step over rows
that the producer quantised to INT8 blocks (ZeRO++ gradient payloads).
Decisions, master, m, v and slot must meet the oracle's bars, as for rows in
the test's own memory.
"""
import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth.workloads import F16, Workload

pytestmark = pytest.mark.gpu

def _case(kind):
    clip = 0.05 if kind == "two_pass_rows" else 0.0
    w = Workload(name=f"ipc_{kind}", psi=8 * 200_003, nranks=8, ranks=(3,), dtype=F16, steps=3,
                 scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10, max_grad_norm=clip)
    return Case(w, 3, 3, extra=(Inject(2, 5, 150_001, np.inf),),
                qbits=8 if kind == "fused_int8_rows" else 0)


KINDS = ["fused_rows", "two_pass_rows", "fused_int8_rows"]


def _checksum(rows):
    """Sum of the rows' bytes (as int64), one per tensor."""
    import torch
    return [int(r.view(torch.uint8).to(torch.int64).sum()) for r in rows]


def _flat(rows):
    """Every tensor of a step's rows: the 16-bit rows, or codes then records."""
    return [t for r in rows for t in (r if isinstance(r, tuple) else (r,))]


def _check_mapped(rows, sums):
    for s, (rs, want) in enumerate(zip(rows, sums), 1):
        ts = _flat(rs)
        assert all(t.is_cuda and t.data_ptr() % 8 == 0 for t in ts)
        assert _checksum(ts) == want, f"step {s}: mapped rows differ from the producer's"


def producer(q, done, kind):
    """Allocates and fills every step's rows (16-bit, or quantised on the
    device to INT8 codes and block records), sends them, and keeps them alive
    until the consumer is done."""
    import torch
    import synth
    import zero_partitioned_mixed_amd as Z
    c = _case(kind)
    w = c.w
    shard, off, valid = c.part
    dev = torch.device("cuda", 0)
    C = torch.empty((w.nranks, c.stride), dtype=torch.float16, device=dev)
    out = []
    for s in range(1, c.steps + 1):
        synth.gpu_contrib_rows(C, w.seed, s, w.dtype, w.contrib_sigma, w.contrib_scale,
                               w.outlier_p, w.outlier_mult, off, valid)
        for inj in c.injections:
            if inj.step == s:
                C[inj.k, inj.col] = inj.value
        if c.qbits:  # one code and one record allocation per row
            q8 = Z.QuantRows.alloc(w.nranks, valid, c.qbits, dev)
            for k, (codes, blocks) in enumerate(q8.rows):
                Z.zero_quantize_blocks(C[k], w.dtype, valid, c.qbits, codes, blocks)
            out.append(list(q8.rows))
        else:  # one allocation per row
            out.append([C[k, :valid].clone() for k in range(w.nranks)])
    torch.cuda.synchronize()
    q.put((out, [_checksum(_flat(rows)) for rows in out]))
    done.wait(300)


@pytest.mark.parametrize("kind", KINDS)
def test_step_over_ipc_mapped_rows(kind):
    import torch
    import torch.multiprocessing as mp
    import zero_partitioned_mixed_amd as Z
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    case = _case(kind)
    ctx = mp.get_context("spawn")
    q, done = ctx.Queue(), ctx.Event()
    p = ctx.Process(target=producer, args=(q, done, kind))
    p.start()
    rows = None
    try:
        rows, sums = q.get(timeout=240)
        _, off, valid = case.part
        H.log(f"ipc {kind}: {len(rows)} steps x {len(rows[0])} rows of {valid} elements mapped "
              f"from pid {p.pid}")
        _check_mapped(rows, sums)
        g = H.DeviceRun(case, full_gather=True, layout="rows")
        for s in range(1, case.steps + 1):
            src = Z.QuantRows(rows[s - 1], case.qbits) if case.qbits else rows[s - 1]
            g.step_obj.step(src, g.gather)
            g.reports.append(g.step_obj.ctrl_dict())
        torch.cuda.synchronize()
        reps = H.oracle_scalars(case)
        stats = H.assert_reports(g.reports, reps)
        exact = H.same_clips(g.reports, reps)
        p_, m, v, slot = g.fetch()
        rp, rm, rv, rslot = H.oracle_elements(case, reps)
        stats["master"] = H.assert_f32_close("master", p_, rp, exact)
        stats["m"] = H.assert_f32_close("m", m, rm, exact)
        stats["v"] = H.assert_f32_close("v", v, rv, exact)
        stats["slot"] = H.assert_16bit_within_ulp("slot", slot, rslot, case.w.dtype, exact)
        assert [r["skip"] for r in g.reports] == [0, 1, 0]
        H.log(f"ipc {kind}: ok {stats}")
    finally:
        rows = src = None  # the mapped rows go before the producer frees them
        done.set()
        p.join(60)
        if p.is_alive():
            p.terminate()
            p.join(10)
    assert p.exitcode == 0
