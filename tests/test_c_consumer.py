"""The C ABI from plain C: tests/c_consumer/shard_step_demo.c links
libzero_shard.so and the HIP runtime's C API only (no Python, no torch) and
drives whole shard steps; its results are checked here against the oracle.

CPU: the program's host mode (partition, size queries, argument checks).
GPU: rank 2 of Psi = 120,007 over N = 3 (fp16) on the fused path with a
dynamic loss scale and an +inf in contribution 1 at step 2 (a skip), and
rank 1 on the two-pass path with clipping at 0.01, three steps each; then
rank 0 as the first but writing only the INT8 all-gather payload, rank 2 as
the second writing the slot and an INT4 payload, and rank 1 as the first over
INT8-quantised contributions writing only the INT8 payload.  Every step's
decisions, the final master/m/v, the slot and the payload against the oracle.
"""
import os
import subprocess

import numpy as np
import pytest

import harness as H
import oracle as O
from harness import Case, Inject
from synth.workloads import F16, Workload

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_consumer", "shard_step_demo")


def _binary():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built; run __graft_entry__.build()")
    return BIN


def test_c_program_host_mode():
    r = subprocess.run([_binary(), "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "host ok"


def _cases():
    """(case, slot written, payload bits) in the program's order."""
    common = dict(psi=120_007, nranks=3, dtype=F16, steps=3, contrib_scale=1024.0,
                  loss_scale=1024.0)

    def fused(rank, qbits=0):
        return Case(Workload(name=f"c_fused_r{rank}", ranks=(rank,), scaler=2, **common), rank, 3,
                    extra=(Inject(2, 1, 123, np.inf),), qbits=qbits)

    def two_pass(rank):
        return Case(Workload(name=f"c_two_pass_r{rank}", ranks=(rank,), scaler=1,
                             max_grad_norm=0.01, **common), rank, 3)

    return [(fused(2), True, 0), (two_pass(1), True, 0), (fused(0), False, 8),
            (two_pass(2), True, 4), (fused(1, qbits=8), False, 8)]


@pytest.mark.gpu
def test_c_program_steps_match_oracle(tmp_path):
    import zero_partitioned_mixed_amd as Z
    out = tmp_path / "c_consumer.bin"
    H.log(f"running {BIN} gpu {out}")
    r = subprocess.run([_binary(), "gpu", str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = out.read_bytes()
    pos = 0
    for c, has_slot, qbits in _cases():
        valid = c.part[2]
        reports = []
        for _ in range(c.steps):
            reports.append(Z.Ctrl.from_buffer_copy(raw[pos:pos + 128]).as_dict())
            pos += 128
        arrays = []
        for _ in range(3):
            arrays.append(np.frombuffer(raw, np.float32, valid, pos))
            pos += 4 * valid
        if has_slot:
            slot = np.frombuffer(raw, np.uint16, valid, pos)
            pos += 2 * valid
        if qbits:
            nb, nblk = O.qcode_bytes(valid, qbits), (valid + O.QBLOCK - 1) // O.QBLOCK
            codes = np.frombuffer(raw, np.uint8, nb, pos)
            rec = np.frombuffer(raw, np.uint8, 8 * nblk, pos + nb)
            pos += nb + 8 * nblk
        reps = H.oracle_scalars(c)
        H.assert_reports(reports, reps)
        exact = H.same_clips(reports, reps)
        p, m, v, oslot = H.oracle_elements(c, reps)
        H.assert_f32_close("master", arrays[0], p, exact)
        H.assert_f32_close("m", arrays[1], m, exact)
        H.assert_f32_close("v", arrays[2], v, exact)
        if has_slot:
            H.assert_16bit_within_ulp("slot", slot, oslot, F16, exact)
        if qbits:
            H.assert_qpayload((codes, rec.view(np.float32)[0::2], rec.view(np.int32)[1::2]),
                              O.quantize(oslot, F16, qbits))
        H.log(f"{c.w.name}: C program matches the oracle; skips {[x['skip'] for x in reports]}")
    assert pos == len(raw)
    assert [x["skip"] for x in reports] == [0, 1, 0]  # the last case's inf block skips step 2
