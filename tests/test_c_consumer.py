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
Then all three ranks at once through the batched calls, on the fused path
(an +inf in rank 1's rows at step 2 skips every rank) and on the two-pass
path, against the oracle's step over the three ranks with shared decisions.
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
    assert [x["skip"] for x in reports] == [0, 1, 0]  # the last case's inf block skips step 2
    for two_pass in (False, True):
        pos = _check_batched(Z, raw, pos, two_pass)
    assert pos == len(raw)


def _check_batched(Z, raw: bytes, pos: int, two_pass: bool) -> int:
    """The program's batched section against the oracle's shard step over all
    three ranks with shared decisions; returns the position after it."""
    import synth
    n, psi, steps, scale = 3, 120_007, 3, 1024.0
    parts = [O.partition(psi, n, r) for r in range(n)]
    reports = []
    for _ in range(steps):
        reports.append([Z.Ctrl.from_buffer_copy(raw[pos + 128 * r:pos + 128 * (r + 1)]).as_dict()
                        for r in range(n)])
        pos += 128 * n
    finals = []
    for _, _, valid in parts:
        finals.append([np.frombuffer(raw, np.float32, valid, pos + 4 * valid * q) for q in range(3)])
        pos += 12 * valid
    gather = np.frombuffer(raw, np.uint16, psi, pos)
    pos += 2 * psi
    hp = O.hparams(lr=1e-3, max_grad_norm=0.01 if two_pass else 0.0, scaler=1 if two_pass else 2,
                   min_scale=1.0, growth_interval=1000)
    sc = O.new_scalars(scale)
    states = [O.RankState.fresh(synth.master_range(0, 0.02, off, valid)) for _, off, valid in parts]
    ogather = synth.param_range(0, 0.02, F16, 0, psi)
    exact = True
    for s in range(1, steps + 1):
        cs = []
        for r, (_, off, valid) in enumerate(parts):
            C = synth.contrib_rows(0, s, n, F16, 1e-3, scale, 0.0, 100.0, off, valid)
            if not two_pass and r == 1 and s == 2:
                C[2, 77] = 0x7C00
            cs.append(C)
        rep = O.shard_step(cs, F16, states, [p[1] for p in parts], sc, hp, ogather, F16)
        for rr in reports[s - 1]:  # one decision, written to every rank's ctrl
            assert repr(rr) == repr(reports[s - 1][0])
            assert rr["skip"] == rep.skip and rr["nonfinite"] == rep.nonfinite and rr["t"] == sc.t
            if not rep.skip:
                assert abs(rr["norm"] - rep.norm) <= H.NORM_RTOL * rep.norm
                exact = exact and np.float32(rr["clip"]) == np.float32(rep.clip)
    for r, st in enumerate(states):
        for name, got, ref in zip(("master", "m", "v"), finals[r], (st.master, st.m, st.v)):
            H.assert_f32_close(f"batched rank{r}.{name}", got, ref, exact)
    H.assert_16bit_within_ulp("batched gather", gather, ogather, F16, exact)
    H.log(f"C program, batched {'two-pass' if two_pass else 'fused'}: matches the oracle; skips "
          f"{[x[0]['skip'] for x in reports]}")
    assert [x[0]["skip"] for x in reports] == ([0, 0, 0] if two_pass else [0, 1, 0])
    return pos
