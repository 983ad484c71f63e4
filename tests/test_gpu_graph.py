"""A whole shard step captured once in a HIP graph and replayed every step.

All step-to-step scalars (t, loss scale, beta powers, skip, the current
state set) live in the device ctrl block and every kernel argument is a fixed
pointer, so one captured step serves every later step.  Each case runs the
same steps eagerly and by replay, with the contributions refilled eagerly and
a synchronisation between replays; every replay's ctrl and the final
master/m/v/slot must equal the eager run's bit for bit, and the oracle's.
"""
import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth import workloads
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


def small(psi, n, rank, dtype=F16, steps=3, **kw):
    return Workload(name="small", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)


CASES = {
    "fused_skip_and_halve": Case(small(100_003, 3, 2, steps=5, scaler=2, contrib_scale=2.0 ** 10,
                                       loss_scale=2.0 ** 10), 2, 5,
                                 extra=(Inject(2, 1, 17_001, np.inf),)),
    "two_pass_clip": Case(small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05, steps=4), 5, 4),
    "fused_int8_rows": Case(small(64 * 1_000 + 37, 8, 7, steps=3), 7, 3, qbits=8),
    "gpt2_sized": Case(workloads.GPT2, 7, 6),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_equals_eager(name):
    import torch
    c = CASES[name]
    eager = H.DeviceRun(c, full_gather=False)
    eager.run()
    g = H.DeviceRun(c, full_gather=False)
    src = g.qrows if g.qrows is not None else g.contrib
    graph = g.step_obj.capture(src, g.gather)
    torch.cuda.synchronize()
    assert g.step_obj.ctrl_dict()["t"] == 0          # capturing ran nothing
    for s in range(1, c.steps + 1):
        g.fill(s)                                    # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        rep = g.step_obj.ctrl_dict()
        assert repr(rep) == repr(eager.reports[s - 1]), (s, rep, eager.reports[s - 1])
        g.reports.append(rep)
    for a, b, what in zip(g.fetch(), eager.fetch(), ("master", "m", "v", "slot")):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), what
    reps = H.oracle_scalars(c)
    H.assert_reports(g.reports, reps)
    exact = H.same_clips(g.reports, reps)
    if c.part[2] <= 1_000_000:
        p, m, v, slot = g.fetch()
        rp, rm, rv, rslot = H.oracle_elements(c, reps)
        H.assert_f32_close("master", p, rp, exact)
        H.assert_f32_close("m", m, rm, exact)
        H.assert_f32_close("v", v, rv, exact)
        H.assert_16bit_within_ulp("slot", slot, rslot, c.w.dtype, exact)
    H.log(f"graph {name}: {c.steps} replays equal the eager steps; skips "
          f"{[r['skip'] for r in g.reports]}")


@pytest.mark.parametrize("qbits", [0, 8])
@pytest.mark.parametrize("clip", [0.0, 0.02])
@pytest.mark.parametrize("write_slot", [True, False])
def test_graph_replay_with_quantised_gather_payload(write_slot, clip, qbits):
    """The step that writes the INT8 all-gather payload (fused, or two-pass
    with clipping; over 16-bit or INT8 contributions), captured once: a skip
    at step 2 (on the fused path zero_fused_restore_q rebuilds the payload
    inside the replay), every replay's ctrl and the final state, slot and
    payload equal to the eager run's bit for bit, the payload also to the
    oracle's."""
    import torch
    import oracle as O
    c = Case(small(100_003, 3, 2, steps=4, scaler=2, contrib_scale=2.0 ** 10,
                   loss_scale=2.0 ** 10, max_grad_norm=clip), 2, 4,
             extra=(Inject(2, 2, 30_001, np.inf),), qbits=qbits)
    eager = H.DeviceRun(c, full_gather=False, qgather=8, write_slot=write_slot)
    eager.run()
    g = H.DeviceRun(c, full_gather=False, qgather=8, write_slot=write_slot)
    src = g.qrows if g.qrows is not None else g.contrib
    graph = g.step_obj.capture(src, g.gather if write_slot else None, g.qg)
    torch.cuda.synchronize()
    assert g.step_obj.ctrl_dict()["t"] == 0
    for s in range(1, c.steps + 1):
        g.fill(s)
        graph.replay()
        torch.cuda.synchronize()
        rep = g.step_obj.ctrl_dict()
        assert repr(rep) == repr(eager.reports[s - 1]), (s, rep, eager.reports[s - 1])
        g.reports.append(rep)
    for a, b, what in zip(g.fetch(), eager.fetch(), ("master", "m", "v", "slot")):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), what
    for a, b, what in zip(g.qpayload(), eager.qpayload(), ("codes", "scales", "zeros")):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                              np.ascontiguousarray(b).view(np.uint8)), what
    reps = H.oracle_scalars(c)
    H.assert_reports(g.reports, reps)
    _, _, _, rslot = H.oracle_elements(c, reps)
    H.assert_qpayload(g.qpayload(), O.quantize(rslot, c.w.dtype, 8))
    H.log(f"graph qgather write_slot={write_slot} clip={clip} qbits={qbits}: {c.steps} replays "
          f"equal; skips {[r['skip'] for r in g.reports]}")


def _toy_ranks(scale=2.0 ** 10):
    """The toy workload's 32 ranks on this GPU, with a dynamic loss scale."""
    import torch
    import synth
    import zero_partitioned_mixed_amd as Z
    w = workloads.TOY
    dev = torch.device("cuda", 0)
    hp = Z.hparams(lr=w.lr, scaler=Z.SCALER_DYNAMIC)
    steps, contribs, parts = [], [], []
    for r in w.ranks:
        _, off, valid = Z.zero_partition(w.psi, w.nranks, r)
        p0 = torch.empty(valid, dtype=torch.float32, device=dev)
        synth.gpu_master_range(p0, w.seed, w.master_sigma, off)
        stride = (valid + 63) // 64 * 64
        steps.append(Z.ShardStep(w.nranks, stride, valid, off, F16, F16, hp,
                                 (p0, torch.zeros_like(p0), torch.zeros_like(p0)), None, scale))
        contribs.append(torch.empty((w.nranks, stride), dtype=torch.float16, device=dev))
        parts.append((off, valid))
    gather = torch.empty(w.psi, dtype=torch.float16, device=dev)
    synth.gpu_param_range(gather, w.seed, w.master_sigma, F16, 0)
    return w, Z.MultiShardStep(steps), contribs, parts, gather


@pytest.mark.parametrize("branches", [1, 4])
def test_all_ranks_graph_replay_equals_eager(branches):
    """The toy's 32 ranks (65 launches a step: 32 fused passes, one shared
    decision, 32 restore checks) captured once with MultiShardStep.capture,
    as one chain or with the ranks' launches on four parallel branches, and
    replayed: every replay's decisions and the final state and parameters
    equal the eager steps bit for bit, including a step that one rank's +inf
    makes all 32 ranks skip."""
    import torch
    import synth
    runs = []
    for mode in ("eager", "graph"):
        w, multi, contribs, parts, gather = _toy_ranks()

        def fill(s):
            for c, (off, valid) in zip(contribs, parts):
                synth.gpu_contrib_rows(c, w.seed, s, F16, w.contrib_sigma, 2.0 ** 10, 0.0, 100.0,
                                       off, valid)
            if s == 2:
                contribs[9][4, 1_000] = float("inf")

        graph = multi.capture(contribs, gather, branches=branches) if mode == "graph" else None
        torch.cuda.synchronize()
        reports = []
        for s in range(1, 5):
            fill(s)
            if graph is None:
                multi.step(contribs, gather)
            else:
                graph.replay()
            torch.cuda.synchronize()
            reports.append([st.ctrl_dict() for st in multi.steps])
        state = [np.concatenate([t.cpu().numpy() for t in st]) for st in
                 (s.current() for s in multi.steps)]
        runs.append((reports, state, gather.view(torch.int16).cpu().numpy()))
    (ra, sa, ga), (rb, sb, gb) = runs
    assert repr(ra) == repr(rb)
    assert [r[0]["skip"] for r in ra] == [0, 1, 0, 0]
    assert all(repr(r[0]) == repr(x) for r in ra for x in r)   # one decision for all ranks
    for x, y in zip(sa, sb):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ga, gb)
    H.log(f"all-ranks graph ({branches} branches): 4 replays equal the eager steps; scales "
          f"{[r[0]['loss_scale'] for r in ra]}")
