"""GPU parity of the row-table calls (zero_fused_step_rows, zero_reduce_grads_rows).

A rank that reads the N ranks' gradient slices where they lie (each mapped
into its process) hands the library one pointer per row instead of one
[N, stride] buffer ("CMU 11-868 L18", Mechanism 1 step 3: the reduce-scatter
leaves each rank the mean over its own slice; paper summary 3.4 Stage 2).  On
one GPU the rows sit in separate allocations, or packed at 8-byte but not
16-byte aligned starts.  Each case is checked against the oracle (same bars as
the strided calls) and bit for bit against the strided call on the same rows.
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
    "f16_fused_n3_tail": (small(100_003, 3, 2), ()),
    "f16_twopass_clip_n3": (small(100_003, 3, 1, max_grad_norm=0.01), ()),
    "bf16_fused_n8": (small(200_000, 8, 3, dtype=BF16), ()),
    "bf16_twopass_clip_n8_wd": (small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05,
                                      weight_decay=0.01), ()),
    "f16_fused_n7_offset_odd": (small(69_990, 7, 5), ()),
    "bf16_fused_n64_ragged": (small(64 * 1_000 + 37, 64, 63, dtype=BF16), ()),
    "f16_fused_inf_skip": (small(100_003, 3, 2, steps=4, scaler=2, contrib_scale=2.0 ** 10,
                                 loss_scale=2.0 ** 10), (Inject(2, 1, 17_001, np.inf),)),
}


def _final(g):
    p, m, v, slot = g.fetch()
    return [a.view(np.uint32) for a in (p, m, v)] + [slot]


def _assert_same(a, b, label):
    ga, gb = _final(a), _final(b)
    for name, x, y in zip(("master", "m", "v", "slot"), ga, gb):
        assert np.array_equal(x, y), f"{label}: {name} differs from the strided call"
    for s, (ra, rb) in enumerate(zip(a.reports, b.reports), 1):
        assert ra == rb, f"{label}: ctrl after step {s} differs"


@pytest.mark.parametrize("layout", ["rows", "rows_shifted"])
@pytest.mark.parametrize("name", list(CASES))
def test_row_table_small(name, layout):
    w, extra = CASES[name]
    c = Case(w, w.ranks[0], w.steps, extra=tuple(extra))
    g, _ = H.run_and_compare(c, f"{name}/{layout}", full=True, layout=layout)
    ref = H.DeviceRun(c, full_gather=True, layout="strided")
    ref.run()
    _assert_same(g, ref, name)


def test_row_table_aliased_rows():
    """Rows may alias: table [A, B, A, C] equals the strided buffer holding
    rows A, B, A, C."""
    import torch
    import zero_partitioned_mixed_amd as Z
    w = small(4 * 9_001, 4, 1)
    c = Case(w, 1, 1)
    g = H.DeviceRun(c, full_gather=False, layout="strided")
    g.fill(1)
    dup = g.contrib.clone()
    dup[2] = dup[0]
    _, off, valid = c.part
    hp = g.step_obj.hp
    outs = []
    for table in (False, True):
        st = Z.ShardStep(w.nranks, c.stride, valid, 0, F16, F16, hp,
                         tuple(t.clone() for t in g.state0))
        gather = g.gather.clone()
        st.step([dup[0], dup[1], dup[0], dup[3]] if table else dup, gather)
        torch.cuda.synchronize()
        outs.append([t[:valid].cpu().numpy().view(np.uint32) for t in st.current()]
                    + [gather.view(torch.int16).cpu().numpy(), st.ctrl_dict()])
    for x, y in zip(outs[0][:4], outs[1][:4]):
        assert np.array_equal(x, y)
    assert outs[0][4] == outs[1][4]


def test_row_table_gpt2_sized():
    """The GPT-2-sized shard (15,554,976 elements, N = 8, fp16, 20 steps) with
    the rows in eight separate allocations: bit-identical to the strided call
    at every element and every step's decisions; oracle decisions at every
    step and oracle elements on a sample."""
    w = workloads.GPT2
    c = Case(w, w.ranks[0], w.steps)
    g = H.DeviceRun(c, full_gather=False, layout="rows")
    g.run()
    ref = H.DeviceRun(c, full_gather=False, layout="strided")
    ref.run()
    _assert_same(g, ref, "gpt2 rows")
    reps = H.oracle_scalars(c)
    H.assert_reports(g.reports, reps)
    exact = H.same_clips(g.reports, reps)
    cols = H.sample_cols(c.part[2], 20_000, seed=11)
    p, m, v, slot = g.fetch(cols)
    rp, rm, rv, rslot = H.oracle_elements(c, reps, cols)
    H.assert_f32_close("master", p, rp, exact)
    H.assert_f32_close("m", m, rm, exact)
    H.assert_f32_close("v", v, rv, exact)
    H.assert_16bit_within_ulp("slot", slot, rslot, w.dtype, exact)
    H.log(f"gpt2 rows: ok, norm {g.reports[-1]['norm']:.9g}")
