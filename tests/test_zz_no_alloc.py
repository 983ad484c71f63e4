"""zero_fused_step_noalloc, the step for callers that cannot allocate, through
the C ABI: its results must equal, bit for bit, those of the calls it stands
for (zero_fused_step with a workspace, zero_grad_norm_overflow for the one
rank, zero_fused_restore) on the same inputs, step by step, and meet the
oracle's bars.  Two calls in a row, the second on a smaller shard: the
array the library keeps the partials in holds the first call's contents
when the second starts."""
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
    return Workload(name="noalloc", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)


DYN = dict(scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)

# the first call on a shard of 3.2M elements (1,563 tiles, a partial last
# tile, an odd slot offset, a skip at step 2), the second on 50,003 elements
CASES = [
    Case(_small(8 * 3_200_001, 8, 5, steps=4, **DYN), 5, 4, extra=(Inject(2, 6, 1_234_567, np.inf),)),
    Case(_small(3 * 50_003, 3, 2, dtype=BF16, steps=3, weight_decay=0.01), 2, 3),
]


def _run_both(c: Case):
    import torch
    import zero_partitioned_mixed_amd as Z
    w = c.w
    ref = H.DeviceRun(c)      # zero_fused_step + zero_grad_norm_overflow + zero_fused_restore
    new = H.DeviceRun(c)      # the same buffers, stepped by zero_fused_step_noalloc
    st = new.step_obj
    for s in range(1, c.steps + 1):
        ref.fill(s)
        ref.step_obj.step(ref.contrib, ref.gather)
        new.fill(s)
        Z.zero_fused_step_noalloc(new.contrib, w.dtype, w.nranks, c.stride, st.pair, st.valid_len,
                                  new.gather, w.slot_dtype, st.offset, st.hp, st.ctrl)
        a, b = ref.step_obj.ctrl_dict(), st.ctrl_dict()
        assert repr(a) == repr(b), (s, a, b)
        ref.reports.append(a)
        new.reports.append(b)
    torch.cuda.synchronize()
    for x, y, name in zip(ref.fetch(), new.fetch(), ("master", "m", "v", "slot")):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    assert torch.equal(ref.gather.view(torch.int16), new.gather.view(torch.int16))
    return new


def test_noalloc_step_equals_the_calls_it_stands_for_twice_in_a_row():
    for i, c in enumerate(CASES):
        H.log(f"noalloc call {i + 1}: psi={c.w.psi} N={c.w.nranks} rank={c.rank} "
              f"valid={c.part[2]} offset={c.part[1]} steps={c.steps}")
        g = _run_both(c)
        reps = H.oracle_scalars(c)
        stats = H.assert_reports(g.reports, reps)
        exact = H.same_clips(g.reports, reps)
        p, m, v, slot = g.fetch()
        rp, rm, rv, rslot = H.oracle_elements(c, reps)
        stats["master"] = H.assert_f32_close("master", p, rp, exact)
        stats["m"] = H.assert_f32_close("m", m, rm, exact)
        stats["v"] = H.assert_f32_close("v", v, rv, exact)
        stats["slot"] = H.assert_16bit_within_ulp("slot", slot, rslot, c.w.slot_dtype, exact)
        H.log(f"noalloc call {i + 1}: ok, skips {[r['skip'] for r in g.reports]} {stats}")
    assert [r["skip"] for r in H.oracle_scalars(CASES[0])] == [0, 1, 0, 0]


def test_noalloc_step_at_the_13b_shard():
    """The 13B shard (1,625,000,000 elements, 793,458 partials in the
    library's array) in the launch configuration the benchmark times: two
    steps, the second skipped by the workload's +inf, through the allocation-
    free call and through the three calls it stands for, on the same
    contributions.  Every step's ctrl is equal bit for bit, and so are master,
    m, v and the slot on 200K sampled positions (both ends, the launch
    boundaries, the injected element and random ones).  Each path writes its
    own slot-sized parameter buffer; together they hold about 150 GB."""
    import torch
    import zero_partitioned_mixed_amd as Z
    from synth import workloads
    torch.cuda.empty_cache()
    w = workloads.P13B
    c = Case(w, 7, 2)
    _, _, valid = c.part
    ref = H.DeviceRun(c, full_gather=False)
    new = H.DeviceRun(c, full_gather=False)
    new.contrib = ref.contrib  # one set of contributions for both paths
    torch.cuda.empty_cache()
    st = new.step_obj
    for s in (1, 2):
        ref.fill(s)
        ref.step_obj.step(ref.contrib, ref.gather)
        Z.zero_fused_step_noalloc(ref.contrib, w.dtype, w.nranks, c.stride, st.pair, valid,
                                  new.gather, w.slot_dtype, st.offset, st.hp, st.ctrl)
        a, b = ref.step_obj.ctrl_dict(), st.ctrl_dict()
        assert repr(a) == repr(b), (s, a, b)
        H.log(f"noalloc 13B step {s}: skip {b['skip']} scale {b['loss_scale']} norm {b['norm']:.12g}")
    assert ref.step_obj.ctrl_dict()["skip"] == 1
    chunk = Z.launch_tiles(w.nranks) * Z.TILE
    extra = [i.col + d for i in c.injections for d in (-1, 0, 1)]
    extra += [b0 + d for b0 in range(chunk, valid, chunk) for d in (-1, 0, 2048)]
    cols = H.sample_cols(valid, 200_000, seed=3, extra=extra)
    for x, y, name in zip(ref.fetch(cols), new.fetch(cols), ("master", "m", "v", "slot")):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    del ref, new, st
    torch.cuda.empty_cache()
