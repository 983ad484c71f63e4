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


def _noalloc_against_calls(c: Case, samples: int, seed: int):
    """Steps c's shard through the allocation-free call and through the three
    calls it stands for, on one set of contributions, each path with its own
    state and slot-sized parameter buffer: every step's ctrl equal bit for
    bit, and master, m, v and the slot on sampled positions (both ends, the
    launch boundaries, the injected elements and random ones).  Returns the
    reports and the sampled results of the allocation-free path."""
    import torch
    import zero_partitioned_mixed_amd as Z
    torch.cuda.empty_cache()
    w = c.w
    _, _, valid = c.part
    ref = H.DeviceRun(c, full_gather=False)
    new = H.DeviceRun(c, full_gather=False)
    new.contrib = ref.contrib  # one set of contributions for both paths
    torch.cuda.empty_cache()
    st = new.step_obj
    for s in range(1, c.steps + 1):
        ref.fill(s)
        ref.step_obj.step(ref.contrib, ref.gather)
        Z.zero_fused_step_noalloc(ref.contrib, w.dtype, w.nranks, c.stride, st.pair, valid,
                                  new.gather, w.slot_dtype, st.offset, st.hp, st.ctrl)
        a, b = ref.step_obj.ctrl_dict(), st.ctrl_dict()
        assert repr(a) == repr(b), (s, a, b)
        new.reports.append(b)
        H.log(f"noalloc {w.name} step {s}: skip {b['skip']} scale {b['loss_scale']} "
              f"norm {b['norm']:.12g}")
    chunk = Z.launch_tiles(w.nranks) * Z.TILE
    extra = [i.col + d for i in c.injections for d in (-1, 0, 1)]
    extra += [b0 + d for b0 in range(chunk, valid, chunk) for d in (-1, 0, 2048)]
    cols = H.sample_cols(valid, samples, seed=seed, extra=extra)
    got = new.fetch(cols)
    for x, y, name in zip(ref.fetch(cols), got, ("master", "m", "v", "slot")):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    reports = new.reports
    del ref, new, st
    torch.cuda.empty_cache()
    return reports, cols, got


def test_noalloc_step_at_the_13b_shard():
    """The 13B shard (1,625,000,000 elements, 793,458 partials in the
    library's array) in the launch configuration the benchmark times: two
    steps, the second skipped by the workload's +inf, through the allocation-
    free call and through the three calls it stands for, on the same
    contributions, equal bit for bit on 200K sampled positions.  Together the
    two paths hold about 150 GB."""
    from synth import workloads
    reports, _, _ = _noalloc_against_calls(Case(workloads.P13B, 7, 2), 200_000, seed=3)
    assert [r["skip"] for r in reports] == [0, 1]


def test_noalloc_step_at_its_size_limit():
    """A shard of exactly ZERO_NOALLOC_MAX_LEN = 2^31 elements (one row, fp16,
    dynamic loss scale): 2^20 tiles, so the fused pass fills the library's
    array up to its last tile partial, and the decision its 64 group slots.
    Three steps, the second skipped by a +inf in the shard's last element;
    equal to the three calls bit for bit, and to the oracle: decisions over
    the whole shard, elements on 50K sampled positions."""
    import zero_partitioned_mixed_amd as Z
    n = Z.NOALLOC_MAX_LEN
    w = Workload(name="noalloc_limit", psi=n, nranks=1, ranks=(0,), dtype=F16, steps=3,
                 inject_inf=((2, 0, n - 1),), **DYN)
    c = Case(w, 0, 3)
    assert c.part[2] == n
    reports, cols, (p, m, v, slot) = _noalloc_against_calls(c, 50_000, seed=5)
    reps = H.oracle_scalars(c)
    stats = H.assert_reports(reports, reps)
    assert [r["skip"] for r in reps] == [0, 1, 0]
    exact = H.same_clips(reports, reps)
    rp, rm, rv, rslot = H.oracle_elements(c, reps, cols)
    stats["master"] = H.assert_f32_close("master", p, rp, exact)
    stats["m"] = H.assert_f32_close("m", m, rm, exact)
    stats["v"] = H.assert_f32_close("v", v, rv, exact)
    stats["slot"] = H.assert_16bit_within_ulp("slot", slot, rslot, w.slot_dtype, exact)
    H.log(f"noalloc at 2^31 elements: ok {stats}")
