"""GPU parity at the full 7B and 13B shard sizes, in the launch configuration
the benchmark times.

The oracle takes every step's global decisions (overflow, skip, norm, clip,
loss scale) over the whole shard, and the per-element results on a sample of
shard positions (both ends, the injected-overflow element and its
neighbours, and 64K random positions).  The 16-bit buffer outside the slot
is checked on its borders and on random positions.
"""
import numpy as np
import pytest

import harness as H
from harness import Case
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
    torch.cuda.empty_cache()


_REPS = {}  # the oracle's per-step decisions, per workload (shared by the layouts)


def run_fullsize(w, layout="strided", qbits=0, steps=None, samples=65_536, qgather=0):
    """qgather = 8 or 4: the step writes the quantised all-gather payload and
    no 16-bit slot (bench.py --qgather); the payload is checked on whole
    sampled blocks and the slot must stay as it was."""
    import synth
    import torch
    c = Case(w, w.ranks[0], w.steps if steps is None else steps, qbits=qbits)
    shard, off, valid = c.part
    H.log(f"{w.name}: shard {shard} at offset {off}, N={w.nranks}, {w.variant}, {c.steps} steps, "
          f"layout {layout}, qbits {qbits}, qgather {qgather}")
    g = H.DeviceRun(c, full_gather=True, layout=layout, qgather=qgather, write_slot=not qgather)
    g.run()
    key = (w.name, qbits, c.steps)
    if key not in _REPS:
        H.log(f"{w.name}: GPU steps done; oracle scalar pass over {valid} x {w.nranks} x {c.steps}"
              f" (qbits {qbits})")
        _REPS[key] = H.oracle_scalars(c)
    reps = _REPS[key]
    stats = H.assert_reports(g.reports, reps)
    H.log(f"{w.name}: scalars ok {stats}; skips {[r['skip'] for r in reps]}")
    extra = [i.col + d for i in c.injections for d in (-1, 0, 1)]
    # both sides of every boundary between the library's launches: of the pass
    # over the N rows (with the payload or not) and of the Adam pass
    import zero_partitioned_mixed_amd as Z
    for chunk in {Z.launch_tiles(w.nranks, payload=bool(qgather)) * Z.TILE,
                  Z.launch_tiles(0) * Z.TILE}:
        extra += [b + d for b in range(chunk, valid, chunk) for d in (-2049, -1, 0, 1, 2048)]
    cols = H.sample_cols(valid, samples, seed=11, extra=extra)
    exact = H.same_clips(g.reports, reps)
    p, m, v, slot = g.fetch(cols)
    rp, rm, rv, rslot = H.oracle_elements(c, reps, cols)
    stats["master"] = H.assert_f32_close("master", p, rp, exact)
    stats["m"] = H.assert_f32_close("m", m, rm, exact)
    stats["v"] = H.assert_f32_close("v", v, rv, exact)
    if qgather:
        assert np.array_equal(slot, synth.param_at(w.seed, w.master_sigma, w.dtype, cols + off)), \
            "the slot changed though the step wrote only the quantised payload"
        stats["qgather"] = check_payload_blocks(g, c, reps, qgather)
    else:
        stats["slot"] = H.assert_16bit_within_ulp("slot", slot, rslot, w.dtype, exact)
    rng = np.random.default_rng(5)
    outside = np.concatenate([np.arange(max(0, off - 4096), off),
                              np.arange(off + valid, min(w.psi, off + valid + 4096)),
                              rng.integers(0, off, 8192)]).astype(np.int64)
    assert np.array_equal(g.gather_bits(outside),
                          synth.param_at(w.seed, w.master_sigma, w.dtype, outside))
    H.log(f"{w.name}: ok {stats}")
    del g
    torch.cuda.empty_cache()


def check_payload_blocks(g, c, reps, bits, nrandom=6):
    """The first, last and injected-overflow blocks and a few random ones:
    codes and records against the oracle's quantisation of its own new
    16-bit parameters over each whole block."""
    import oracle as O
    _, _, valid = c.part
    nblk = (valid + O.QBLOCK - 1) // O.QBLOCK
    rng = np.random.default_rng(23)
    picks = {0, nblk - 1, *(i.col // O.QBLOCK for i in c.injections),
             *rng.integers(0, nblk, nrandom).tolist()}
    for b in sorted(picks):
        lo, hi = b * O.QBLOCK, min(valid, (b + 1) * O.QBLOCK)
        cols = np.arange(lo, hi, dtype=np.int64)
        _, _, _, rslot = H.oracle_elements(c, reps, cols)
        ref = O.quantize(rslot, c.w.dtype, bits)
        c0, c1 = O.qcode_bytes(lo, bits), O.qcode_bytes(hi, bits)
        codes = g.qg.codes[c0:c1].cpu().numpy()
        rec = g.qg.blocks[8 * b:8 * b + 8].cpu().numpy()
        assert np.array_equal(codes, ref.codes[:c1 - c0]), f"block {b}: codes differ"
        assert rec[:4].view(np.uint32)[0] == ref.scale.view(np.uint32)[0], f"block {b}: scale"
        assert rec[4:].view(np.int32)[0] == ref.zero[0], f"block {b}: zero point"
    return {"blocks_checked": len(picks)}


def test_psi7e9_clip_two_pass_fullsize():
    run_fullsize(workloads.P7B)


def test_psi13e9_dynamic_scale_fused_fullsize():
    run_fullsize(workloads.P13B)


def test_psi13e9_row_table_fullsize():
    """The 13B shard with its eight contribution rows in eight separate
    allocations, through zero_fused_step_rows (bench.py --rows)."""
    run_fullsize(workloads.P13B, layout="rows")


def test_psi13e9_int8_blocks_fullsize():
    """The 13B shard with INT8 block-quantised contributions, through
    zero_fused_step_q (bench.py --quant 8): its first two steps (the second
    holds the injected +inf, so its block dequantises to NaN and the step is
    skipped), decisions over the whole shard, elements on a sample with their
    whole blocks."""
    run_fullsize(workloads.P13B, qbits=8, steps=2, samples=2_000)


def test_psi13e9_int8_gather_payload_fullsize():
    """The 13B shard through zero_fused_step_qgather writing the INT8
    all-gather payload and no 16-bit slot (bench.py --qgather 8): its five
    steps, the second skipped by the injected +inf (zero_fused_restore_q then
    rebuilds the payload from the kept master), decisions over the whole
    shard, state on a sample, payload on whole sampled blocks."""
    run_fullsize(workloads.P13B, qgather=8)


# Psi = 2^32 + 12,441 over two ranks: rank 1's shard of 2^31 + 6,220 elements
# starts at 2^31 + 6,221, so its element indices, its slot's offset in the
# parameter buffer and the global indices of its inputs all pass 2^31 (the
# last ones 2^32), and it has a ragged last tile.
PSI_PAST_2_31 = (1 << 32) + 12_441
PAST_2_31 = {
    "fused": Workload(name="psi2e32_n2_dynscale", psi=PSI_PAST_2_31, nranks=2, ranks=(1,),
                      dtype=F16, steps=3, contrib_scale=2.0 ** 15, scaler=2,
                      loss_scale=2.0 ** 15, inject_inf=((2, 1, (1 << 31) + 17),)),
    "two_pass": Workload(name="psi2e32_n2_clip", psi=PSI_PAST_2_31, nranks=2, ranks=(1,),
                         dtype=BF16, steps=2, outlier_p=1e-3, max_grad_norm=1.0),
}


@pytest.mark.parametrize("variant", [*PAST_2_31, "int4_rows_int8_payload"])
def test_shard_past_2_31_elements(variant):
    """A shard longer than 2^31 elements at an offset past 2^31: the fused
    step with a dynamic scale and a +inf past element 2^31 at step 2 (skip and
    halve, then the restore), and the two-pass step with clipping, each in the
    benchmark's launch configuration (33 launches of 32,768 tiles per pass),
    against the oracle's whole-shard decisions and on 65K sampled elements;
    the parameter buffer outside the slot unchanged.  The third case takes
    the fused step's contributions as INT4 blocks and writes the INT8
    all-gather payload instead of the slot (byte and nibble offsets past
    2^30), checked on 2,000 sampled elements and whole sampled blocks."""
    w = PAST_2_31["fused" if variant == "int4_rows_int8_payload" else variant]
    _, off, valid = Case(w, 1, 1).part
    assert valid == (1 << 31) + 6_220 and off == (1 << 31) + 6_221
    if variant == "int4_rows_int8_payload":
        run_fullsize(w, qbits=4, qgather=8, samples=2_000)
    else:
        run_fullsize(w)
