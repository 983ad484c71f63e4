"""GPU parity of the steps that also write the quantised all-gather payload
of the new parameters (zero_fused_step_qgather and its row-table and
quantised-contribution forms, with zero_fused_restore_q; and
zero_adam_step_qgather on the two-pass path).

"CMU 11-868 L18", Other memory optimizations: ZeRO++ quantises the
parameters block-wise to INT8 with a zero point for the forward all-gather.
The payload (codes, scales, zero points) must equal, bit for bit, the
oracle's quantisation of the oracle's own new 16-bit parameters; the step
itself meets the usual bars; without a 16-bit slot the gather buffer stays
untouched.  On the GPU side the payload must also equal what
zero_quantize_blocks writes from the slot after the plain step on the same
inputs.
"""
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


def small(psi, n, rank, dtype=F16, steps=3, **kw):
    return Workload(name="small", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)


DYN = dict(scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)

# name: (workload, payload bits, write the 16-bit slot, extra injections)
# Slot offsets: 75,000 (8-byte aligned slot), 66,670 (4-byte), 150,005 (odd).
CASES = {
    "f16_n8_aligned_q8": (small(200_000, 8, 3), 8, True, ()),
    "bf16_n8_aligned_q4": (small(200_000, 8, 3, dtype=BF16), 4, True, ()),
    "f16_n3_4byte_tail_q8": (small(100_003, 3, 2), 8, True, ()),
    "f16_n3_4byte_tail_q4": (small(100_003, 3, 2), 4, True, ()),
    "f16_n7_odd_offset_q8": (small(7 * 30_001, 7, 5), 8, True, ()),
    "bf16_n7_odd_offset_q4": (small(7 * 30_001, 7, 5, dtype=BF16), 4, True, ()),
    "bf16_n64_ragged_q8": (small(64 * 1_000 + 37, 64, 63, dtype=BF16), 8, True, ()),
    "f16_n8_no_slot_q8": (small(200_000, 8, 3), 8, False, ()),
    "bf16_n3_no_slot_q4": (small(100_003, 3, 1, dtype=BF16), 4, False, ()),
    "f16_one_partial_tile_q4": (small(8 * 1_501, 8, 6), 4, True, ()),
    "f16_exact_tiles_q8": (small(8 * 4 * 2048, 8, 2), 8, True, ()),
    "f16_empty_rank_q8": (small(9, 4, 3), 8, True, ()),
    # skips: the restore rewrites slot and payload from the kept master
    "f16_skip_mid_q8": (small(100_003, 3, 2, steps=4, **DYN), 8, True,
                        (Inject(2, 1, 17_001, np.inf),)),
    "f16_skip_last_q4": (small(100_003, 3, 2, steps=3, **DYN), 4, True,
                         (Inject(3, 0, 33_000, -np.inf),)),
    "f16_skip_last_no_slot_q8": (small(200_000, 8, 3, steps=3, **DYN), 8, False,
                                 (Inject(3, 7, 24_999, np.nan),)),
    "f16_skip_every_step_q8": (small(100_003, 3, 2, steps=3, **DYN), 8, True,
                               tuple(Inject(s, 0, 5, np.inf) for s in (1, 2, 3))),
    # the two-pass path (clipping on): zero_adam_step_qgather
    "bf16_twopass_clip_q8": (small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05), 8, True, ()),
    "f16_twopass_clip_odd_offset_q4": (small(7 * 30_001, 7, 5, max_grad_norm=0.01), 4, True, ()),
    "f16_twopass_no_slot_q8": (small(100_003, 3, 1, max_grad_norm=0.02), 8, False, ()),
    "f16_twopass_skip_q4": (small(100_003, 3, 2, steps=4, max_grad_norm=0.02, **DYN), 4, True,
                            (Inject(3, 1, 33_332, np.inf),)),
    "bf16_twopass_n64_no_slot_q4": (small(64 * 1_000 + 37, 64, 63, dtype=BF16,
                                          max_grad_norm=0.05), 4, False, ()),
}


@pytest.mark.parametrize("name", list(CASES))
def test_qgather_step_matches_oracle(name):
    w, bits, write_slot, extra = CASES[name]
    c = Case(w, w.ranks[0], w.steps, extra=tuple(extra))
    H.run_and_compare(c, name, qgather=bits, write_slot=write_slot)


# ZeRO++ end to end: the contributions as a row table or as INT8/INT4 blocks,
# the payload leaving the same pass.
# name: (workload, contribution bits (0: 16-bit), layout, payload bits, slot, injections)
SOURCES = {
    "rows_f16_n8_q8": (small(200_000, 8, 3), 0, "rows", 8, True, ()),
    "rows_shifted_bf16_n7_odd_offset_q4": (small(7 * 30_001, 7, 5, dtype=BF16), 0,
                                           "rows_shifted", 4, True, ()),
    "rows_f16_skip_no_slot_q8": (small(100_003, 3, 2, steps=4, **DYN), 0, "rows", 8, False,
                                 (Inject(2, 1, 17_001, np.inf),)),
    "q8_in_q8_out_f16_n8": (small(200_000, 8, 3), 8, "strided", 8, True, ()),
    "q8_in_q4_out_bf16_n3_tail": (small(100_003, 3, 2, dtype=BF16), 8, "strided", 4, True, ()),
    "q4_in_q8_out_f16_n7_odd_offset": (small(7 * 30_001, 7, 5), 4, "strided", 8, True, ()),
    "q4_in_q4_out_no_slot_bf16_n64": (small(64 * 1_000 + 37, 64, 63, dtype=BF16), 4, "strided",
                                      4, False, ()),
    "q8_in_q8_out_skip_last": (small(100_003, 3, 2, steps=3, **DYN), 8, "strided", 8, True,
                               (Inject(3, 0, 33_000, -np.inf),)),
    "q8_in_q8_out_twopass_clip": (small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05), 8,
                                  "strided", 8, True, ()),
    "rows_twopass_clip_q4": (small(100_003, 3, 1, max_grad_norm=0.02), 0, "rows", 4, True, ()),
}


@pytest.mark.parametrize("name", list(SOURCES))
def test_qgather_from_other_sources_matches_oracle(name):
    w, qbits, layout, bits, write_slot, extra = SOURCES[name]
    c = Case(w, w.ranks[0], w.steps, extra=tuple(extra), qbits=qbits)
    H.run_and_compare(c, name, layout=layout, qgather=bits, write_slot=write_slot)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("name,w,extra", [
    ("n8", small(8 * 50_001, 8, 7, steps=4, **DYN), (Inject(3, 2, 40_000, np.inf),)),
    ("n5_bf16", small(5 * 20_003, 5, 4, dtype=BF16, steps=3), ()),
    ("n8_two_pass", small(8 * 50_001, 8, 6, steps=4, max_grad_norm=0.03, **DYN),
     (Inject(2, 5, 10, np.nan),)),
])
def test_qgather_step_equals_step_then_quantize(name, w, extra, bits):
    """The payload equals the plain step followed by zero_quantize_blocks over
    the new slot, bit for bit, and the step's own results (state, slot,
    decisions) are unchanged by the fusion."""
    import torch
    import zero_partitioned_mixed_amd as Z
    c = Case(w, w.ranks[0], w.steps, extra=tuple(extra))
    H.log(f"qgather vs step+quantize {name} bits={bits}: part {c.part}")
    a = H.DeviceRun(c, full_gather=True, qgather=bits)
    a.run()
    b = H.DeviceRun(c, full_gather=True)
    b.run()
    assert repr(a.reports) == repr(b.reports)  # exact for floats, and NaN norms compare equal
    for x, y in zip(a.fetch(), b.fetch()):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)
    _, off, valid = c.part
    q = Z.QGather.alloc(valid, bits, b.gather.device)
    Z.zero_quantize_blocks(b.gather[off:], w.dtype, valid, bits, q.codes, q.blocks)
    torch.cuda.synchronize()
    got = a.qpayload()
    b.qg = q
    want = b.qpayload()
    assert np.array_equal(got[0], want[0]), "codes differ"
    assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32)), "scales differ"
    assert np.array_equal(got[2], want[2]), "zero points differ"
    H.log(f"qgather vs step+quantize {name} bits={bits}: equal, skips "
          f"{[r['skip'] for r in a.reports]}")
