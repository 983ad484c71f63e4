"""GPU parity of the block-quantised (ZeRO++) calls against the oracle.

"CMU 11-868 L18", Other memory optimizations: ZeRO++ sends parameters
block-quantised to INT8 with a zero point, and the gradient reduce-scatter in
INT8 or INT4.  Codes and block parameters must match the oracle bit for bit
(floating point decides each code, so both sides take the same fp32 steps);
dequantised 16-bit values bit for bit; the shard step over quantised
contributions to the same bars as the 16-bit step.
"""
import numpy as np
import pytest

import harness as H
import oracle as O
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


def _values(length, seed):
    """Blocks of different character: small normal, offset normal, one-sided,
    wide uniform, all zero, heavy-tailed; inf, -inf and NaN in three blocks."""
    rng = np.random.default_rng(seed)
    kinds = [lambda n: rng.normal(0, 1e-3, n), lambda n: rng.normal(3, 1, n),
             lambda n: -np.abs(rng.normal(0, 20, n)), lambda n: rng.uniform(-6e4, 6e4, n),
             lambda n: np.zeros(n), lambda n: rng.standard_t(2, n)]
    x = np.empty(length, np.float64)
    for b0 in range(0, length, O.QBLOCK):
        n = min(O.QBLOCK, length - b0)
        x[b0:b0 + n] = kinds[(b0 // O.QBLOCK) % len(kinds)](n)
    for k, bad in enumerate((np.inf, -np.inf, np.nan)):
        i = (7 + 3 * k) * O.QBLOCK + 11
        if i < length:
            x[i] = bad
    return x.astype(np.float32)


def _to_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


LENGTHS = [1, 5, 2047, 2048, 2049, 13 * 2048 + 77, 100_003]


@pytest.mark.parametrize("length", LENGTHS)
@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_quantize_matches_oracle(dtype, bits, length):
    import torch
    import zero_partitioned_mixed_amd as Z
    src = O.from_f32(_values(length, seed=length + bits), dtype)
    ref = O.quantize(src, dtype, bits)
    q = Z.QuantRows.alloc(1, length, bits, torch.device("cuda", 0))
    codes, blocks = q.rows[0]
    codes.fill_(0xA5)   # canary: every code byte must be written
    Z.zero_quantize_blocks(_to_gpu(src.view(np.int16)), dtype, length, bits, codes, blocks)
    torch.cuda.synchronize()
    got_codes = codes.cpu().numpy()[:ref.codes.size]
    blk = blocks.cpu().numpy().view(np.uint8)[:8 * ref.scale.size]
    got_scale = blk.view(np.float32)[0::2]
    got_zero = blk.view(np.int32)[1::2]
    assert np.array_equal(got_codes, ref.codes), "codes differ"
    assert np.array_equal(got_scale.view(np.uint32), ref.scale.view(np.uint32)), "scales differ"
    assert np.array_equal(got_zero, ref.zero), "zero points differ"
    H.log(f"quantize dtype={dtype} bits={bits} len={length}: {ref.scale.size} blocks equal")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_dequantize_matches_oracle(dtype, bits):
    import torch
    import zero_partitioned_mixed_amd as Z
    length = 9 * 2048 + 1001
    src = O.from_f32(_values(length, seed=3), dtype)
    ref = O.quantize(src, dtype, bits)
    want = O.cast(O.dequantize(ref), dtype)
    nbytes = (ref.codes.size + 15) // 16 * 16
    codes = np.zeros(nbytes, np.uint8)
    codes[:ref.codes.size] = ref.codes
    blocks = np.empty(2 * ref.scale.size, np.float32)
    blocks[0::2] = ref.scale
    blocks.view(np.int32)[1::2] = ref.zero
    dst = torch.full((length + 4,), 7.0, dtype=torch.float16 if dtype == F16 else torch.bfloat16,
                     device="cuda")
    Z.zero_dequantize_blocks(_to_gpu(codes), _to_gpu(blocks), bits, length, dst, dtype)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:length], want)
    assert np.all(got[length:] == O.from_f32(np.array([7.0], np.float32), dtype)[0])


def small(psi, n, rank, dtype=F16, steps=3, **kw):
    return Workload(name="small", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)


CASES = {
    "f16_fused_n3_tail_q8": (small(100_003, 3, 2), 8, ()),
    "f16_fused_n3_tail_q4": (small(100_003, 3, 2), 4, ()),
    "bf16_fused_n8_q8": (small(200_000, 8, 3, dtype=BF16), 8, ()),
    "bf16_fused_n8_q4": (small(200_000, 8, 3, dtype=BF16), 4, ()),
    "bf16_twopass_clip_n8_q8": (small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05), 8, ()),
    "f16_twopass_clip_n3_q4": (small(100_003, 3, 1, max_grad_norm=0.01), 4, ()),
    "f16_fused_n64_ragged_q4": (small(64 * 1_000 + 37, 64, 63), 4, ()),
    "f16_fused_n13_offset_odd_q8": (small(13 * 5_001, 13, 7, contrib_scale=2.0 ** 8, scaler=1,
                                          loss_scale=2.0 ** 8), 8, ()),
    "f16_fused_inf_skip_q8": (small(100_003, 3, 2, steps=4, scaler=2, contrib_scale=2.0 ** 10,
                                    loss_scale=2.0 ** 10), 8, (Inject(2, 1, 17_001, np.inf),)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_quantized_step_small(name):
    w, bits, extra = CASES[name]
    H.run_and_compare(Case(w, w.ranks[0], w.steps, extra=tuple(extra), qbits=bits), name)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_step_gpt2_sized(bits):
    """The GPT-2-sized shard (15,554,976 elements, N = 8, fp16, static scale
    2^16, 20 steps) with INT8 or INT4 contributions: every step's decisions
    against the oracle's full pass, elements on a sample (whole quantisation
    blocks around each sampled column)."""
    w = workloads.GPT2
    c = Case(w, w.ranks[0], w.steps, qbits=bits)
    g = H.DeviceRun(c, full_gather=False)
    g.run()
    reps = H.oracle_scalars(c)
    H.assert_reports(g.reports, reps)
    exact = H.same_clips(g.reports, reps)
    cols = H.sample_cols(c.part[2], 300, seed=17)
    p, m, v, slot = g.fetch(cols)
    rp, rm, rv, rslot = H.oracle_elements(c, reps, cols)
    H.assert_f32_close("master", p, rp, exact)
    H.assert_f32_close("m", m, rm, exact)
    H.assert_f32_close("v", v, rv, exact)
    H.assert_16bit_within_ulp("slot", slot, rslot, w.dtype, exact)
    H.log(f"gpt2 q{bits}: ok, norm {g.reports[-1]['norm']:.9g} (16-bit path: see parity tests)")


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("shift", [1, 2, 3])
@pytest.mark.parametrize("bits", [8, 4])
def test_quantize_and_dequantize_unaligned(bits, shift, dtype):
    """16-bit buffers at 2-, 4- and 6-byte offsets (a parameter slot at any
    offset), in both formats: the 16-bit loads and the narrower stores give
    the same codes and values as the oracle."""
    import torch
    import zero_partitioned_mixed_amd as Z
    length = 5 * 2048 + 333
    src = O.from_f32(_values(length, seed=40 + shift), dtype)
    ref = O.quantize(src, dtype, bits)
    buf = torch.zeros(length + 8, dtype=torch.int16, device="cuda")
    buf[shift:shift + length] = _to_gpu(src.view(np.int16))
    q = Z.QuantRows.alloc(1, length, bits, torch.device("cuda", 0))
    codes, blocks = q.rows[0]
    Z.zero_quantize_blocks(buf[shift:], dtype, length, bits, codes, blocks)
    tdt = torch.float16 if dtype == F16 else torch.bfloat16
    dst = torch.full((length + 8,), 7.0, dtype=tdt, device="cuda")
    Z.zero_dequantize_blocks(codes, blocks, bits, length, dst[shift:], dtype)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy()[:ref.codes.size], ref.codes)
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    want = O.cast(O.dequantize(ref), dtype)
    seven = O.from_f32(np.array([7.0], np.float32), dtype)[0]
    assert np.array_equal(got[shift:shift + length], want)
    assert np.all(got[:shift] == seven) and np.all(got[shift + length:] == seven)


@pytest.mark.parametrize("bits", [8, 4])
def test_quantized_all_gather_of_updated_slot(bits):
    """ZeRO++'s parameter path on one rank: after a fused step writes the
    rank's 16-bit slot (at an odd offset of the full buffer), the slot is
    block-quantised for the all-gather and dequantised on the receiving side
    into the same place of a second full buffer.  Checked against the oracle's
    step, quantiser and dequantiser."""
    import torch
    import zero_partitioned_mixed_amd as Z
    w = small(7 * 30_001, 7, 5, steps=2)
    c = Case(w, 5, 2)
    _, off, valid = c.part
    assert off % 2 == 1
    g = H.DeviceRun(c, full_gather=True)
    g.run()
    slot = g.gather[off:off + valid]
    q = Z.QuantRows.alloc(1, valid, bits, slot.device)
    codes, blocks = q.rows[0]
    Z.zero_quantize_blocks(slot, F16, valid, bits, codes, blocks)
    received = torch.zeros_like(g.gather)
    Z.zero_dequantize_blocks(codes, blocks, bits, valid, received[off:], F16)
    torch.cuda.synchronize()
    reps = H.oracle_scalars(c)
    _, _, _, oslot = H.oracle_elements(c, reps)
    got_slot = slot.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_slot, oslot)      # the step itself (fp16 slot) is exact here
    ref = O.quantize(oslot, F16, bits)
    assert np.array_equal(codes.cpu().numpy()[:ref.codes.size], ref.codes)
    got = received.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[off:off + valid], O.cast(O.dequantize(ref), F16))
    assert not got[:off].any() and not got[off + valid:].any()
