"""GPU parity: the HIP shard step through the C ABI against the CPU oracle.

Bars: fp32 master/m/v within |d| <= 1e-6 |x| + 1e-9; 16-bit parameters
within 1 ulp; overflow flags, skip decisions, t and loss scales exact; the
gradient norm within 1e-5 relative.  Sizes span many workgroup tiles with a
ragged tail; every slot alignment class, N from 1 to 64, both 16-bit formats,
both paths (fused single pass, two-pass with clipping), overflow at the first,
middle and last element, NaN, inf in the padding, empty ranks, and the
skip-and-halve sequence of the dynamic loss scaler.
"""
from dataclasses import replace

import numpy as np
import pytest

import harness as H
from harness import Case, Inject
from synth import workloads
from synth.workloads import BF16, F16, Workload

pytestmark = pytest.mark.gpu

_BELOW_ONE = float(np.nextafter(np.float32(1.0), np.float32(0.0)))  # 1 - 2^-24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import synth
    synth.gpu()
    import zero_partitioned_mixed_amd  # noqa: F401  (fails loudly when the library is missing)
    torch.cuda.init()
    yield


def run_case(c: Case, label: str, full: bool = True):
    return H.run_and_compare(c, label, full)


def small(psi, n, rank, dtype=F16, steps=3, **kw):
    w = Workload(name="small", psi=psi, nranks=n, ranks=(rank,), dtype=dtype, steps=steps, **kw)
    return w


# --------------------------------------------------------------------------- generator
def test_device_generator_matches_host():
    import torch
    import synth
    w = workloads.P13B
    n, stride, off, ln = 8, 4096, 1_625_000_000 * 7 + 12_345, 4000
    c = torch.empty((n, stride), dtype=torch.float16, device="cuda")
    synth.gpu_contrib_rows(c, w.seed, 3, F16, 1e-3, 2.0 ** 15, 1e-3, 100.0, off, ln)
    ref = synth.contrib_rows(w.seed, 3, n, F16, 1e-3, 2.0 ** 15, 1e-3, 100.0, off, ln, stride=stride)
    assert np.array_equal(c.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    for dt, tdt in ((F16, torch.float16), (BF16, torch.bfloat16)):
        p = torch.empty(5000, dtype=tdt, device="cuda")
        synth.gpu_param_range(p, 0, 0.02, dt, 10 ** 10)
        assert np.array_equal(p.view(torch.int16).cpu().numpy().view(np.uint16),
                              synth.param_range(0, 0.02, dt, 10 ** 10, 5000))
    mm = torch.empty(5000, dtype=torch.float32, device="cuda")
    synth.gpu_master_range(mm, 0, 0.02, 999)
    assert np.array_equal(mm.cpu().numpy(), synth.master_range(0, 0.02, 999, 5000))


# --------------------------------------------------------------------------- cast
CAST_VALUES = np.array(
    [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 7e4, 2.0 ** -24, 2.0 ** -25,
     3 * 2.0 ** -25, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11), 1e-8, 1e-30, 1e-40, 1.4e-45,
     3.3895314e38, 3.4e38, np.inf, -np.inf, np.nan, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11,
     1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 0.1, 0.2, -0.3], np.float32)


@pytest.mark.parametrize("dtype", [F16, BF16])
@pytest.mark.parametrize("offset", [0, 1, 2, 3, 4, 8, 13])
def test_cast_to_gather(dtype, offset):
    import torch
    import oracle as O
    import zero_partitioned_mixed_amd as Z
    rng = np.random.default_rng(offset)
    vals = np.concatenate([CAST_VALUES, rng.normal(0, 1, 5000).astype(np.float32),
                           (rng.normal(0, 1, 3000) * 2.0 ** rng.integers(-30, 20, 3000)).astype(np.float32)])
    n = vals.size
    master = torch.from_numpy(vals).cuda()
    tdt = torch.float16 if dtype == F16 else torch.bfloat16
    gather = torch.full((n + offset + 40,), 7.0, dtype=tdt, device="cuda")
    Z.zero_cast_to_gather(master, n, gather, dtype, offset)
    bits = gather.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = O.from_f32(vals, dtype)
    got = bits[offset:offset + n]
    nan = np.isnan(vals)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(O.to_f32(got[nan], dtype)))
    canary = O.from_f32(np.array([7.0], np.float32), dtype)[0]
    assert np.all(bits[:offset] == canary) and np.all(bits[offset + n:] == canary)


# --------------------------------------------------------------------------- small cases
SMALL = {
    "f16_fused_n3_tail_rank": (small(100_003, 3, 2), ()),
    "f16_twopass_clip_n3": (small(100_003, 3, 1, max_grad_norm=0.01), ()),
    "bf16_fused_n8_aligned": (small(200_000, 8, 3, dtype=BF16), ()),
    "bf16_twopass_clip_n8_wd": (small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05,
                                      weight_decay=0.01), ()),
    "f16_fused_n1": (small(50_001, 1, 0, contrib_scale=2.0 ** 8, scaler=1, loss_scale=2.0 ** 8), ()),
    "f16_fused_n7_offset_odd": (small(69_990, 7, 5), ()),
    "bf16_fused_n64_ragged": (small(64 * 1_000 + 37, 64, 63, dtype=BF16), ()),
    "f16_fused_n32_gpt2ish": (small(32 * 4_099, 32, 17, contrib_scale=2.0 ** 16, scaler=1,
                                    loss_scale=2.0 ** 16, weight_decay=0.01), ()),
    "f16_fused_inf_first": (small(100_003, 3, 2, steps=4, scaler=2, contrib_scale=2.0 ** 10,
                                  loss_scale=2.0 ** 10), (Inject(2, 0, 0, np.inf),)),
    "f16_fused_nan_last": (small(100_003, 3, 2, steps=4, scaler=2, contrib_scale=2.0 ** 10,
                                 loss_scale=2.0 ** 10), (Inject(3, 2, 33_332, np.nan),)),
    "f16_fused_inf_and_neg_inf_mid": (small(100_003, 3, 2, steps=3), (
        Inject(2, 0, 17_001, np.inf), Inject(2, 1, 17_001, -np.inf))),
    "f16_fused_inf_in_padding": (small(100_003, 3, 2, steps=2), (Inject(1, 1, 33_340, np.inf),)),
    "bf16_twopass_inf_skip": (small(200_000, 8, 5, dtype=BF16, max_grad_norm=0.05, steps=4),
                              (Inject(2, 7, 12_345, np.inf),)),
    "f16_fused_skip_offset_odd": (small(69_990, 7, 5, steps=3, scaler=2, contrib_scale=2.0 ** 10,
                                        loss_scale=2.0 ** 10), (Inject(2, 3, 4_000, np.inf),)),
    "bf16_fused_skip_offset_2mod4": (small(100_003, 3, 2, dtype=BF16, steps=3),
                                     (Inject(2, 0, 2_049, np.nan),)),
    "f16_fused_zero_gradients": (small(100_003, 3, 2, contrib_sigma=0.0, weight_decay=0.01), ()),
    "bf16_twopass_zero_gradients_clip": (small(100_003, 3, 1, dtype=BF16, contrib_sigma=0.0,
                                               max_grad_norm=1.0), ()),
    "f16_fused_skip_every_step_to_floor": (
        small(60_016, 4, 3, steps=4, scaler=2, contrib_scale=4.0, loss_scale=4.0, min_scale=1.0),
        tuple(Inject(s, s % 4, 100 * s, np.inf) for s in range(1, 5))),
    "f16_fused_dynamic_growth": (small(60_016, 4, 3, steps=6, scaler=2, growth_interval=2,
                                       contrib_scale=2.0 ** 12, loss_scale=2.0 ** 12),
                                 (Inject(4, 1, 5, np.inf),)),
    # growth asked for at every step from the largest power of two in fp32:
    # the scale stays 2^127 instead of overflowing to inf (bf16 contributions
    # carry that scale; the unscaled gradient is ~1e-3)
    "bf16_fused_growth_at_fp32_max": (small(60_016, 4, 3, dtype=BF16, steps=4, scaler=2,
                                            growth_interval=1, contrib_scale=2.0 ** 127,
                                            loss_scale=2.0 ** 127), ()),
    "bf16_twopass_growth_at_fp32_max": (small(100_003, 3, 1, dtype=BF16, steps=3, scaler=2,
                                              growth_interval=1, contrib_scale=2.0 ** 127,
                                              loss_scale=2.0 ** 127, max_grad_norm=1.0), ()),
    # degenerate hyperparameters: no moments (each step uses g and g*g alone);
    # moments that barely decay (1 - beta is one fp32 ulp below 1, so the bias
    # corrections are near 6e-8 t); lr = 0 with weight decay (the master must
    # not move); eps = 0, where an element whose gradient sums to exactly 0
    # divides 0 by 0 and its master and parameter turn NaN on both sides
    "f16_fused_betas_zero": (small(100_003, 3, 2, beta1=0.0, beta2=0.0), ()),
    "bf16_twopass_betas_near_one": (small(100_003, 3, 1, dtype=BF16, beta1=_BELOW_ONE,
                                          beta2=_BELOW_ONE, max_grad_norm=0.05), ()),
    "f16_fused_lr_zero_wd": (small(100_003, 3, 2, lr=0.0, weight_decay=0.1), ()),
    "f16_fused_eps_zero": (small(100_003, 3, 2, eps=0.0, contrib_scale=2.0 ** 10, scaler=1,
                                 loss_scale=2.0 ** 10), ()),
    "bf16_twopass_eps_zero_clip": (small(200_000, 8, 5, dtype=BF16, eps=0.0, max_grad_norm=0.05),
                                   ()),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(name):
    w, extra = SMALL[name]
    g, _ = run_case(Case(w, w.ranks[0], w.steps, extra=tuple(extra)), name)
    if "growth_at_fp32_max" in name:
        assert all(r["loss_scale"] == 2.0 ** 127 for r in g.reports)
    if "eps_zero" in name:   # the case is only degenerate if some element met 0/0
        assert np.isnan(g.fetch()[0]).any()
    if name == "f16_fused_lr_zero_wd":
        _, off, valid = g.c.part
        p0 = H.synth.master_range(w.seed, w.master_sigma, off, valid)
        assert np.array_equal(g.fetch()[0].view(np.uint32), p0.view(np.uint32))


# Shards long enough for the restore's unrolled loop (eight whole tiles per
# workgroup of its 256-workgroup grid, so at least 2,048 tiles) plus its
# one-tile remainder and a partial last tile; a skip at step 2 makes the
# restore rewrite the slot.  Offsets: 8-byte, 4-byte and 2-byte aligned slots.
@pytest.mark.parametrize("psi,n,rank", [(2 * 4_200_001, 2, 1), (3 * 4_200_002, 3, 1),
                                        (2 * 4_200_004, 2, 1)])
def test_restore_after_skip_long_shard(psi, n, rank):
    w = small(psi, n, rank, steps=3, **DYN)
    _, off, valid = H.O.partition(psi, n, rank)
    assert valid // 2048 >= 2048
    c = Case(w, rank, 3, extra=(Inject(2, n - 1, valid - 7, np.inf),))
    g, _ = run_case(c, f"restore long shard psi={psi} n={n} offset%4={off % 4}")
    assert [r["skip"] for r in g.reports] == [0, 1, 0]


@pytest.mark.parametrize("dtype", [F16, BF16])
def test_clip_threshold_just_above_the_norm(dtype):
    """max_grad_norm set to an fp32 value in (norm, norm + 1e-6] of the first
    step's gradient: the coefficient max / (norm + 1e-6) is below 1, so the
    step is clipped (as torch's clip_grad_norm_ clips it) although the norm
    does not exceed the threshold."""
    w0 = small(100_003, 3, 1, dtype=dtype, steps=1)
    norm = H.oracle_scalars(Case(w0, 1, 1))[0]["norm"]
    mx = np.float32(norm)
    while float(mx) <= norm:
        mx = np.nextafter(mx, np.float32(np.inf))
    assert norm < float(mx) <= norm + 1e-6
    w = replace(w0, max_grad_norm=float(mx), steps=2)
    c = Case(w, 1, 2)
    reps = H.oracle_scalars(c)
    assert reps[0]["clip"] < 1.0
    g, _ = run_case(c, f"clip window dtype={dtype} max={float(mx)!r} norm={norm!r}")
    assert g.reports[0]["clip"] == reps[0]["clip"] < 1.0


DYN = dict(scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)

# Contributions in one 16-bit format, the gathered parameters in the other.
# name: (workload, contribution bits (0: 16-bit), layout, payload bits, injections)
MIXED = {
    "f16_in_bf16_slot_fused_skip": (small(8 * 25_007, 8, 3, steps=4, gather_dtype=BF16, **DYN),
                                    0, "strided", 0, (Inject(2, 6, 10_001, np.inf),)),
    "bf16_in_f16_slot_fused_n3_odd": (small(100_003, 3, 2, dtype=BF16, gather_dtype=F16), 0,
                                      "strided", 0, ()),
    "f16_in_bf16_slot_two_pass_clip": (small(200_000, 8, 5, max_grad_norm=0.05,
                                             gather_dtype=BF16), 0, "strided", 0, ()),
    "bf16_in_f16_slot_two_pass_n64": (small(64 * 1_000 + 37, 64, 63, dtype=BF16,
                                            max_grad_norm=0.05, gather_dtype=F16), 0,
                                      "strided", 0, ()),
    "f16_rows_in_bf16_slot_int8_payload": (small(8 * 25_007, 8, 6, gather_dtype=BF16), 0, "rows",
                                           8, ()),
    "bf16_int4_rows_in_f16_slot_int8_payload": (small(8 * 25_007, 8, 7, dtype=BF16,
                                                      gather_dtype=F16), 4, "strided", 8, ()),
}


@pytest.mark.parametrize("name", list(MIXED))
def test_mixed_formats(name):
    """The slot's 16-bit format differs from the contributions': every kernel
    instantiation with the two formats apart, against the oracle (slot and
    payload in the slot's format)."""
    w, qbits, layout, payload, extra = MIXED[name]
    assert w.slot_dtype != w.dtype
    H.run_and_compare(Case(w, w.ranks[0], w.steps, extra=tuple(extra), qbits=qbits), name,
                      layout=layout, qgather=payload)


def test_empty_tail_rank():
    import torch
    import zero_partitioned_mixed_amd as Z
    # psi = 10 over 7 ranks: shard 2, rank 6 owns nothing
    w = small(10, 7, 6)
    c = Case(w, 6, 2)
    assert c.part == (2, 12, 0)
    g = H.DeviceRun(c)
    before = g.gather.clone()
    g.run()
    assert torch.equal(g.gather.view(torch.int16), before.view(torch.int16))
    for r in g.reports:
        assert r["sumsq"] == 0.0 and r["skip"] == 0
    assert g.reports[-1]["t"] == 2


def test_run_to_run_bitwise():
    w = small(300_007, 8, 6, dtype=BF16, max_grad_norm=0.02)
    outs = []
    for _ in range(2):
        g = H.DeviceRun(Case(w, 6, 3))
        g.run()
        outs.append((g.fetch(), [r["sumsq"] for r in g.reports]))
    (a, sa), (b, sb) = outs
    assert sa == sb
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                              y.view(np.uint32) if y.dtype == np.float32 else y)


# --------------------------------------------------------------------------- toy: all 32 shards
def _toy(inject=None, w=None):
    import torch
    import oracle as O
    import synth
    import zero_partitioned_mixed_amd as Z
    w = workloads.TOY if w is None else w
    n = w.nranks
    H.log(f"toy: psi={w.psi} N={n} all shards, steps={w.steps}, inject={inject}")
    gather = torch.empty(w.psi, dtype=torch.float16, device="cuda")
    synth.gpu_param_range(gather, w.seed, w.master_sigma, F16, 0)
    hp = Z.hparams(lr=w.lr)
    steps, contribs, parts = [], [], []
    for r in range(n):
        shard, off, valid = Z.zero_partition(w.psi, n, r)
        stride = (shard + 63) // 64 * 64
        p0 = torch.empty(valid, dtype=torch.float32, device="cuda")
        synth.gpu_master_range(p0, w.seed, w.master_sigma, off)
        s0 = (p0, torch.zeros_like(p0), torch.zeros_like(p0))
        steps.append(Z.ShardStep(n, stride, valid, off, F16, F16, hp, s0))
        contribs.append(torch.empty((n, stride), dtype=torch.float16, device="cuda"))
        parts.append((off, valid, stride))
    multi = Z.MultiShardStep(steps)
    gpu_reps = []
    for s in range(1, w.steps + 1):
        for r, (off, valid, stride) in enumerate(parts):
            synth.gpu_contrib_rows(contribs[r], w.seed, s, F16, w.contrib_sigma, 1.0, 0.0, 100.0,
                                   off, valid)
            if inject and inject[0] == s and inject[1] == r:
                contribs[r][inject[2], inject[3]] = float("inf")
        multi.step(contribs, gather)
        gpu_reps.append([Z.read_ctrl(st.ctrl) for st in steps])
    torch.cuda.synchronize()
    # oracle: the same step over all 32 ranks with shared scalars
    ohp = O.hparams(lr=w.lr)
    sc = O.new_scalars(1.0)
    states = [O.RankState.fresh(synth.master_range(w.seed, w.master_sigma, off, valid))
              for off, valid, _ in parts]
    ogather = synth.param_range(w.seed, w.master_sigma, F16, 0, w.psi)
    for s in range(1, w.steps + 1):
        cs = []
        for r, (off, valid, stride) in enumerate(parts):
            C = synth.contrib_rows(w.seed, s, n, F16, w.contrib_sigma, 1.0, 0.0, 100.0, off, valid)
            if inject and inject[0] == s and inject[1] == r:
                C[inject[2], inject[3]] = 0x7C00
            cs.append(C)
        rep = O.shard_step(cs, F16, states, [p[0] for p in parts], sc, ohp, ogather, F16)
        for rr in gpu_reps[s - 1]:  # every rank agrees on the global decisions
            assert rr["skip"] == rep.skip and rr["nonfinite"] == rep.nonfinite
            assert rr["t"] == sc.t
            if np.isfinite(rep.norm):
                assert abs(rr["norm"] - rep.norm) <= H.NORM_RTOL * rep.norm
            else:
                assert not np.isfinite(rr["norm"]) and np.isnan(rr["norm"]) == np.isnan(rep.norm)
    for r, st in enumerate(steps):
        cur = st.current()
        for name, t, ref in zip(("master", "m", "v"), cur,
                                (states[r].master, states[r].m, states[r].v)):
            H.assert_f32_close(f"rank{r}.{name}", t.cpu().numpy(), ref)
    got = gather.view(torch.int16).cpu().numpy().view(np.uint16)
    H.assert_16bit_within_ulp("gather", got, ogather, F16)
    H.log("toy: ok")


def test_toy_all_shards():
    _toy()


def test_toy_overflow_on_one_rank_skips_all():
    _toy(inject=(2, 5, 3, 19_000))


def test_64_ranks_combined_in_one_decision():
    """ZERO_MAX_RANKS = 64 shards of a ragged buffer (the last one short)
    stepped on one GPU with one shared decision per step."""
    w = Workload(name="ranks64", psi=64 * 3_001 - 40, nranks=64, ranks=tuple(range(64)),
                 dtype=F16, steps=2)
    _toy(w=w)


def test_max_contributions_in_one_buffer():
    """ZERO_MAX_CONTRIB = 1024 contribution rows in one [N, stride] buffer
    (128 chunks of eight rows in the generic loop), fused and two-pass."""
    run_case(Case(small(1024 * 2_101, 1024, 1023), 1023, 2), "n1024_fused")
    run_case(Case(small(1024 * 2_101, 1024, 5, dtype=BF16, max_grad_norm=0.01), 5, 2),
             "n1024_two_pass")


# --------------------------------------------------------------------------- full configs
def test_gpt2_sized_full():
    w = workloads.GPT2
    run_case(Case(w, w.ranks[0], w.steps), w.name, full=False)


def test_psi1_5b_n64_full():
    w = workloads.P1_5B
    run_case(Case(w, w.ranks[0], w.steps), w.name, full=False)


# --------------------------------------------------------------------------- paired state, finalize groups
def test_pair_store_load_round_trip():
    import torch
    import zero_partitioned_mixed_amd as Z
    dev = torch.device("cuda", 0)
    for n in (1, 7, 2048, 2049, 100_003):
        flat = tuple(torch.randn(n, device=dev) for _ in range(3))
        pair = Z.paired_state(n, dev)
        pair[0].fill_(float("nan"))
        ctrl = torch.empty(Z.zero_ctrl_bytes(), dtype=torch.uint8, device=dev)
        Z.zero_ctrl_init(ctrl, 1.0)
        Z.zero_pair_store(flat, pair, n, ctrl)
        back = tuple(torch.empty(n, device=dev) for _ in range(3))
        Z.zero_pair_load(pair, back, n, ctrl)
        for a, b in zip(flat, back):
            assert torch.equal(a, b)
        # one buffer [tile][set][master|m|v][2048]: set 0 holds the data, set 1 is untouched
        p = pair[0][:Z.zero_pair_elems(n)].view(-1, 2, 3, 2048)
        assert torch.isnan(p[:, 1]).all()
        for q in range(3):
            assert torch.equal(p[:, 0, q].reshape(-1)[:n], flat[q])


@pytest.mark.parametrize("tiles", [16384, 16385])
def test_finalize_single_and_grouped(tiles):
    """One finalize workgroup takes up to 16384 per-tile partials; beyond that
    the grouped path (ranges, then the last group to arrive) runs."""
    w = small(tiles * 2048 - 1000, 1, 0, dtype=BF16, steps=2, max_grad_norm=0.5)
    run_case(Case(w, 0, 2), f"finalize_{tiles}_tiles", full=False)


@pytest.mark.parametrize("pad", [8, 4096 + 24])
@pytest.mark.parametrize("two_pass", [False, True])
def test_row_strides_beyond_the_shard(pad, two_pass):
    """Row strides that are any multiple of eight elements beyond the shard
    (here shard + 8 and shard + 4120, neither a multiple of 64), with an inf
    in every row's padding that must be ignored."""
    kw = dict(max_grad_norm=0.02) if two_pass else {}
    w = small(3 * 33_335 - 2, 3, 2, dtype=BF16, **kw)
    c0 = Case(w, 2, 2)
    valid = c0.part[2]
    stride = (c0.part[0] + 63) // 64 * 64 + pad
    extra = tuple(Inject(1, k, stride - 1, np.inf) for k in range(3))
    c = Case(w, 2, 2, extra=extra, stride_pad=pad)
    assert c.stride == stride and c.stride % 64 != 0 and stride - 1 >= valid
    run_case(c, f"stride_pad_{pad}_{'two_pass' if two_pass else 'fused'}")
