"""Several ranks' shards on one GPU through the batched calls
(zero_fused_step_shards and zero_fused_restore_shards; zero_reduce_grads_shards
and zero_adam_step_shards) against every rank's own calls (zero_fused_step and
zero_fused_restore; zero_reduce_grads and zero_adam_step), bit for bit: every
step's ctrl of every rank, every rank's state, and the whole parameter
buffer.  The oracle checks of MultiShardStep (the toy's 32 shards, 64 ranks
of a ragged buffer, an overflow on one rank, the ZeRO layouts) take the
batched calls by default."""
import itertools

import numpy as np
import pytest

import harness as H
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


def _ws(psi, n, ranks, dtype=F16, steps=3, **kw):
    return Workload(name="shards", psi=psi, nranks=n, ranks=tuple(ranks), dtype=dtype, steps=steps,
                    **kw)


DYN = dict(scaler=2, contrib_scale=2.0 ** 10, loss_scale=2.0 ** 10)

# (workload, injected +inf as (step, rank index, row, column) or None)
CASES = {
    # 32 ranks of 10 tiles, N = 32 (the any-N kernel), a skip on every rank at step 2
    "toy_skip": (_ws(workloads.TOY.psi, 32, range(32), **DYN), (2, 9, 4, 1_000)),
    # 64 ranks (two launches of 32 shards), bf16 rows into an fp16 parameter buffer, shard
    # length 3,001 (slots at 8-, 4- and 2-byte alignment), the last shard short
    "ranks64_mixed_ragged": (_ws(64 * 3_001 - 40, 64, range(64), dtype=BF16, gather_dtype=F16,
                                 weight_decay=0.01), None),
    # N = 8 (the eight-row kernel), fp16 rows into a bf16 buffer, a skip at step 3
    "n8_skip": (_ws(8 * 40_001, 8, range(8), gather_dtype=BF16, steps=4, **DYN), (3, 7, 0, 40_000)),
    # three ranks of 1,500 tiles of a 64-rank buffer: one launch each (2,048 tiles a launch at N = 64)
    "launch_split": (_ws(64 * 1_500 * 2048, 64, (0, 1, 63), dtype=BF16, steps=2), None),
    # 16-element shards, the last rank's empty
    "tiny_empty_rank": (_ws(1_000, 64, range(64), steps=2), None),
    # the two-pass path (clipping): the toy's 32 shards with a skip at step 2 (every applied
    # step clips at 1e-3), 64 ranks of mixed formats with decay, N = 8 with a threshold that
    # binds on some steps only, 16-element shards with an empty rank
    "two_pass_toy_skip": (_ws(workloads.TOY.psi, 32, range(32), max_grad_norm=1e-3, **DYN),
                          (2, 9, 4, 1_000)),
    "two_pass_ranks64_mixed": (_ws(64 * 3_001 - 40, 64, range(64), dtype=BF16, gather_dtype=F16,
                                   weight_decay=0.01, max_grad_norm=0.05), None),
    "two_pass_n8": (_ws(8 * 40_001, 8, range(8), gather_dtype=BF16, steps=4, max_grad_norm=0.06,
                        outlier_p=1e-4), None),
    "two_pass_tiny_empty_rank": (_ws(1_000, 64, range(64), steps=2, max_grad_norm=0.01), None),
}


def _run(w, inject, batched: bool, graph: bool = False):
    import torch
    import synth
    import zero_partitioned_mixed_amd as Z
    dev = torch.device("cuda", 0)
    hp = Z.hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                   max_grad_norm=w.max_grad_norm, scaler=w.scaler, min_scale=w.min_scale,
                   growth_interval=w.growth_interval)
    tdt = torch.float16 if w.dtype == F16 else torch.bfloat16
    gdt = torch.float16 if w.slot_dtype == F16 else torch.bfloat16
    steps, contribs, parts = [], [], []
    for r in w.ranks:
        _, off, valid = Z.zero_partition(w.psi, w.nranks, r)
        p0 = torch.empty(max(valid, 1), dtype=torch.float32, device=dev)
        synth.gpu_master_range(p0, w.seed, w.master_sigma, off)
        stride = max((valid + 63) // 64 * 64, 64)
        g = torch.empty_like(p0) if w.max_grad_norm > 0 else None
        steps.append(Z.ShardStep(w.nranks, stride, valid, off, w.dtype, w.slot_dtype, hp,
                                 (p0, torch.zeros_like(p0), torch.zeros_like(p0)), g,
                                 w.loss_scale))
        contribs.append(torch.empty((w.nranks, stride), dtype=tdt, device=dev))
        parts.append((off, valid))
    gather = torch.empty(w.psi, dtype=gdt, device=dev)
    synth.gpu_param_range(gather, w.seed, w.master_sigma, w.slot_dtype, 0)
    multi = Z.MultiShardStep(steps, batched=batched)
    assert (multi._batch_table(contribs, gather, [None] * len(steps)) is not None) == batched
    g = multi.capture(contribs, gather) if graph else None
    torch.cuda.synchronize()
    reports = []
    for s in range(1, w.steps + 1):
        for c, (off, valid) in zip(contribs, parts):
            if valid:
                synth.gpu_contrib_rows(c, w.seed, s, w.dtype, w.contrib_sigma, w.contrib_scale,
                                       w.outlier_p, w.outlier_mult, off, valid)
        if inject and inject[0] == s:
            contribs[inject[1]][inject[2], inject[3]] = float("inf")
        if g is None:
            multi.step(contribs, gather)
        else:
            g.replay()
        torch.cuda.synchronize()
        reports.append([st.ctrl_dict() for st in steps])
    state = [np.concatenate([t[:valid].cpu().numpy() for t in st.current()])
             for st, (_, valid) in zip(steps, parts)]
    return reports, state, gather.view(torch.int16).cpu().numpy()


# every compiled form of the batched step: contribution format, slot format,
# the eight-row kernel or any N; all n ranks of a buffer of n shards of 5,001
# elements (three whole tiles and a ragged one each, slots at every
# alignment), the second step skipped so that the restore runs in each slot
# format
FORMS = {f"{path}_{a}_to_{b}_n{n}": (_ws(n * 5_001, n, range(n), dtype=da, gather_dtype=db,
                                          steps=3, max_grad_norm=clip, **DYN), (2, 0, n - 1, 4_321))
         for (path, clip), (a, da), (b, db), n in itertools.product(
             (("fused", 0.0), ("two_pass", 0.02)), (("f16", F16), ("bf16", BF16)),
             (("f16", F16), ("bf16", BF16)), (8, 3))}


@pytest.mark.parametrize("name", list(CASES) + list(FORMS))
def test_batched_shards_equal_their_own_calls(name):
    w, inject = CASES[name] if name in CASES else FORMS[name]
    H.log(f"shards {name}: psi={w.psi} N={w.nranks} ranks={len(w.ranks)} inject={inject}")
    ra, sa, ga = _run(w, inject, batched=False)
    rb, sb, gb = _run(w, inject, batched=True)
    assert repr(ra) == repr(rb)
    for x, y in zip(sa, sb):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ga, gb)
    skips = [r[0]["skip"] for r in rb]
    assert all(repr(r[0]) == repr(x) for r in rb for x in r)  # one decision for all ranks
    if inject:
        assert skips[inject[0] - 1] == 1 and sum(skips) == 1
    H.log(f"shards {name}: batched equals per-rank calls; skips {skips}")


@pytest.mark.parametrize("name", ["toy_skip", "two_pass_toy_skip"])
def test_batched_shards_in_a_graph(name):
    """The batched step (three launches) captured once and replayed equals
    the per-rank calls run eagerly, with a skip at step 2."""
    w, inject = CASES[name]
    ra, sa, ga = _run(w, inject, batched=False)
    rb, sb, gb = _run(w, inject, batched=True, graph=True)
    assert repr(ra) == repr(rb)
    for x, y in zip(sa, sb):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ga, gb)


def _draw(seed: int):
    """A random multi-rank step: N, Psi (ragged, sometimes with empty tail
    ranks), a random subset of the ranks (at most 64) in random order, the
    formats in and out, the path, the scaler, the step count, decay, and
    sometimes a +inf in one rank's rows."""
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.choice([1, 2, 3, 5, 8, 8, 13, 32, 64]))
    psi = int(rng.integers(1, 200_000))
    nr = int(rng.integers(1, n + 1))
    ranks = tuple(int(r) for r in rng.permutation(n)[:nr])
    dtype = int(rng.choice([F16, BF16]))
    gdt = int(rng.choice([F16, BF16]))
    steps = int(rng.integers(1, 4))
    scaler = int(rng.choice([0, 1, 2]))
    scale = float(2.0 ** int(rng.integers(4, 12))) if scaler else 1.0
    kw = dict(contrib_scale=scale, loss_scale=scale, scaler=scaler, growth_interval=2,
              weight_decay=float(rng.choice([0.0, 0.01])), gather_dtype=gdt)
    if rng.random() < 0.5:
        kw["max_grad_norm"] = float(rng.choice([1e-3, 0.05, 10.0]))
    w = _ws(psi, n, ranks, dtype=dtype, steps=steps, **kw)
    inject = None
    if rng.random() < 0.3 and steps > 1:
        i = int(rng.integers(0, nr))
        _, _, valid = H.O.partition(psi, n, ranks[i])
        if valid:
            inject = (int(rng.integers(1, steps + 1)), i, int(rng.integers(0, n)),
                      int(rng.integers(0, valid)))
    return w, inject


@pytest.mark.parametrize("seed", range(1, 49))
def test_random_batched_shards_equal_their_own_calls(seed):
    """48 random multi-rank steps through the batched calls and through every
    rank's own calls: bit for bit, as in the fixed cases."""
    w, inject = _draw(seed)
    ra, sa, ga = _run(w, inject, batched=False)
    rb, sb, gb = _run(w, inject, batched=True)
    assert repr(ra) == repr(rb)
    for x, y in zip(sa, sb):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ga, gb)
    H.log(f"random shards {seed}: psi={w.psi} N={w.nranks} ranks={len(w.ranks)} "
          f"{w.variant} inject={inject}: batched equals per-rank calls")
