"""ZeRO-0/1/2/3 data layouts of a mixed-precision Adam step (test infrastructure).

Two uses:

* Byte accounting.  ``plan(stage, psi, N, r)`` lists the model-state buffers
  one rank allocates under each stage, and ``Tracker`` sums what is actually
  allocated, the way the simulation README's byte tracker measures per-GPU
  memory ("zero-stages-simulation" README, per-GPU model-state table).  The
  buffers follow the mixed-precision bill: fp16 parameters and gradients,
  fp32 master, momentum and variance ("ZeRO: Memory Optimizations Toward
  Training Trillion Parameter Models" summary, 3.4 "Model-State Memory
  Analysis"), partitioned cumulatively by stage (same page, Stage 1, 2 and 3;
  "ZeRO Stage 1/2/3" guide, sections 2-4).

* The exactness invariant.  ``run(stage, ...)`` performs whole steps of the
  toy workload in each layout: ZeRO-0 steps everything on one replica after
  the all-reduce mean; ZeRO-1 keeps the full averaged gradient and updates a
  slice; ZeRO-2 reduces only the owned slice; ZeRO-3 also keeps only the
  owned slice of the 16-bit parameters (the simulation README's "during
  backward / gradient sync / optimizer step" table).  The README reports the
  four layouts train identically; the oracle must reproduce that bit for bit.
"""
from __future__ import annotations

import numpy as np

from . import (F16, SumSq, adam, cast, finalize, inv_scale, new_scalars, partition, reduce)

STAGES = (0, 1, 2, 3)

_ITEMSIZE = {"fp16": 2, "fp32": 4}


def plan(stage: int, psi: int, nranks: int, rank: int) -> list[tuple[str, str, int]]:
    """Model-state buffers of one rank: (name, storage type, element count)."""
    if stage not in STAGES:
        raise ValueError(stage)
    shard, _, _ = partition(psi, nranks, rank)
    full_p = stage <= 2
    full_g = stage <= 1
    full_o = stage == 0
    return [
        ("param.fp16", "fp16", psi if full_p else shard),
        ("grad.fp16", "fp16", psi if full_g else shard),
        ("master.fp32", "fp32", psi if full_o else shard),
        ("adam_m.fp32", "fp32", psi if full_o else shard),
        ("adam_v.fp32", "fp32", psi if full_o else shard),
    ]


def planned_bytes(stage: int, psi: int, nranks: int, rank: int) -> int:
    return sum(_ITEMSIZE[t] * n for _, t, n in plan(stage, psi, nranks, rank))


class Tracker:
    """Allocates the buffers of a plan and counts their bytes."""

    def __init__(self):
        self.buffers: dict[str, np.ndarray] = {}

    def alloc(self, name: str, storage: str, count: int) -> np.ndarray:
        dt = np.uint16 if storage == "fp16" else np.float32
        a = np.zeros(count, dt)
        self.buffers[name] = a
        return a

    @property
    def nbytes(self) -> int:
        return sum(a.nbytes for a in self.buffers.values())


def allocate_rank(stage: int, psi: int, nranks: int, rank: int) -> Tracker:
    t = Tracker()
    for name, storage, count in plan(stage, psi, nranks, rank):
        t.alloc(name, storage, count)
    return t


def run(stage: int, psi: int, nranks: int, steps: int, contrib_fn, master0: np.ndarray, hp,
        loss_scale: float = 1.0, dtype_in: int = F16, dtype_out: int = F16):
    """``steps`` shard steps of one workload laid out as ZeRO-``stage``.

    ``contrib_fn(step)`` returns the [N, psi] 16-bit contributions of that
    step (step = 1, 2, ...).  Returns the full master, m, v (fp32, psi), the
    full 16-bit parameters as every rank would see them after the all-gather
    (stage <= 2) or as the concatenation of the owned parameter shards
    (stage 3), and the per-step reports.
    """
    st = new_scalars(loss_scale)
    reports = []
    if stage == 0:
        master = np.array(master0, np.float32)
        m = np.zeros(psi, np.float32)
        v = np.zeros(psi, np.float32)
        params = cast(master, dtype_out)
        for s in range(1, steps + 1):
            C = contrib_fn(s)
            g, flag = reduce(C, dtype_in, psi, inv_scale(nranks, st.scale))
            rep = finalize(hp, st, flag, SumSq().add(g))
            if not rep.skip:
                adam(master, m, v, g, hp, rep.clip, st.pow1, st.pow2)
                params = cast(master, dtype_out)
            reports.append(rep.as_dict())
        return master, m, v, params, reports

    parts = [partition(psi, nranks, r) for r in range(nranks)]
    own = []  # per rank: master, m, v of its valid slice
    for _, off, valid in parts:
        sl = np.array(master0[off:off + valid], np.float32)
        own.append((sl, np.zeros(valid, np.float32), np.zeros(valid, np.float32)))
    params_full = cast(np.asarray(master0, np.float32), dtype_out)
    param_shards = [params_full[off:off + valid].copy() for _, off, valid in parts]
    for s in range(1, steps + 1):
        C = contrib_fn(s)
        inv = inv_scale(nranks, st.scale)
        grads, flag, acc = [], 0, SumSq()
        if stage == 1:
            g_full, flag = reduce(C, dtype_in, psi, inv)  # all-reduce mean: full gradient on every rank
            for _, off, valid in parts:
                grads.append(g_full[off:off + valid].copy())
        else:  # reduce-scatter: each rank reduces only its slice
            for _, off, valid in parts:
                g, f = reduce(np.ascontiguousarray(C[:, off:off + valid]), dtype_in, valid, inv)
                grads.append(g)
                flag |= f
        for g in grads:
            acc.add(g)
        rep = finalize(hp, st, flag, acc)
        if not rep.skip:
            for (p, mm, vv), g, (_, off, valid), r in zip(own, grads, parts, range(nranks)):
                adam(p, mm, vv, g, hp, rep.clip, st.pow1, st.pow2)
                if stage == 3:
                    param_shards[r] = cast(p, dtype_out)
                else:  # the rank's slot of the buffer the all-gather fills
                    params_full[off:off + valid] = cast(p, dtype_out)
        reports.append(rep.as_dict())
    master = np.concatenate([o[0] for o in own])
    m = np.concatenate([o[1] for o in own])
    v = np.concatenate([o[2] for o in own])
    params = np.concatenate(param_shards) if stage == 3 else params_full
    return master, m, v, params, reports
