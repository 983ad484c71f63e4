#!/usr/bin/env python3
"""Benchmark of the ZeRO per-rank shard step on one MI355X.

A step is one pass of the whole hot path over one rank's shard with its N
gradient contributions already resident in HBM: reduce + unscale + average,
overflow check and global norm, Adam(W) on the fp32 master/m/v, cast into the
rank's slot of the full 16-bit parameter buffer (plus, on the fused path, the
step decision and the restore check; on the two-pass path, the g buffer).

Prints ONE JSON line.  ``value`` is the effective bandwidth: the step's
algorithmic bytes (2N + 26 per element fused, 2N + 34 two-pass) divided by
the measured time per step.  ``roofline`` reports the dominant kernel against
the 8 TB/s HBM peak with its own HIP-event timing; ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused ZeRO shard step effective GB/s + % of HBM peak (1 MI355X)"
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "psi1.3e10_n8_dynscale"


def _fmt(x, nd=3):
    return float(f"{x:.{nd}g}") if x is not None else None


def kernel_isa_digest(kernel: str):
    """SHA-256 of the named kernel's machine code in the built library (from
    libzero_shard.isa.json, which the build writes), or None."""
    from zero_partitioned_mixed_amd import build as zbuild
    try:
        with open(zbuild.ISA_JSON) as f:
            return json.load(f).get(kernel)
    except (OSError, ValueError):
        return None


def measured_traffic(label: str, workload: str):
    """HBM bytes per pass (one call of the entry point, all its launches) from
    the committed PMC summary of this kernel and workload, or None when there
    is none or when the profiled kernel's machine code differs from the one in
    the built library (the counters then describe another kernel)."""
    path = os.path.join(PROFILES, f"{label}_{workload}_pmc.md")
    try:
        fields = {}
        for line in open(path):
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
        digest = kernel_isa_digest(fields["kernel"])
        if digest is None or fields.get("isa_sha256") != digest:
            return None
        return int(fields["traffic_bytes_per_pass"]), fields["kernel"], digest
    except (OSError, KeyError, ValueError):
        return None


def quant_bytes_per_elem(w, bits: int) -> float:
    """Algorithmic bytes per element with block-quantised contributions: N
    rows of bits/8-byte codes plus one 8-byte block record per 2048 elements
    per row, instead of N 16-bit values."""
    return w.bytes_per_elem - 2 * w.nranks + w.nranks * (bits / 8 + 8 / 2048)


def setup(w, torch, synth, Z, rows=False, qbits=0, bucket=0):
    """Buffers of the measured rank, inputs generated in HBM.  With `rows`, the
    N contribution rows live in N separate allocations and the step goes
    through the row-table calls; with `qbits`, the rows are block-quantised
    (INT8 or INT4, quantised on the GPU from the 16-bit rows) and the step
    goes through the quantised calls."""
    rank = w.ranks[-1]
    shard, off, valid = Z.zero_partition(w.psi, w.nranks, rank)
    stride = w.stride
    dev = torch.device("cuda", 0)
    tdt = torch.float16 if w.dtype == Z.F16 else torch.bfloat16
    # Optimizer state first, as a training job allocates it at start-up, then
    # the gradient contributions and the parameter buffer.  The order decides
    # which physical memory each buffer gets: over fresh processes on one machine,
    # the 13B step's median went from 6.04 to 6.14 TB/s (14 runs each), and
    # runs below 5.7 TB/s from 6 of 20 to none of 20 in a second sample.
    p0 = torch.empty(valid, dtype=torch.float32, device=dev)
    synth.gpu_master_range(p0, w.seed, w.master_sigma, off)
    state0 = (p0, torch.zeros_like(p0), torch.zeros_like(p0))
    fused = w.max_grad_norm <= 0
    g = None if fused else torch.empty_like(p0)
    hp = Z.hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                   max_grad_norm=w.max_grad_norm, scaler=w.scaler, min_scale=w.min_scale,
                   growth_interval=w.growth_interval)
    st = Z.ShardStep(w.nranks, stride, valid, off, w.dtype, w.dtype, hp, state0, g,
                     w.loss_scale, bucket=bucket)
    if fused:  # the flat state is only needed to load the paired copy
        torch.cuda.synchronize()
        del state0, p0
        st.state = None
        torch.cuda.empty_cache()
    contrib = torch.empty((w.nranks, stride), dtype=tdt, device=dev)
    synth.gpu_contrib_rows(contrib, w.seed, 1, w.dtype, w.contrib_sigma, w.contrib_scale,
                           w.outlier_p, w.outlier_mult, off, valid)
    gather = torch.empty(w.psi, dtype=tdt, device=dev)
    synth.gpu_param_range(gather, w.seed, w.master_sigma, w.dtype, 0)
    if qbits:
        q = Z.QuantRows.alloc(w.nranks, valid, qbits, dev)
        for k, (codes, blocks) in enumerate(q.rows):
            Z.zero_quantize_blocks(contrib[k], w.dtype, valid, qbits, codes, blocks)
        torch.cuda.synchronize()
        del contrib
        torch.cuda.empty_cache()
        contrib = q
    elif rows:
        table = [torch.empty(valid, dtype=tdt, device=dev) for _ in range(w.nranks)]
        for k, r in enumerate(table):
            r.copy_(contrib[k, :valid])
        torch.cuda.synchronize()
        del contrib
        torch.cuda.empty_cache()
        contrib = table
    torch.cuda.synchronize()
    return dict(rank=rank, shard=shard, off=off, valid=valid, stride=stride, contrib=contrib,
                gather=gather, step=st, fused=fused)


def timed_steps(b, steps, warmup, torch, Z, graph=False, qg=None):
    """Warmup, then two timed passes of `steps` steps each on the same stream:
    the first with events only around the whole loop (the step time), the
    second with events also around each launch of the dominant kernel (the
    fused pass, or the Adam pass; plus the reduce pass on the two-pass path).
    Event records between kernels cost a few microseconds each, so they are
    kept out of the loop that gives the step time.  With `qg` (a QGather) the
    step writes the quantised all-gather payload instead of the 16-bit slot."""
    st, contrib, gather = b["step"], b["contrib"], b["gather"]
    slot = None if qg is not None else gather
    for _ in range(warmup):
        st.step(contrib, slot, qg)
    torch.cuda.synchronize()
    run_step = lambda: st.step(contrib, slot, qg)  # noqa: E731
    if graph:  # one captured step, replayed: the step's scalars live on the device
        g = st.capture(contrib, slot, qg)
        torch.cuda.synchronize()
        run_step = g.replay
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        run_step()
    t1.record()
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / steps
    # per-step spread: one event at each step boundary
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    bounds[0].record()
    for i in range(steps):
        run_step()
        bounds[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    ev_red = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    for i in range(steps):
        if b["fused"]:  # the fused launches (one per piece), then decision and restore
            ev[i][0].record()
            st.run_pieces(contrib, slot, qg)
            ev[i][1].record()
            st.decide()
            st.complete(slot, qg)
        else:  # the reduce launches (one per piece), the decision, then the Adam pass
            ev_red[i][0].record()
            st.run_pieces(contrib, slot, qg)
            ev_red[i][1].record()
            st.decide()
            ev[i][0].record()
            st.complete(slot, qg)
            ev[i][1].record()
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(c) for a, c in ev]
    red_ms = [a.elapsed_time(c) for a, c in ev_red] if not b["fused"] else []
    ctrl = st.ctrl_dict()
    return step_ms, per_step, kern_ms, red_ms, ctrl


def timed_skip_steps(b, w, torch, reps=3, qg=None):
    """Steps that the workload's injected +inf forces to skip (the 13B
    shard's step 2): the fused pass, the decision (skip, halve the scale) and
    the restore of the slot (or, with `qg`, of the quantised payload, with no
    16-bit slot) from the kept master, timed whole and per part with HIP
    events on the launch stream.  The contribution element is put back
    afterwards."""
    (_, k, col), = w.inject_inf
    st, contrib = b["step"], b["contrib"]
    gather = None if qg is not None else b["gather"]
    cell = contrib[k][col:col + 1] if isinstance(contrib, list) else contrib[k, col:col + 1]
    orig = cell.clone()
    cell.fill_(float("inf"))
    torch.cuda.synchronize()
    rows = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        st.run_pieces(contrib, gather, qg)
        e[1].record()
        st.decide()
        e[2].record()
        st.complete(gather, qg)
        e[3].record()
        torch.cuda.synchronize()
        c = st.ctrl_dict()
        if not c["skip"]:
            raise RuntimeError("the injected +inf did not skip the step")
        rows.append([e[0].elapsed_time(e[3]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                     c["loss_scale"]])
    cell.copy_(orig)
    torch.cuda.synchronize()
    ms, dec_ms, restore_ms, _ = sorted(rows)[len(rows) // 2]
    valid = b["valid"]
    # the kept master read, the slot or the payload (codes and one record per block) written
    rbytes = int(round(valid * (4 + (2 if qg is None else qg.bits / 8 + 8 / 2048))))
    return {"ms": _fmt(ms, 5), "decision_ms": _fmt(dec_ms, 4), "restore_ms": _fmt(restore_ms, 5),
            "restore_gbps": _fmt(rbytes / (restore_ms * 1e-3) / 1e9, 5),
            "restore_bytes": rbytes, "steps": reps,
            "loss_scales_after": [r[3] for r in rows]}


def copy_bandwidth(torch, synth, nbytes=8 << 30, reps=10):
    """Plain device copy: a reachable-bandwidth reference line."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        synth.gpu_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        synth.gpu_copy(src, dst, nbytes)
    c.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(c) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9, ms


def stream_rates(torch, synth, nbytes=8 << 30, reps=5):
    """Plain streams of 8 GiB per array on the same GPU, in the launch form
    that measured fastest for them (launches of 65,536 workgroups of 8 KiB,
    three resident per CU): reads alone, writes alone, a copy, two bytes read
    per byte written (the fused step's mix) and four (the reduce pass's mix,
    over 4 GiB written).  Reference lines for the kernels' fraction of what
    the HBM delivers to a simple stream."""
    n = nbytes // 4
    a = torch.full((n,), 0.5, dtype=torch.float32, device="cuda")
    b = torch.full((n,), 0.25, dtype=torch.float32, device="cuda")
    d = torch.empty(n, dtype=torch.float32, device="cuda")
    # bytes written per stream and bytes moved in all
    moved = {"read": (nbytes, nbytes), "write": (nbytes, nbytes), "copy": (nbytes, 2 * nbytes),
             "mix_2r1w": (nbytes, 3 * nbytes), "mix_4r1w": (nbytes // 2, 5 * nbytes // 2)}
    out = {}
    for kind, (span, total) in moved.items():
        run = lambda: synth.gpu_stream(kind, a, b, d, span, 65536, 48 * 1024)  # noqa: E731
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        out[kind] = _fmt(total / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 5)
    del a, b, d
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, sample_elems):
    """The CPU oracle, single-threaded, timed on one step of a contiguous sample
    of the same shard (inputs generated beforehand, not timed)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle as O
    import synth
    rank = w.ranks[-1]
    _, off, valid = O.partition(w.psi, w.nranks, rank)
    if len(w.ranks) > 1:  # every rank's shard: the whole buffer, element by element the same work
        off, valid = 0, w.psi
    S = min(sample_elems, valid)
    C = np.empty((w.nranks, S), np.uint16)
    chunk = 1 << 22

    def gen(i0):
        n = min(chunk, S - i0)
        part = synth.contrib_rows(w.seed, 1, w.nranks, w.dtype, w.contrib_sigma, w.contrib_scale,
                                  w.outlier_p, w.outlier_mult, off + i0, n)
        C[:, i0:i0 + n] = part

    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(gen, range(0, S, chunk)))
    p = synth.master_range(w.seed, w.master_sigma, off, S)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    hp = O.hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                   max_grad_norm=w.max_grad_norm, scaler=w.scaler, min_scale=w.min_scale,
                   growth_interval=w.growth_interval)
    st = O.new_scalars(w.loss_scale)
    t0 = time.perf_counter()
    g, flag = O.reduce(C, w.dtype, S, O.inv_scale(w.nranks, st.scale))
    rep = O.finalize(hp, st, flag, O.SumSq().add(g))
    if not rep.skip:
        O.adam(p, m, v, g, hp, rep.clip, st.pow1, st.pow2)
        O.cast(p, w.dtype)
    dt = time.perf_counter() - t0
    gbps = w.bytes_per_elem * S / dt / 1e9
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": _fmt(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one step over {S} contiguous elements of the measured "
                      f"{'buffer' if len(w.ranks) > 1 else 'shard'} "
                      f"({S / valid:.2%} of it), single-threaded C oracle, {dt:.2f} s; "
                      f"host: {cpu_model}, 1 of {os.cpu_count()} cores",
            "elements_per_s": _fmt(S / dt, 4)}


def measure(w, args, bucket, torch, synth, Z) -> dict:
    """One workload's timed steps (with the flags' contribution form, payload,
    buckets and launch) and the fields of its bench line."""
    b = setup(w, torch, synth, Z, rows=args.rows, qbits=args.quant, bucket=bucket)
    b_pieces = b["step"].pieces()
    pieces = len(b_pieces)
    row_pass_n = w.nranks if b["fused"] else 0  # the timed pass reads the N rows (fused) or not
    valid = b["valid"]
    qg = Z.QGather.alloc(valid, args.qgather, torch.device("cuda", 0)) if args.qgather else None
    ms_step, per_step, kern_ms, red_ms, ctrl = timed_steps(b, args.steps, args.warmup, torch, Z,
                                                           graph=args.graph, qg=qg)
    skip = None
    if b["fused"] and w.inject_inf and not args.quant and pieces == 1:
        skip = timed_skip_steps(b, w, torch, qg=qg)
    bpe = quant_bytes_per_elem(w, args.quant) if args.quant else w.bytes_per_elem
    if args.qgather:  # the 2-byte slot replaced by the codes and one 8-byte record per block
        bpe = bpe - 2 + args.qgather / 8 + 8 / 2048
    step_bytes = int(round(bpe * valid))
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    kern_avg = sum(kern_ms) / len(kern_ms)
    if b["fused"]:
        kern_name = ("fused_kernel_q%d" % args.quant if args.quant else
                     "fused_kernel_rows" if args.rows else "fused_kernel")
        if args.qgather:
            kern_name = ("fused_qgather_kernel_q%d" % args.qgather if kern_name == "fused_kernel"
                         else "%s_qgather%d" % (kern_name, args.qgather))
        kern_bytes = step_bytes
    elif args.qgather:
        kern_name = "adam_qgather_kernel_q%d" % args.qgather
        kern_bytes = int(round((4 + 24 + args.qgather / 8 + 8 / 2048) * valid))  # payload, no slot
    else:
        kern_name = "adam_kernel"
        kern_bytes = (4 + 26) * valid  # g + master/m/v in and out + the 16-bit slot
    kern_gbps = kern_bytes / (kern_avg * 1e-3) / 1e9
    del b, qg
    torch.cuda.empty_cache()

    out = {
        "value": _fmt(gbps, 5),
        "unit": "GB/s",
        "ms_per_step": _fmt(ms_step, 5),
        "config": {"workload": w.name, "psi": w.psi, "nranks": w.nranks, "rank": w.ranks[-1],
                   "shard_elems": valid, "variant": w.variant,
                   "contrib_dtype": "fp16" if w.dtype == Z.F16 else "bf16",
                   "bytes_per_elem": _fmt(bpe, 6), "step_bytes": step_bytes,
                   "contrib_layout": ("int%d_blocks" % args.quant if args.quant else
                                      "row_table" if args.rows else "strided"),
                   "gather_payload": ("int%d_blocks" % args.qgather if args.qgather else
                                      "16bit_slot"),
                   "bucket_elems": bucket, "calls_per_pass": pieces,
                   "launch": "hip_graph" if args.graph else "stream"},
        "step_ms_median": _fmt(per_step[len(per_step) // 2], 5),
        "step_ms_min": _fmt(per_step[0], 5),
        "pct_hbm_peak": _fmt(100 * gbps / HBM_PEAK_GBPS, 4),
        "elements_per_s": _fmt(valid / (ms_step * 1e-3), 5),
        "roofline": {"bound": "hbm", "kernel": kern_name, "achieved": _fmt(kern_gbps, 5),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": _fmt(kern_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None,
                     "kernel_ms": _fmt(kern_avg, 5), "bytes_per_pass": kern_bytes,
                     "launches_per_pass": sum(Z.launches(n, row_pass_n, payload=bool(
                         args.qgather) and row_pass_n > 0) for _, n in b_pieces)},
        "reduce_kernel": None,
        "last_step": {"norm": ctrl["norm"], "skip": ctrl["skip"], "t": ctrl["t"],
                      "loss_scale": ctrl["loss_scale"]},
    }
    # the committed counters cover the pass issued as one call
    measured = measured_traffic(kern_name, w.name) if pieces == 1 else None
    if measured is not None:
        traffic, profiled_kernel, digest = measured
        out["roofline"].update(traffic=traffic, traffic_ratio=_fmt(traffic / kern_bytes, 5),
                               traffic_kernel=profiled_kernel, traffic_isa_sha256=digest[:16])
    if red_ms:
        red_avg = sum(red_ms) / len(red_ms)
        red_bpe = 4 + (w.nranks * (args.quant / 8 + 8 / 2048) if args.quant else 2 * w.nranks)
        red_bytes = int(round(red_bpe * valid))
        out["reduce_kernel"] = {"ms": _fmt(red_avg, 5),
                                "gbps": _fmt(red_bytes / (red_avg * 1e-3) / 1e9, 5),
                                "bytes_per_pass": red_bytes}
        red = measured_traffic("reduce_kernel", w.name) if pieces == 1 and not args.quant else None
        if red is not None:
            out["reduce_kernel"].update(traffic=red[0], traffic_ratio=_fmt(red[0] / red_bytes, 5))
    if skip is not None:
        out["skip_step"] = skip
    return out


def measure_all_shards(w, args, torch, synth, Z) -> dict:
    """A workload whose every rank runs on this GPU (the toy: 32 shards of
    637,824 elements): each step is every rank's fused pass, one decision
    over all ranks' partials (standing in for the scalar all-reduce), and
    every rank's restore check.  Tiny shards: the step is launch-bound."""
    dev = torch.device("cuda", 0)
    hp = Z.hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                   max_grad_norm=w.max_grad_norm, scaler=w.scaler, min_scale=w.min_scale,
                   growth_interval=w.growth_interval)
    if w.max_grad_norm > 0:
        raise SystemExit("the all-shards bench times the fused path")
    tdt = torch.float16 if w.dtype == Z.F16 else torch.bfloat16
    steps, contribs, total = [], [], 0
    for r in w.ranks:
        _, off, valid = Z.zero_partition(w.psi, w.nranks, r)
        p0 = torch.empty(valid, dtype=torch.float32, device=dev)
        synth.gpu_master_range(p0, w.seed, w.master_sigma, off)
        stride = (valid + 63) // 64 * 64
        steps.append(Z.ShardStep(w.nranks, stride, valid, off, w.dtype, w.dtype, hp,
                                 (p0, torch.zeros_like(p0), torch.zeros_like(p0)), None,
                                 w.loss_scale))
        c = torch.empty((w.nranks, stride), dtype=tdt, device=dev)
        synth.gpu_contrib_rows(c, w.seed, 1, w.dtype, w.contrib_sigma, w.contrib_scale,
                               w.outlier_p, w.outlier_mult, off, valid)
        contribs.append(c)
        total += valid
    gather = torch.empty(w.psi, dtype=tdt, device=dev)
    synth.gpu_param_range(gather, w.seed, w.master_sigma, w.dtype, 0)
    multi = Z.MultiShardStep(steps)
    run = lambda: multi.step(contribs, gather)  # noqa: E731
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    if args.graph:
        run = multi.capture(contribs, gather).replay
        torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    a, c = ev(), ev()
    a.record()
    for _ in range(args.steps):
        run()
    c.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(c) / args.steps
    # the ranks' fused passes alone (one event pair around them: one batched
    # launch)
    kern = []
    for _ in range(args.steps):
        e0, e1 = ev(), ev()
        e0.record()
        multi.run_passes(contribs, gather)
        e1.record()
        multi.decide()
        multi.complete(contribs, gather)
        kern.append((e0, e1))
    torch.cuda.synchronize()
    kern_ms = sum(x.elapsed_time(y) for x, y in kern) / len(kern)
    ctrl = steps[0].ctrl_dict()
    step_bytes = w.bytes_per_elem * total
    gbps = step_bytes / (ms * 1e-3) / 1e9
    kgbps = step_bytes / (kern_ms * 1e-3) / 1e9
    batched = multi.takes_batched(contribs, gather)
    passes = -(-len(steps) // Z.BATCH_SHARDS) if batched else len(steps)
    launches = 2 * passes + 1
    return {
        "value": _fmt(gbps, 5),
        "unit": "GB/s",
        "ms_per_step": _fmt(ms, 5),
        "config": {"workload": w.name, "psi": w.psi, "nranks": w.nranks, "ranks": len(w.ranks),
                   "shard_elems": total // len(w.ranks), "variant": w.variant,
                   "contrib_dtype": "fp16" if w.dtype == Z.F16 else "bf16",
                   "bytes_per_elem": w.bytes_per_elem, "step_bytes": step_bytes,
                   "contrib_layout": "strided", "gather_payload": "16bit_slot",
                   "launches_per_step": launches,
                   "launch": "hip_graph" if args.graph else "stream"},
        "pct_hbm_peak": _fmt(100 * gbps / HBM_PEAK_GBPS, 4),
        "elements_per_s": _fmt(total / (ms * 1e-3), 5),
        "roofline": {"bound": "hbm", "kernel": "fused_shards_kernel" if batched else "fused_kernel",
                     "achieved": _fmt(kgbps, 5), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": _fmt(kgbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel_ms": _fmt(kern_ms, 5), "bytes_per_pass": step_bytes,
                     "launches_per_pass": passes,
                     "note": "every rank's fused pass together; each shard is about ten tiles, so "
                             "a pass is one launch over all of them (per 32 ranks), and the step "
                             "is bound by its three launches, not by HBM"},
        "last_step": {"norm": ctrl["norm"], "skip": ctrl["skip"], "t": ctrl["t"],
                      "loss_scale": ctrl["loss_scale"]},
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--quant", type=int, choices=(0, 4, 8), default=0,
                    help="block-quantised (ZeRO++) INT8 or INT4 contributions through the "
                         "quantised calls")
    ap.add_argument("--qgather", type=int, choices=(0, 4, 8), default=0,
                    help="the step writes the ZeRO++ INT8 or INT4 all-gather payload of the new "
                         "parameters instead of the 16-bit slot")
    ap.add_argument("--bucket", type=int, default=0,
                    help="the shard's gradient arrives in pieces of this many elements (rounded "
                         "down to a multiple of 2048), each reduced or stepped by its own launch; "
                         "the pages' reduce_bucket_size is 5e8")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as one captured HIP graph replayed each step")
    ap.add_argument("--rows", action="store_true",
                    help="contribution rows in N separate allocations, through the row-table "
                         "calls (one pointer per row) instead of one [N, stride] buffer")
    ap.add_argument("--cpu-sample", type=int, default=160 << 20,
                    help="elements of the shard the CPU oracle baseline steps over")
    ap.add_argument("--cpu-full", action="store_true",
                    help="the CPU oracle baseline steps over the whole shard (13B: about two "
                         "minutes single-threaded and 46 GB of host memory)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true")
    ap.add_argument("--no-7b", action="store_true",
                    help="leave out the 7B two-pass line that the default run appends as 'c4'")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only the plain copy kernel (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one rank's shard step on ONE GPU; the library has no multi-GPU "
              "path (collectives between GPUs are outside it). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import zero_partitioned_mixed_amd as Z
    from synth import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    if args.copy_only:
        gbps, ms = copy_bandwidth(torch, synth)
        print(json.dumps({"copy_gbps": _fmt(gbps, 4), "copy_ms": _fmt(ms, 4), "bytes": 2 * (8 << 30)}))
        return

    w = workloads.BY_NAME[args.workload]
    bucket = args.bucket // Z.TILE * Z.TILE
    if args.bucket and not bucket:
        print("--bucket must be at least 2048 elements", file=sys.stderr)
        sys.exit(2)
    if len(w.ranks) > 1:  # every rank of the workload on this GPU (the toy)
        if args.quant or args.qgather or bucket or args.rows:
            print("the all-shards workload is timed with the plain fused step only", file=sys.stderr)
            sys.exit(2)
        head = measure_all_shards(w, args, torch, synth, Z)
    else:
        head = measure(w, args, bucket, torch, synth, Z)
    out = {
        "metric": METRIC,
        "value": head.pop("value"),
        "unit": head.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
    }
    out.update(head)
    plain = not (args.quant or args.qgather or bucket or args.graph or args.rows)
    if args.workload == DEFAULT_WORKLOAD and plain and not args.no_7b:
        # the 7B shard (clipping on, so the two-pass path), measured in the
        # same run after the 13B buffers are freed
        c4 = measure(workloads.P7B, args, 0, torch, synth, Z)
        out["c4"] = {key: c4[key] for key in ("value", "unit", "ms_per_step", "pct_hbm_peak",
                                             "step_ms_median", "step_ms_min", "elements_per_s",
                                             "config", "roofline", "reduce_kernel", "last_step")}
    try:
        out["device"] = synth.gpu_device_info(0)
    except (RuntimeError, OSError, AttributeError) as e:  # informational only
        out["device"] = {"error": str(e)}
    if not args.no_copy:
        cg, _ = copy_bandwidth(torch, synth)
        out["copy_gbps"] = _fmt(cg, 5)
        out["pct_of_copy"] = _fmt(100 * out["value"] / cg, 4)
        out["stream_gbps"] = stream_rates(torch, synth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, (1 << 62) if args.cpu_full else args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
