"""Shared driver for the GPU parity tests: the same seeded workload run through
the C ABI on the GPU and through the CPU oracle, then compared.

Inputs come only from the seeded generator (``synth``): the GPU side fills
HBM with the device build, the oracle side draws exactly the elements it
needs with the host build.  Nothing the GPU computes is fed to the oracle.

Oracle side, for one rank of a workload:
  scalar pass   every step over the whole shard (chunked, threads; the
                squared norm is exact, so chunking cannot change it) ->
                per-step skip / clip / loss scale / bias-correction powers;
  element pass  the per-element step sequence for a set of shard positions
                (the whole shard, or a sample at full size).
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

import oracle as O
import synth
from synth.workloads import BF16, F16, Workload

# Bars.  The graded ones: fp32 |d| <= 1e-6 |x| + 1e-9, 16-bit within 1 ulp,
# norm within 1e-5 relative, flags and decisions exact.  The 1e-9 floor makes
# the fp32 bar nearly vacuous for v (about 1e-10 after one step of a 1e-3
# gradient), so every fp32 array must also lie within F32_ULPS units in the
# last place of the oracle's, with no floor.  And the path is built to agree
# with the oracle operation for operation, so the comparisons also require
# equal bits unless a caller says otherwise (a clip coefficient formed from
# a GPU norm one fp64 rounding away from the oracle's may move g by an ulp).
F32_RTOL = 1e-6
F32_ATOL = 1e-9
F32_ULPS = 4
NORM_RTOL = 1e-5
THREADS = max(1, min(16, os.cpu_count() or 1))
CHUNK = 1 << 20
assert CHUNK % O.QBLOCK == 0  # oracle chunks start quantisation blocks


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@dataclass(frozen=True)
class Inject:
    step: int
    k: int
    col: int        # column in the shard's contribution row (>= valid_len: padding)
    value: float    # written in the contribution dtype


@dataclass(frozen=True)
class Case:
    w: Workload
    rank: int
    steps: int
    extra: tuple = ()          # Inject entries on top of the workload's own
    stride_pad: int = 0        # extra padding columns beyond the workload stride
    qbits: int = 0             # 8 or 4: contributions arrive block-quantised (ZeRO++)

    @property
    def part(self):
        return O.partition(self.w.psi, self.w.nranks, self.rank)

    @property
    def stride(self):
        shard = self.part[0]
        return (shard + 63) // 64 * 64 + self.stride_pad

    @property
    def injections(self):
        own = tuple(Inject(s, k, i, float("inf")) for (s, k, i) in self.w.inject_inf)
        return own + tuple(self.extra)


def o_hparams(w: Workload):
    return O.hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                     max_grad_norm=w.max_grad_norm, scaler=w.scaler, min_scale=w.min_scale,
                     growth_interval=w.growth_interval)


def bits16(value: float, dtype: int) -> int:
    return int(O.from_f32(np.array([value], np.float32), dtype)[0])


# ----------------------------------------------------------------------------- oracle side
def _contrib_chunk(c: Case, step: int, col0: int, ncol: int) -> np.ndarray:
    w = c.w
    _, off, _ = c.part
    C = synth.contrib_rows(w.seed, step, w.nranks, w.dtype, w.contrib_sigma, w.contrib_scale,
                           w.outlier_p, w.outlier_mult, off + col0, ncol)
    for inj in c.injections:
        if inj.step == step and col0 <= inj.col < col0 + ncol:
            C[inj.k, inj.col - col0] = bits16(inj.value, w.dtype)
    return C


def _reduce(c: Case, C: np.ndarray, ncol: int, inv: float):
    """The oracle's reduce of a contribution chunk whose first column starts a
    quantisation block: plain, or over the rows block-quantised by the oracle."""
    if not c.qbits:
        return O.reduce(C, c.w.dtype, ncol, inv)
    rows = [O.quantize(C[k, :ncol], c.w.dtype, c.qbits) for k in range(C.shape[0])]
    return O.reduce_q(rows, ncol, inv)


def oracle_scalars(c: Case) -> list[dict]:
    """Per-step decisions of the oracle over the whole shard."""
    w = c.w
    _, _, valid = c.part
    hp = o_hparams(w)
    st = O.new_scalars(w.loss_scale)
    chunks = [(i, min(CHUNK, valid - i)) for i in range(0, valid, CHUNK)]
    out = []
    with ThreadPoolExecutor(THREADS) as ex:
        for s in range(1, c.steps + 1):
            inv = O.inv_scale(w.nranks, st.scale)

            def work(ch, s=s, inv=inv):
                C = _contrib_chunk(c, s, ch[0], ch[1])
                g, flag = _reduce(c, C, ch[1], inv)
                return O.SumSq().add(g), flag

            acc, flag = O.SumSq(), 0
            for a, f in ex.map(work, chunks):
                acc.merge(a)
                flag |= f
            rep = O.finalize(hp, st, flag, acc).as_dict()
            rep.update(inv=inv, pow1=st.pow1, pow2=st.pow2, t=st.t, scale_next=st.scale)
            out.append(rep)
            if valid * w.nranks > (1 << 28):
                log(f"oracle scalars step {s}: norm {rep['norm']:.9g} skip {rep['skip']}")
    return out


def _elements(c: Case, reps: list[dict], cols: np.ndarray | None, col0: int = 0, ncol: int = 0):
    """master, m, v after all steps for shard columns `cols` (or the range)."""
    w = c.w
    _, off, _ = c.part
    hp = o_hparams(w)
    if cols is None:
        p = synth.master_range(w.seed, w.master_sigma, off + col0, ncol)
    else:
        p = synth.master_at(w.seed, w.master_sigma, off + cols)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    for s, rep in enumerate(reps, 1):
        if rep["skip"]:
            continue
        if cols is None:
            C = _contrib_chunk(c, s, col0, ncol)
        elif c.qbits:  # whole quantisation blocks around the sampled columns
            g = np.empty(cols.size, np.float32)
            blk = cols // O.QBLOCK
            for b in np.unique(blk):
                b0 = int(b) * O.QBLOCK
                nb = min(O.QBLOCK, c.part[2] - b0)
                gb, _ = _reduce(c, _contrib_chunk(c, s, b0, nb), nb, rep["inv"])
                g[blk == b] = gb[cols[blk == b] - b0]
            O.adam(p, m, v, g, hp, rep["clip"], rep["pow1"], rep["pow2"])
            continue
        else:
            C = synth.contrib_at(w.seed, s, w.nranks, w.dtype, w.contrib_sigma, w.contrib_scale,
                                 w.outlier_p, w.outlier_mult, off + cols)
            for inj in c.injections:
                if inj.step == s:
                    C[inj.k, cols == inj.col] = bits16(inj.value, w.dtype)
        g, _ = _reduce(c, np.ascontiguousarray(C), p.size, rep["inv"])
        O.adam(p, m, v, g, hp, rep["clip"], rep["pow1"], rep["pow2"])
    return p, m, v


def oracle_elements(c: Case, reps: list[dict], cols: np.ndarray | None = None):
    """(master, m, v, slot bits) of the oracle at `cols` (whole shard if None)."""
    w = c.w
    _, off, valid = c.part
    if cols is not None:
        p, m, v = _elements(c, reps, cols)
        idx = off + cols
    else:
        chunks = [(i, min(CHUNK, valid - i)) for i in range(0, valid, CHUNK)]
        with ThreadPoolExecutor(THREADS) as ex:
            parts = list(ex.map(lambda ch: _elements(c, reps, None, ch[0], ch[1]), chunks))
        p = np.concatenate([x[0] for x in parts]) if parts else np.zeros(0, np.float32)
        m = np.concatenate([x[1] for x in parts]) if parts else np.zeros(0, np.float32)
        v = np.concatenate([x[2] for x in parts]) if parts else np.zeros(0, np.float32)
        idx = None
    if any(not r["skip"] for r in reps):
        slot = O.cast(p, w.slot_dtype)
    elif idx is not None:  # never applied: the initial 16-bit parameters
        slot = O.cast(synth.master_at(w.seed, w.master_sigma, idx), w.slot_dtype)
    else:
        slot = O.cast(synth.master_range(w.seed, w.master_sigma, off, valid), w.slot_dtype)
    return p, m, v, slot


# ----------------------------------------------------------------------------- GPU side
ROW_LAYOUTS = ("strided", "rows", "rows_shifted")


class DeviceRun:
    """One rank's buffers in HBM and its steps through the C ABI.

    layout: how the contribution rows are handed to the library.
      strided       one [N, stride] buffer (zero_fused_step / zero_reduce_grads);
      rows          N separate allocations, one pointer per row (the *_rows calls);
      rows_shifted  N rows packed in one buffer at 8-byte but not 16-byte
                    aligned starts (as a peer's slice at an odd multiple of
                    four elements would be), through the *_rows calls.
    The row copies are filled from the strided buffer, so all three hand the
    library the same values."""

    def __init__(self, c: Case, full_gather: bool = True, layout: str = "strided",
                 qgather: int = 0, write_slot: bool = True, bucket: int = 0):
        import torch
        import zero_partitioned_mixed_amd as Z
        self.c, self.Z, self.torch = c, Z, torch
        w = c.w
        shard, off, valid = c.part
        self.shard, self.off, self.valid = shard, off, valid
        dev = torch.device("cuda", 0)
        tdt = torch.float16 if w.dtype == F16 else torch.bfloat16
        self.tdt = tdt
        self.contrib = torch.empty((w.nranks, c.stride), dtype=tdt, device=dev)
        n_state = max(valid, 1)
        p0 = torch.empty(n_state, dtype=torch.float32, device=dev)
        synth.gpu_master_range(p0, w.seed, w.master_sigma, off)
        z = lambda: torch.zeros(n_state, dtype=torch.float32, device=dev)
        self.state0 = (p0, z(), z())
        fused = w.max_grad_norm <= 0
        self.g = None if fused else torch.empty(n_state, dtype=torch.float32, device=dev)
        self.gather_len = w.psi if full_gather else valid
        self.gather_off = off if full_gather else 0
        gdt = torch.float16 if w.slot_dtype == F16 else torch.bfloat16
        self.gather = torch.empty(max(self.gather_len, 1), dtype=gdt, device=dev)
        synth.gpu_param_range(self.gather, w.seed, w.master_sigma, w.slot_dtype,
                              0 if full_gather else off)
        hp = Z.hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                       weight_decay=w.weight_decay, max_grad_norm=w.max_grad_norm,
                       scaler=w.scaler, min_scale=w.min_scale, growth_interval=w.growth_interval)
        self.step_obj = Z.ShardStep(w.nranks, c.stride, valid, self.gather_off, w.dtype,
                                    w.slot_dtype, hp, self.state0, self.g, w.loss_scale,
                                    bucket=bucket)
        self.reports = []
        if layout not in ROW_LAYOUTS:
            raise ValueError(layout)
        self.layout = layout
        self.rows = None
        self.qrows = None
        # qgather = 8 or 4: the step also writes the quantised all-gather
        # payload (zero_fused_step_qgather); write_slot=False passes no gather
        self.qg = Z.QGather.alloc(valid, qgather, dev) if qgather else None
        if self.qg is not None and fused:
            # canaries: the step or the restore writes every code byte and record
            self.qg.codes.fill_(0xA5)
            self.qg.blocks.fill_(0xA5)
        elif self.qg is not None and valid:
            # the two-pass path writes nothing on a skipped step, so the payload
            # starts as the caller's would: the initial slot, quantised
            Z.zero_quantize_blocks(self.gather[self.gather_off:], w.slot_dtype, valid, qgather,
                                   self.qg.codes, self.qg.blocks)
        self.write_slot = write_slot
        if not write_slot and not qgather and fused:
            raise ValueError("the fused step without a payload writes the 16-bit slot")
        n = w.nranks
        if c.qbits:
            self.qrows = Z.QuantRows.alloc(n, valid, c.qbits, dev)
        if layout == "rows":
            self.rows = [torch.empty(max(valid, 1), dtype=tdt, device=dev) for _ in range(n)]
        elif layout == "rows_shifted":
            span = (valid + 7) // 8 * 8 + 8          # a multiple of 8 elements
            self.row_buf = torch.empty(4 + n * span, dtype=tdt, device=dev)
            self.rows = [self.row_buf[4 + k * span:4 + k * span + max(valid, 1)] for k in range(n)]
            for r in self.rows:
                assert r.data_ptr() % 8 == 0 and r.data_ptr() % 16 == 8

    def fill(self, step: int) -> None:
        w, c = self.c.w, self.c
        synth.gpu_contrib_rows(self.contrib, w.seed, step, w.dtype, w.contrib_sigma,
                               w.contrib_scale, w.outlier_p, w.outlier_mult, self.off, self.valid)
        for inj in c.injections:
            if inj.step == step:
                self.contrib[inj.k, inj.col] = inj.value
        if self.rows is not None and self.valid:
            for k, r in enumerate(self.rows):
                r[:self.valid].copy_(self.contrib[k, :self.valid])
        if self.qrows is not None and self.valid:
            for k, (codes, blocks) in enumerate(self.qrows.rows):
                self.Z.zero_quantize_blocks(self.contrib[k], w.dtype, self.valid, c.qbits, codes,
                                            blocks)

    def run(self, steps: int | None = None, record: bool = True) -> None:
        steps = self.c.steps if steps is None else steps
        for s in range(1, steps + 1):
            self.fill(s)
            src = self.qrows if self.qrows is not None else (
                self.contrib if self.rows is None else self.rows)
            self.step_obj.step(src, self.gather if self.write_slot else None, self.qg)
            if record:
                self.reports.append(self.step_obj.ctrl_dict())
        self.torch.cuda.synchronize()

    def current(self):
        return self.step_obj.current()

    def fetch(self, cols: np.ndarray | None = None):
        """(master, m, v, slot bits) at shard columns `cols` (all if None)."""
        torch = self.torch
        st = self.current()
        if cols is None:
            sl = slice(0, self.valid)
            out = [t[sl].cpu().numpy() for t in st]
            slot = self.gather[self.gather_off:self.gather_off + self.valid]
        else:
            ix = torch.from_numpy(cols.astype(np.int64)).to(st[0].device)
            out = [t.index_select(0, ix).cpu().numpy() for t in st]
            slot = self.gather.index_select(0, ix + self.gather_off)
        slot = slot.view(torch.int16).cpu().numpy().view(np.uint16)
        return out[0], out[1], out[2], slot

    def qpayload(self):
        """(codes, scales, zero points) of the quantised all-gather payload."""
        q = self.qg
        nblk = (self.valid + O.QBLOCK - 1) // O.QBLOCK
        codes = q.codes.cpu().numpy()[:O.qcode_bytes(self.valid, q.bits)]
        rec = q.blocks.cpu().numpy().view(np.uint8)[:8 * nblk]
        return codes, rec.view(np.float32)[0::2], rec.view(np.int32)[1::2]

    def gather_bits(self, idx: np.ndarray) -> np.ndarray:
        torch = self.torch
        ix = torch.from_numpy(idx.astype(np.int64)).to(self.gather.device)
        return self.gather.index_select(0, ix).view(torch.int16).cpu().numpy().view(np.uint16)


def run_and_compare(c: Case, label: str, full: bool = True, layout: str = "strided",
                    qgather: int = 0, write_slot: bool = True, bucket: int = 0):
    """Runs case `c` on the GPU and checks every step's decisions and the final
    master/m/v/slot of the whole shard against the oracle; with `full`, also
    that the gather buffer is unchanged outside the slot.  With `qgather`, the
    quantised all-gather payload must equal, bit for bit, the oracle's
    quantisation of the oracle's final slot; without `write_slot`, the whole
    gather buffer must be unchanged."""
    log(f"{label}: psi={c.w.psi} N={c.w.nranks} rank={c.rank} dtype={c.w.dtype} "
        f"variant={c.w.variant} steps={c.steps} offset={c.part[1]} valid={c.part[2]} "
        f"layout={layout} qbits={c.qbits} qgather={qgather} write_slot={write_slot} "
        f"bucket={bucket}")
    g = DeviceRun(c, full_gather=full, layout=layout, qgather=qgather, write_slot=write_slot,
               bucket=bucket)
    g.run()
    ref_reps = oracle_scalars(c)
    stats = assert_reports(g.reports, ref_reps)
    exact = same_clips(g.reports, ref_reps)
    p, m, v, slot = g.fetch()
    rp, rm, rv, rslot = oracle_elements(c, ref_reps)
    stats["master"] = assert_f32_close("master", p, rp, exact)
    stats["m"] = assert_f32_close("m", m, rm, exact)
    stats["v"] = assert_f32_close("v", v, rv, exact)
    if write_slot:
        stats["slot"] = assert_16bit_within_ulp("slot", slot, rslot, c.w.slot_dtype, exact)
    if qgather:
        stats["qgather"] = assert_qpayload(g.qpayload(),
                                           O.quantize(rslot, c.w.slot_dtype, qgather))
    w = c.w
    _, off, valid = c.part
    if full:  # nothing outside the slot changed (nothing at all without a slot)
        outside = np.r_[0:off, off + valid:w.psi] if write_slot else np.arange(w.psi)
        if outside.size:
            got = g.gather_bits(outside)
            ref = synth.param_range(w.seed, w.master_sigma, w.slot_dtype, 0, w.psi)[outside]
            assert np.array_equal(got, ref), "gather buffer changed outside the slot"
    log(f"{label}: ok {stats}")
    return g, stats


def assert_qpayload(got, ref) -> dict:
    """Codes, scales (as bits) and zero points equal."""
    codes, scale, zero = got
    assert np.array_equal(codes, ref.codes[:O.qcode_bytes(ref.length, ref.bits)]), "codes differ"
    assert np.array_equal(scale.view(np.uint32), ref.scale.view(np.uint32)), "scales differ"
    assert np.array_equal(zero, ref.zero), "zero points differ"
    return {"blocks": int(ref.scale.size), "nan_blocks": int(np.isnan(ref.scale).sum())}


# ----------------------------------------------------------------------------- comparisons
def ordinal32(x: np.ndarray) -> np.ndarray:
    """fp32 values as integers ordered like the values (adjacent floats differ
    by 1; +0 and -0 both map to 0)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, -(b & 0x7FFFFFFF), b)


def ulps32(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    return np.abs(ordinal32(got) - ordinal32(ref))


def assert_f32_close(name: str, got: np.ndarray, ref: np.ndarray, exact: bool = True) -> dict:
    """The graded bar (1e-6 |x| + 1e-9), at most F32_ULPS ulps with no floor,
    NaN where and only where the oracle has NaN, and, with `exact`, equal bits."""
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    got64, ref64 = got.astype(np.float64), ref.astype(np.float64)
    gnan, rnan = np.isnan(got64), np.isnan(ref64)
    if (gnan != rnan).any():
        i = int(np.flatnonzero(gnan != rnan)[0])
        raise AssertionError(f"{name}: NaN at {i} on one side only: gpu {got[i]!r} oracle {ref[i]!r}")
    both_nan = gnan & rnan
    d = np.abs(got64 - ref64)
    bad = ~both_nan & ~(d <= F32_RTOL * np.abs(ref64) + F32_ATOL)
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {got.size} outside the bar; first at "
                             f"{i}: gpu {got[i]!r} oracle {ref[i]!r}")
    u = np.where(both_nan, 0, ulps32(got, ref))
    if (u > F32_ULPS).any():
        i = int(np.argmax(u))
        raise AssertionError(f"{name}: {int((u > F32_ULPS).sum())} of {got.size} more than "
                             f"{F32_ULPS} ulps apart; worst at {i}: gpu {got[i]!r} oracle {ref[i]!r}")
    same = (got.view(np.uint32) == ref.view(np.uint32)) | both_nan
    if exact and not same.all():
        i = int(np.flatnonzero(~same)[0])
        raise AssertionError(f"{name}: {int((~same).sum())} of {got.size} differ in their bits; "
                             f"first at {i}: gpu {got[i]!r} oracle {ref[i]!r}")
    return {"bit_exact_frac": float(same.mean()) if got.size else 1.0,
            "max_ulps": int(u.max()) if got.size else 0,
            "max_abs": float(d[~both_nan].max()) if (~both_nan).any() else 0.0}


def _ordinal16(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _isnan16(b: np.ndarray, dtype: int) -> np.ndarray:
    b = b.astype(np.uint32)
    exp, man = (0x7C00, 0x03FF) if dtype == F16 else (0x7F80, 0x007F)
    return ((b & exp) == exp) & ((b & man) != 0)


def assert_16bit_within_ulp(name: str, got: np.ndarray, ref: np.ndarray, dtype: int,
                            exact: bool = True) -> dict:
    """Within 1 ulp (the graded bar) and, with `exact`, equal bits.  NaN must
    stand where and only where the oracle has NaN, with any sign and payload:
    IEEE 754 fixes neither for the NaN an invalid operation makes (0/0 gives
    the negative default NaN on the host's SSE units and the positive one on
    the GPU), as in the fp32 comparisons."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    gnan, rnan = _isnan16(got, dtype), _isnan16(ref, dtype)
    if (gnan != rnan).any():
        i = int(np.flatnonzero(gnan != rnan)[0])
        raise AssertionError(f"{name}: NaN at {i} on one side only: gpu {got[i]:#06x} "
                             f"oracle {ref[i]:#06x}")
    both_nan = gnan & rnan
    d = np.where(both_nan, 0, np.abs(_ordinal16(got) - _ordinal16(ref)))
    bad = d > 1
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} of {got.size} more than 1 ulp apart; "
                             f"first at {i}: gpu {got[i]:#06x} oracle {ref[i]:#06x}")
    same = (got.astype(np.uint16) == ref.astype(np.uint16)) | both_nan
    if exact and not same.all():
        i = int(np.flatnonzero(~same)[0])
        raise AssertionError(f"{name}: {int((~same).sum())} of {got.size} differ in their bits; "
                             f"first at {i}: gpu {got[i]:#06x} oracle {ref[i]:#06x}")
    return {"bit_exact_frac": float(same.mean()) if got.size else 1.0}


def same_clips(gpu: list[dict], ref: list[dict]) -> bool:
    """Whether every applied step used the oracle's clip coefficient bit for
    bit; then master, m, v and the slot must be bit-identical too."""
    return all(r["skip"] or np.float32(g["clip"]) == np.float32(r["clip"]) for g, r in zip(gpu, ref))


def assert_reports(gpu: list[dict], ref: list[dict]) -> dict:
    assert len(gpu) == len(ref)
    worst = 0.0
    for s, (g, r) in enumerate(zip(gpu, ref), 1):
        for key in ("nonfinite", "skip"):
            assert g[key] == r[key], (s, key, g[key], r[key])
        assert g["t"] == r["t"], (s, "t", g["t"], r["t"])
        assert g["scale_used"] == r["scale_used"], (s, "scale", g["scale_used"], r["scale_used"])
        assert g["loss_scale"] == r["scale_next"], (s, "next scale")
        if np.isfinite(r["norm"]):
            rel = abs(g["norm"] - r["norm"]) / max(r["norm"], 1e-300)
            assert rel <= NORM_RTOL, (s, "norm", g["norm"], r["norm"])
            worst = max(worst, rel)
            if not r["skip"]:
                assert g["clip"] == r["clip"] or abs(g["clip"] - r["clip"]) <= 2 ** -23 * r["clip"], (
                    s, "clip", g["clip"], r["clip"])
        else:
            assert np.isnan(g["norm"]) == np.isnan(r["norm"]) and not np.isfinite(g["norm"]), (s, "norm")
        assert g["beta1_pow"] == r["pow1"] and g["beta2_pow"] == r["pow2"], (s, "beta powers")
    return {"norm_max_rel": worst}


def sample_cols(valid: int, count: int, seed: int, extra=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    head = np.arange(min(valid, 1024))
    tail = np.arange(max(0, valid - 1024), valid)
    rnd = rng.integers(0, valid, size=count) if valid else np.zeros(0, np.int64)
    ex = np.array([e for e in extra if 0 <= e < valid], np.int64)
    return np.unique(np.concatenate([head, tail, rnd, ex]).astype(np.int64))
