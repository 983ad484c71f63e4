"""CPU oracle for the ZeRO per-rank shard step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain, slow,
single-threaded C) with ctypes and adds the multi-rank orchestration the
ZeRO pages describe (one shard per rank, global norm and overflow over all
ranks).  It shares no code with the GPU library.

Parity unpinned: Adam trajectories beyond the closed forms and the library
cross-check exercised by the tests (the pages print none).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

F16 = 1
BF16 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=gnu11", "-fPIC", "-shared",
             "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


class Hparams(ctypes.Structure):
    """Adam(W), clipping and loss-scaler settings (mirrors ``oracle_hparams``)."""

    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("max_grad_norm", ctypes.c_float), ("scaler", ctypes.c_int32),
                ("min_scale", ctypes.c_float), ("growth_interval", ctypes.c_int32)]


class Scalars(ctypes.Structure):
    """Per-run scalars carried between steps (mirrors ``oracle_scalars``)."""

    _fields_ = [("pow1", ctypes.c_double), ("pow2", ctypes.c_double), ("scale", ctypes.c_float),
                ("good", ctypes.c_int32), ("t", ctypes.c_int32), ("pad", ctypes.c_int32)]


class Report(ctypes.Structure):
    """What one step decided (mirrors ``oracle_report``)."""

    _fields_ = [("sumsq", ctypes.c_double), ("norm", ctypes.c_double),
                ("scale_used", ctypes.c_float), ("clip", ctypes.c_float),
                ("nonfinite", ctypes.c_int32), ("skip", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


class _SumSqC(ctypes.Structure):
    _fields_ = [("limb", ctypes.c_uint64 * 10), ("has_nan", ctypes.c_int32),
                ("has_inf", ctypes.c_int32)]


_lib = None


def lib():
    """The oracle library (``ORACLE_LIB`` may name another build of oracle.c:
    the mutation tests use it to run the pins against planted mistakes)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB", _LIB)
        if path == _LIB and not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(path)
        L.oracle_to_f32.restype = ctypes.c_float
        L.oracle_to_f32.argtypes = [ctypes.c_uint16, ctypes.c_int32]
        L.oracle_from_f32.restype = ctypes.c_uint16
        L.oracle_from_f32.argtypes = [ctypes.c_float, ctypes.c_int32]
        L.oracle_to_f32_array.argtypes = [_u16p, ctypes.c_int64, ctypes.c_int32, _f32p]
        L.oracle_from_f32_array.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, _u16p]
        L.oracle_from_f32_bits_range.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_int32,
                                                 _u16p]
        L.oracle_partition.restype = ctypes.c_int
        L.oracle_partition.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _i64p,
                                       _i64p, _i64p]
        L.oracle_inv_scale.restype = ctypes.c_float
        L.oracle_inv_scale.argtypes = [ctypes.c_int32, ctypes.c_float]
        L.oracle_reduce.argtypes = [_u16p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_float, _f32p, _i32p]
        L.oracle_sumsq_clear.argtypes = [ctypes.POINTER(_SumSqC)]
        L.oracle_sumsq_add.argtypes = [ctypes.POINTER(_SumSqC), _f32p, ctypes.c_int64]
        L.oracle_sumsq_merge.argtypes = [ctypes.POINTER(_SumSqC), ctypes.POINTER(_SumSqC)]
        L.oracle_sumsq_value.restype = ctypes.c_double
        L.oracle_sumsq_value.argtypes = [ctypes.POINTER(_SumSqC)]
        L.oracle_scalars_init.argtypes = [ctypes.POINTER(Scalars), ctypes.c_float]
        L.oracle_finalize.argtypes = [ctypes.POINTER(Hparams), ctypes.POINTER(Scalars),
                                      ctypes.c_int32, ctypes.POINTER(_SumSqC),
                                      ctypes.POINTER(Report)]
        L.oracle_adam.argtypes = [_f32p, _f32p, _f32p, _f32p, ctypes.c_int64,
                                  ctypes.POINTER(Hparams), ctypes.c_float, ctypes.c_double,
                                  ctypes.c_double]
        L.oracle_cast.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, _u16p]
        _u8p = ctypes.POINTER(ctypes.c_uint8)
        L.oracle_qblock.restype = ctypes.c_int64
        L.oracle_qblock.argtypes = []
        L.oracle_quantize.argtypes = [_u16p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _u8p,
                                      _f32p, _i32p]
        L.oracle_dequantize.argtypes = [_u8p, _f32p, _i32p, ctypes.c_int32, ctypes.c_int64, _f32p]
        L.oracle_reduce_q.argtypes = [ctypes.POINTER(_u8p), ctypes.POINTER(_f32p),
                                      ctypes.POINTER(_i32p), ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int64, ctypes.c_float, _f32p, _i32p]
        _lib = L
    return _lib


def _p(a: np.ndarray, ptype):
    return a.ctypes.data_as(ptype)


def _need(a: np.ndarray, dtype) -> np.ndarray:
    if a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"expected C-contiguous {np.dtype(dtype)} array, got {a.dtype}")
    return a


# --------------------------------------------------------------------------- conversions
def to_f32(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_to_f32_array(_p(bits, _u16p), bits.size, dtype, _p(out, _f32p))
    return out


def from_f32(values: np.ndarray, dtype: int) -> np.ndarray:
    values = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(values.shape, np.uint16)
    lib().oracle_from_f32_array(_p(values, _f32p), values.size, dtype, _p(out, _u16p))
    return out


def from_f32_bits_range(b0: int, n: int, dtype: int, out: np.ndarray | None = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, np.uint16)
    lib().oracle_from_f32_bits_range(b0, n, dtype, _p(out, _u16p))
    return out


# --------------------------------------------------------------------------- the step pieces
def partition(psi: int, nranks: int, rank: int) -> tuple[int, int, int]:
    """(shard length, offset, valid length) of rank ``rank``."""
    s, o, v = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib().oracle_partition(psi, nranks, rank, ctypes.byref(s), ctypes.byref(o),
                                ctypes.byref(v))
    if rc != 0:
        raise ValueError(f"invalid partition request psi={psi} N={nranks} r={rank}")
    return s.value, o.value, v.value


def inv_scale(nranks: int, loss_scale: float) -> float:
    return lib().oracle_inv_scale(nranks, loss_scale)


def reduce(C: np.ndarray, dtype: int, valid: int, inv: float) -> tuple[np.ndarray, int]:
    """Sum the rows of ``C`` ([n, stride] 16-bit patterns) in fp32 and multiply by ``inv``."""
    _need(C, np.uint16)
    n, stride = C.shape
    g = np.empty(valid, np.float32)
    flag = ctypes.c_int32()
    lib().oracle_reduce(_p(C, _u16p), dtype, n, stride, valid, inv, _p(g, _f32p),
                        ctypes.byref(flag))
    return g, int(flag.value)


class SumSq:
    """Exact sum of squares of binary32 values (order independent)."""

    def __init__(self):
        self._c = _SumSqC()
        lib().oracle_sumsq_clear(ctypes.byref(self._c))

    def add(self, g: np.ndarray) -> "SumSq":
        g = _need(np.ascontiguousarray(g), np.float32)
        lib().oracle_sumsq_add(ctypes.byref(self._c), _p(g, _f32p), g.size)
        return self

    def merge(self, other: "SumSq") -> "SumSq":
        lib().oracle_sumsq_merge(ctypes.byref(self._c), ctypes.byref(other._c))
        return self

    def value(self) -> float:
        return lib().oracle_sumsq_value(ctypes.byref(self._c))

    def limbs(self) -> tuple:
        return tuple(self._c.limb) + (self._c.has_nan, self._c.has_inf)


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.0,
            scaler=0, min_scale=1.0, growth_interval=1000) -> Hparams:
    return Hparams(lr, beta1, beta2, eps, weight_decay, max_grad_norm, scaler, min_scale,
                   growth_interval)


def new_scalars(loss_scale: float) -> Scalars:
    st = Scalars()
    lib().oracle_scalars_init(ctypes.byref(st), loss_scale)
    return st


def finalize(hp: Hparams, st: Scalars, nonfinite: int, acc: SumSq) -> Report:
    rep = Report()
    lib().oracle_finalize(ctypes.byref(hp), ctypes.byref(st), int(bool(nonfinite)),
                          ctypes.byref(acc._c), ctypes.byref(rep))
    return rep


def adam(p: np.ndarray, m: np.ndarray, v: np.ndarray, g: np.ndarray, hp: Hparams, clip: float,
         pow1: float, pow2: float) -> None:
    """In-place Adam(W) on binary32 arrays of equal length."""
    for a in (p, m, v, g):
        _need(a, np.float32)
    n = p.size
    assert m.size == n and v.size == n and g.size == n
    lib().oracle_adam(_p(p, _f32p), _p(m, _f32p), _p(v, _f32p), _p(g, _f32p), n,
                      ctypes.byref(hp), clip, pow1, pow2)


def cast(p: np.ndarray, dtype: int) -> np.ndarray:
    _need(p, np.float32)
    out = np.empty(p.size, np.uint16)
    lib().oracle_cast(_p(p, _f32p), p.size, dtype, _p(out, _u16p))
    return out


# --------------------------------------------------------------------------- block quantisation
QBLOCK = 2048  # the reading's block size; the library reports its own in qblock()
_u8p = ctypes.POINTER(ctypes.c_uint8)


def qblock() -> int:
    """Elements per quantisation block, as the oracle library defines it."""
    return int(lib().oracle_qblock())


@dataclass
class QBuffer:
    """A block-quantised buffer: packed codes, one (scale, zero) per block."""
    codes: np.ndarray   # uint8: len bytes (8 bits) or ceil(len/2) (4 bits)
    scale: np.ndarray   # float32, one per 2048-element block
    zero: np.ndarray    # int32, one per block
    bits: int
    length: int


def qcode_bytes(length: int, bits: int) -> int:
    return length if bits == 8 else (length + 1) // 2


def quantize(src: np.ndarray, dtype: int, bits: int) -> QBuffer:
    """Block-quantise 16-bit patterns ``src`` to INT8 or INT4 codes."""
    assert bits in (4, 8)
    src = _need(np.ascontiguousarray(src), np.uint16)
    n = src.size
    nblk = (n + qblock() - 1) // qblock()
    codes = np.zeros(max(qcode_bytes(n, bits), 1), np.uint8)
    scale = np.zeros(max(nblk, 1), np.float32)
    zero = np.zeros(max(nblk, 1), np.int32)
    lib().oracle_quantize(_p(src, _u16p), dtype, n, bits, _p(codes, _u8p), _p(scale, _f32p),
                          _p(zero, _i32p))
    return QBuffer(codes[:qcode_bytes(n, bits)], scale[:nblk], zero[:nblk], bits, n)


def dequantize(q: QBuffer) -> np.ndarray:
    """fp32 values S_b * (q_i - Z_b) of a quantised buffer."""
    out = np.empty(q.length, np.float32)
    codes = np.ascontiguousarray(q.codes) if q.codes.size else np.zeros(1, np.uint8)
    lib().oracle_dequantize(_p(codes, _u8p), _p(q.scale, _f32p), _p(q.zero, _i32p), q.bits,
                            q.length, _p(out, _f32p))
    return out


def reduce_q(rows: list, valid: int, inv: float) -> tuple[np.ndarray, int]:
    """The reduce over N quantised contribution rows (each a QBuffer of at
    least ``valid`` elements, same bits)."""
    n = len(rows)
    bits = rows[0].bits
    keep = [(np.ascontiguousarray(r.codes), np.ascontiguousarray(r.scale),
             np.ascontiguousarray(r.zero)) for r in rows]
    cp = (_u8p * n)(*[_p(c, _u8p) for c, _, _ in keep])
    sp = (_f32p * n)(*[_p(sc, _f32p) for _, sc, _ in keep])
    zp = (_i32p * n)(*[_p(z, _i32p) for _, _, z in keep])
    g = np.empty(valid, np.float32)
    flag = ctypes.c_int32()
    lib().oracle_reduce_q(cp, sp, zp, bits, n, valid, inv, _p(g, _f32p), ctypes.byref(flag))
    return g, int(flag.value)


# --------------------------------------------------------------------------- one full step
@dataclass
class RankState:
    """One rank's optimizer state for its valid elements (fp32 master, m, v)."""

    master: np.ndarray
    m: np.ndarray
    v: np.ndarray

    @classmethod
    def fresh(cls, master0: np.ndarray) -> "RankState":
        master0 = np.array(master0, dtype=np.float32, copy=True)
        z = np.zeros_like(master0)
        return cls(master0, z, z.copy())


def shard_step(contribs: list, dtype_in: int, states: list, offsets: list, scalars: Scalars,
               hp: Hparams, gather: np.ndarray | None, dtype_out: int) -> Report:
    """One ZeRO shard step for a set of ranks that share global scalars.

    ``contribs[r]`` is rank r's [N, stride] contribution array (its valid
    columns are ``states[r].master.size``).  The overflow flag and the squared
    norm are taken over all given ranks together, standing in for the scalar
    all-reduce between ranks; with one rank they are that rank's own.  When
    the step is applied, each rank's cast lands in ``gather`` at its offset.
    """
    n = contribs[0].shape[0]
    inv = inv_scale(n, scalars.scale)
    acc = SumSq()
    flag = 0
    grads = []
    for C, st in zip(contribs, states):
        g, f = reduce(C, dtype_in, st.master.size, inv)
        acc.add(g)
        flag |= f
        grads.append(g)
    rep = finalize(hp, scalars, flag, acc)
    if not rep.skip:
        for g, st, off in zip(grads, states, offsets):
            adam(st.master, st.m, st.v, g, hp, rep.clip, scalars.pow1, scalars.pow2)
            if gather is not None:
                gather[off:off + st.master.size] = cast(st.master, dtype_out)
    return rep
