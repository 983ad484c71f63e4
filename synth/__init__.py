"""Seeded synthetic inputs for the ZeRO per-rank shard step.

One counter-based generator (splitmix64 keyed by seed, stream, step,
contribution index and global element index; ``synth_core.h``) is built for
the host (gcc, used on the oracle side) and for the device (hipcc, used to
fill HBM for the GPU side).  Both builds give bit-identical values, so an
oracle can draw exactly the elements it checks.  The module holds none of the
shard step's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F16 = 1
BF16 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_CPU_SRC = os.path.join(_HERE, "synth_cpu.c")
_GPU_SRC = os.path.join(_HERE, "synth_gpu.hip")
_CPU_LIB = os.path.join(_HERE, "libsynth_cpu.so")
_GPU_LIB = os.path.join(_HERE, "libsynth_gpu.so")

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-fPIC", "-shared", "-Wall"]


def build(gpu: bool = True) -> None:
    tmp = _CPU_LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-Wall", "-Wextra", "-o", tmp, _CPU_SRC], check=True)
    os.replace(tmp, _CPU_LIB)
    if gpu:
        tmp = _GPU_LIB + ".tmp"
        subprocess.run(["hipcc", *HIPCC_FLAGS, "-o", tmp, _GPU_SRC], check=True,
                       stderr=subprocess.DEVNULL)
        os.replace(tmp, _GPU_LIB)


def outlier_threshold(p: float) -> int:
    """Integer threshold t with P(bits < t) = p for uniform 64-bit words."""
    return int(p * 2.0 ** 64) if p > 0 else 0


_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i64p = ctypes.POINTER(ctypes.c_int64)
_cpu = None
_gpu = None


def cpu():
    global _cpu
    if _cpu is None:
        if not os.path.exists(_CPU_LIB):
            build(gpu=False)
        L = ctypes.CDLL(_CPU_LIB)
        u64, u32, i32, i64, f64 = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32,
                                   ctypes.c_int64, ctypes.c_double)
        L.synth_contrib_rows.argtypes = [u64, u32, i32, i32, f64, f64, u64, f64, i64, i64, i64,
                                         _u16p]
        L.synth_contrib_at.argtypes = [u64, u32, i32, i32, f64, f64, u64, f64, _i64p, i64, _u16p]
        L.synth_master_range.argtypes = [u64, f64, i64, i64, _f32p]
        L.synth_master_at.argtypes = [u64, f64, _i64p, i64, _f32p]
        L.synth_param_range.argtypes = [u64, f64, i32, i64, i64, _u16p]
        L.synth_param_at.argtypes = [u64, f64, i32, _i64p, i64, _u16p]
        L.synth_bits_range.argtypes = [u64, u32, u32, u32, i64, i64, _u64p]
        L.synth_normal_range.argtypes = [u64, u32, u32, u32, i64, i64, _f64p]
        _cpu = L
    return _cpu


# --------------------------------------------------------------------------- host generator
def contrib_rows(seed, step, n, dtype, sigma, scale, outlier_p, outlier_mult, idx0, length,
                 stride=None, out=None) -> np.ndarray:
    """[n, stride] uint16 bit patterns of contributions for elements idx0..idx0+length-1."""
    stride = length if stride is None else stride
    if out is None:
        out = np.empty((n, stride), np.uint16)
    assert out.shape == (n, stride) and out.dtype == np.uint16 and out.flags.c_contiguous
    cpu().synth_contrib_rows(seed, step, n, dtype, sigma, scale, outlier_threshold(outlier_p),
                             outlier_mult, idx0, length, stride, out.ctypes.data_as(_u16p))
    return out


def contrib_at(seed, step, n, dtype, sigma, scale, outlier_p, outlier_mult,
               idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty((n, idx.size), np.uint16)
    cpu().synth_contrib_at(seed, step, n, dtype, sigma, scale, outlier_threshold(outlier_p),
                           outlier_mult, idx.ctypes.data_as(_i64p), idx.size,
                           out.ctypes.data_as(_u16p))
    return out


def master_range(seed, sigma, idx0, length) -> np.ndarray:
    out = np.empty(length, np.float32)
    cpu().synth_master_range(seed, sigma, idx0, length, out.ctypes.data_as(_f32p))
    return out


def master_at(seed, sigma, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, np.float32)
    cpu().synth_master_at(seed, sigma, idx.ctypes.data_as(_i64p), idx.size,
                          out.ctypes.data_as(_f32p))
    return out


def param_range(seed, sigma, dtype, idx0, length) -> np.ndarray:
    out = np.empty(length, np.uint16)
    cpu().synth_param_range(seed, sigma, dtype, idx0, length, out.ctypes.data_as(_u16p))
    return out


def param_at(seed, sigma, dtype, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, np.uint16)
    cpu().synth_param_at(seed, sigma, dtype, idx.ctypes.data_as(_i64p), idx.size,
                         out.ctypes.data_as(_u16p))
    return out


def bits_range(seed, stream, step, k, idx0, length) -> np.ndarray:
    out = np.empty(length, np.uint64)
    cpu().synth_bits_range(seed, stream, step, k, idx0, length, out.ctypes.data_as(_u64p))
    return out


def normal_range(seed, stream, step, k, idx0, length) -> np.ndarray:
    out = np.empty(length, np.float64)
    cpu().synth_normal_range(seed, stream, step, k, idx0, length, out.ctypes.data_as(_f64p))
    return out


# --------------------------------------------------------------------------- device generator
def gpu():
    global _gpu
    if _gpu is None:
        if not os.path.exists(_GPU_LIB):
            raise RuntimeError(f"{_GPU_LIB} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (its HIP runtime first: one runtime in the process)
        L = ctypes.CDLL(_GPU_LIB)
        u64, u32, i32, i64, f64, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_double, ctypes.c_void_p)
        L.synth_gpu_contrib_rows.argtypes = [u64, u32, i32, i32, f64, f64, u64, f64, i64, i64,
                                             i64, vp, vp]
        L.synth_gpu_master_range.argtypes = [u64, f64, i64, i64, vp, vp]
        L.synth_gpu_param_range.argtypes = [u64, f64, i32, i64, i64, vp, vp]
        L.synth_gpu_copy.argtypes = [vp, vp, i64, i32, vp]
        L.synth_gpu_stream.argtypes = [i32, vp, vp, vp, i64, i64, u32, vp]
        pi = ctypes.POINTER(i32)
        L.synth_gpu_device_info.argtypes = [i32, pi, pi, pi, pi]
        for f in (L.synth_gpu_contrib_rows, L.synth_gpu_master_range, L.synth_gpu_param_range,
                  L.synth_gpu_copy, L.synth_gpu_stream, L.synth_gpu_device_info):
            f.restype = ctypes.c_int
        _gpu = L
    return _gpu


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def gpu_contrib_rows(out, seed, step, dtype, sigma, scale, outlier_p, outlier_mult, idx0,
                     length) -> None:
    """Fill a [n, stride] 16-bit device tensor with contributions of elements idx0.."""
    n, stride = out.shape
    assert out.is_contiguous() and out.element_size() == 2
    _check(gpu().synth_gpu_contrib_rows(seed, step, n, dtype, sigma, scale,
                                        outlier_threshold(outlier_p), outlier_mult, idx0, length,
                                        stride, ctypes.c_void_p(out.data_ptr()), _stream()),
           "synth_gpu_contrib_rows")


def gpu_master_range(out, seed, sigma, idx0) -> None:
    assert out.is_contiguous() and out.element_size() == 4
    _check(gpu().synth_gpu_master_range(seed, sigma, idx0, out.numel(),
                                        ctypes.c_void_p(out.data_ptr()), _stream()),
           "synth_gpu_master_range")


def gpu_param_range(out, seed, sigma, dtype, idx0) -> None:
    assert out.is_contiguous() and out.element_size() == 2
    _check(gpu().synth_gpu_param_range(seed, sigma, dtype, idx0, out.numel(),
                                       ctypes.c_void_p(out.data_ptr()), _stream()),
           "synth_gpu_param_range")


def gpu_copy(src, dst, nbytes: int, grid: int = 0) -> None:
    _check(gpu().synth_gpu_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                nbytes, grid, _stream()), "synth_gpu_copy")


STREAM_KINDS = {"read": 0, "write": 1, "copy": 2, "mix_2r1w": 3, "mix_4r1w": 4}


def gpu_stream(kind: str, a, b, d, nbytes: int, chunk: int, lds: int) -> None:
    """A plain memory stream over nbytes of each array (reference lines for the
    benchmark): read a, write d, copy a to d, d = a + b (two bytes read per
    byte written), or d = a + a' + b + b' with a' and b' nbytes further on in
    a and b (four bytes read per byte written; a and b hold 2 * nbytes);
    launches of at most `chunk` workgroups of 8 KiB, each reserving `lds`
    bytes of LDS."""
    if kind == "mix_4r1w":
        for t in (a, b):
            assert t.numel() * t.element_size() >= 2 * nbytes, "mix_4r1w reads 2 * nbytes of a and b"
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)  # noqa: E731
    _check(gpu().synth_gpu_stream(STREAM_KINDS[kind], ptr(a), ptr(b), ptr(d), nbytes, chunk, lds,
                                  _stream()), "synth_gpu_stream")


def gpu_device_info(device: int = 0) -> dict:
    """Peak memory clock, bus width, CU count and shader clock of a device, and
    the HBM peak they imply.  HBM3E moves four bits per pin per clock that the
    device reports (MI355X: 2000 MHz, 8 Gb/s per pin), so the peak is
    bus_bits / 8 * 4 * clock."""
    v = [ctypes.c_int32() for _ in range(4)]
    _check(gpu().synth_gpu_device_info(device, *[ctypes.byref(x) for x in v]), "device_info")
    mem_khz, bus, cus, clk = (x.value for x in v)
    return {"mem_clock_mhz": mem_khz / 1e3, "bus_bits": bus, "cus": cus, "clock_mhz": clk / 1e3,
            "hbm_peak_gbps_from_props": round(4 * mem_khz * 1e3 * bus / 8 / 1e9, 1)}
