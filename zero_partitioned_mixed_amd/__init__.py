"""Python binding of libzero_shard.so, the ZeRO per-rank shard step for MI355X.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions carry the C names (include/zero_shard.h) and take torch
device tensors, passing their data pointers and torch's current HIP stream.
The library must be built (``__graft_entry__.build()``); importing the package
without it raises ImportError, and there is no CPU fallback.

``ShardStep`` sequences the calls of one rank's step (two-pass when clipping
is on, fused single pass otherwise); ``MultiShardStep`` runs several ranks'
shards held on one GPU with shared global scalars.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzero_shard.so")

F16 = 1
BF16 = 2
SCALER_NONE, SCALER_STATIC, SCALER_DYNAMIC = 0, 1, 2
MAX_RANKS = 64

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950); there is no fallback path")

# torch first: its HIP runtime must be the one in the process when this library
# loads.  The library asks for libamdhip64.so.7, which resolves to torch's
# bundled runtime once that is loaded; loaded the other way round, the process
# holds two HIP runtimes and this library's finds no device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class Hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("max_grad_norm", ctypes.c_float), ("scaler", _i32),
                ("min_scale", ctypes.c_float), ("growth_interval", _i32)]


class Ctrl(ctypes.Structure):
    _fields_ = [("sumsq", ctypes.c_double), ("norm", ctypes.c_double),
                ("beta1_pow", ctypes.c_double), ("beta2_pow", ctypes.c_double),
                ("loss_scale", ctypes.c_float), ("scale_used", ctypes.c_float),
                ("clip", ctypes.c_float), ("nonfinite", _i32), ("skip", _i32), ("t", _i32),
                ("good_steps", _i32), ("cur", _i32), ("arrive", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32 * 15)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


TILE = 2048  # ZERO_TILE
QBLOCK = 2048  # ZERO_QBLOCK
PARTIAL_BYTES = 16  # ZERO_PARTIAL_BYTES
LAUNCH_TILES = 32768  # ZERO_LAUNCH_TILES
LAUNCH_ROW_TILES = 131072  # ZERO_LAUNCH_ROW_TILES
LAUNCH_MIN_TILES = 2048  # ZERO_LAUNCH_MIN_TILES
LAUNCH_PAYLOAD_TILES = 16384  # ZERO_LAUNCH_PAYLOAD_TILES
NOALLOC_MAX_LEN = 1 << 31  # ZERO_NOALLOC_MAX_LEN
BATCH_SHARDS = 32  # ZERO_BATCH_SHARDS


def launch_tiles(nranks: int = 0, payload: bool = False) -> int:
    """Most tiles per launch of a pass that reads nranks contribution rows
    (0: the Adam passes); the library's zero_launch_tiles.  payload: the fused
    step that also writes the quantised all-gather payload."""
    t = LAUNCH_TILES if nranks <= 8 else max(LAUNCH_MIN_TILES, LAUNCH_ROW_TILES // nranks)
    return min(t, LAUNCH_PAYLOAD_TILES) if payload else t


def launches(valid_len: int, nranks: int = 0, payload: bool = False) -> int:
    """Kernel launches one call of a streaming pass over valid_len elements
    is issued as (nranks and payload as in launch_tiles)."""
    tiles = -(-valid_len // TILE)
    return -(-tiles // launch_tiles(nranks, payload))


class State(ctypes.Structure):
    _fields_ = [("master", _vp), ("m", _vp), ("v", _vp)]


class Shard(ctypes.Structure):
    """zero_shard: one shard of the batched calls."""
    _fields_ = [("contrib", _vp), ("stride", _i64), ("pair", _vp), ("valid_len", _i64),
                ("offset", _i64), ("ctrl", _vp), ("ws", _vp), ("ws_bytes", ctypes.c_size_t),
                ("state", State), ("g", _vp)]


_sig = {
    "zero_partition": (ctypes.c_int, [_i64, _i32, _i32, ctypes.POINTER(_i64),
                                      ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "zero_ctrl_bytes": (ctypes.c_size_t, []),
    "zero_workspace_bytes": (ctypes.c_size_t, [_i64]),
    "zero_pair_elems": (ctypes.c_size_t, [_i64]),
    "zero_ctrl_init": (ctypes.c_int, [_vp, ctypes.c_float, _vp]),
    "zero_reduce_grads": (ctypes.c_int, [_vp, _i32, _i32, _i64, _i64, _vp, _vp, _vp,
                                         ctypes.c_size_t, _vp]),
    "zero_reduce_grads_rows": (ctypes.c_int, [ctypes.POINTER(_vp), _i32, _i32, _i64, _vp, _vp,
                                              _vp, ctypes.c_size_t, _vp]),
    "zero_grad_norm_overflow": (ctypes.c_int, [_i32, ctypes.POINTER(_vp), ctypes.POINTER(_i64),
                                               ctypes.POINTER(_vp), ctypes.POINTER(Hparams),
                                               _i32, _vp]),
    "zero_adam_step": (ctypes.c_int, [ctypes.POINTER(State), _vp, _i64, ctypes.POINTER(Hparams),
                                      _vp, _vp, _i32, _i64, _vp]),
    "zero_cast_to_gather": (ctypes.c_int, [_vp, _i64, _vp, _i32, _i64, _vp]),
    "zero_fused_step": (ctypes.c_int, [_vp, _i32, _i32, _i64, ctypes.POINTER(State), _i64, _vp,
                                       _i32, _i64, ctypes.POINTER(Hparams), _vp, _vp,
                                       ctypes.c_size_t, _vp]),
    "zero_fused_step_rows": (ctypes.c_int, [ctypes.POINTER(_vp), _i32, _i32,
                                            ctypes.POINTER(State), _i64, _vp, _i32, _i64,
                                            ctypes.POINTER(Hparams), _vp, _vp, ctypes.c_size_t,
                                            _vp]),
    "zero_fused_restore": (ctypes.c_int, [ctypes.POINTER(State), _i64, _vp, _i32, _i64, _vp,
                                          _vp]),
    "zero_pair_store": (ctypes.c_int, [ctypes.POINTER(State), ctypes.POINTER(State), _i64, _vp,
                                       _vp]),
    "zero_pair_load": (ctypes.c_int, [ctypes.POINTER(State), ctypes.POINTER(State), _i64, _vp,
                                      _vp]),
    "zero_qblock_count": (ctypes.c_size_t, [_i64]),
    "zero_qcode_bytes": (ctypes.c_size_t, [_i64, _i32]),
    "zero_quantize_blocks": (ctypes.c_int, [_vp, _i32, _i64, _i32, _vp, _vp, _vp]),
    "zero_dequantize_blocks": (ctypes.c_int, [_vp, _vp, _i32, _i64, _vp, _i32, _vp]),
    "zero_reduce_grads_q": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i32,
                                           _i64, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "zero_fused_step_q": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i32,
                                         ctypes.POINTER(State), _i64, _vp, _i32, _i64,
                                         ctypes.POINTER(Hparams), _vp, _vp, ctypes.c_size_t, _vp]),
    "zero_fused_step_qgather": (ctypes.c_int, [_vp, _i32, _i32, _i64, ctypes.POINTER(State), _i64,
                                               _vp, _i32, _i64, _i32, _vp, _vp,
                                               ctypes.POINTER(Hparams), _vp, _vp, ctypes.c_size_t,
                                               _vp]),
    "zero_fused_step_rows_qgather": (ctypes.c_int, [ctypes.POINTER(_vp), _i32, _i32,
                                                    ctypes.POINTER(State), _i64, _vp, _i32, _i64,
                                                    _i32, _vp, _vp, ctypes.POINTER(Hparams), _vp,
                                                    _vp, ctypes.c_size_t, _vp]),
    "zero_fused_step_q_qgather": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32,
                                                 _i32, ctypes.POINTER(State), _i64, _vp, _i32,
                                                 _i64, _i32, _vp, _vp, ctypes.POINTER(Hparams),
                                                 _vp, _vp, ctypes.c_size_t, _vp]),
    "zero_fused_restore_q": (ctypes.c_int, [ctypes.POINTER(State), _i64, _vp, _i32, _i64, _i32, _vp,
                                            _vp, _vp, _vp]),
    "zero_adam_step_qgather": (ctypes.c_int, [ctypes.POINTER(State), _vp, _i64,
                                              ctypes.POINTER(Hparams), _vp, _vp, _i32, _i64, _i32,
                                              _vp, _vp, _vp]),
    "zero_fused_step_noalloc": (ctypes.c_int, [_vp, _i32, _i32, _i64, ctypes.POINTER(State), _i64,
                                               _vp, _i32, _i64, ctypes.POINTER(Hparams), _vp, _vp]),
    "zero_fused_step_shards": (ctypes.c_int, [ctypes.POINTER(Shard), _i32, _i32, _i32, _vp, _i32,
                                              ctypes.POINTER(Hparams), _vp]),
    "zero_fused_restore_shards": (ctypes.c_int, [ctypes.POINTER(Shard), _i32, _vp, _i32, _vp]),
    "zero_reduce_grads_shards": (ctypes.c_int, [ctypes.POINTER(Shard), _i32, _i32, _i32, _vp]),
    "zero_adam_step_shards": (ctypes.c_int, [ctypes.POINTER(Shard), _i32, ctypes.POINTER(Hparams),
                                             _vp, _i32, _vp]),
    "zero_launch_tiles": (ctypes.c_int64, [_i32]),
    "zero_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTS = tuple(_sig)


class ZeroError(RuntimeError):
    def __init__(self, call: str, code: int):
        msg = _lib.zero_last_error().decode()
        super().__init__(f"{call} returned {code}: {msg}")
        self.code = code


def _check(call: str, rc: int) -> None:
    if rc != 0:
        raise ZeroError(call, rc)


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(None)
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows(rows):
    """Host array of row pointers: each entry a GPU tensor (its data pointer)
    or an integer device address."""
    ptrs = []
    for r in rows:
        if isinstance(r, int):
            ptrs.append(r)
        else:
            ptrs.append(_ptr(r).value)
    return (_vp * max(len(ptrs), 1))(*ptrs), len(ptrs)


def _at(x, nbytes: int):
    """x advanced by nbytes: an integer device address, or a 1-D tensor sliced."""
    if isinstance(x, int):
        return x + nbytes
    return x[nbytes // x.element_size():]


def _state(s) -> State:
    master, m, v = s
    return State(_ptr(master), _ptr(m), _ptr(v))


def hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.0,
            scaler=SCALER_NONE, min_scale=1.0, growth_interval=1000) -> Hparams:
    return Hparams(lr, beta1, beta2, eps, weight_decay, max_grad_norm, scaler, min_scale,
                   growth_interval)


# ----------------------------------------------------------------------------- the C calls
def zero_partition(psi: int, nranks: int, rank: int) -> tuple[int, int, int]:
    s, o, v = _i64(), _i64(), _i64()
    _check("zero_partition", _lib.zero_partition(psi, nranks, rank, ctypes.byref(s),
                                                 ctypes.byref(o), ctypes.byref(v)))
    return s.value, o.value, v.value


def zero_ctrl_bytes() -> int:
    return _lib.zero_ctrl_bytes()


def zero_workspace_bytes(valid_len: int) -> int:
    return _lib.zero_workspace_bytes(valid_len)


def zero_pair_elems(valid_len: int) -> int:
    return _lib.zero_pair_elems(valid_len)


def paired_state(valid_len: int, device):
    """A paired (fused-path) state: one fp32 buffer of zero_pair_elems
    floats, returned as the (master, m, v) views the paired calls take (m and
    v start ZERO_TILE and 2 * ZERO_TILE floats into the buffer)."""
    import torch
    buf = torch.empty(max(zero_pair_elems(valid_len), 3 * TILE), dtype=torch.float32,
                      device=device)
    return buf, buf[TILE:], buf[2 * TILE:]


def zero_ctrl_init(ctrl, loss_scale: float) -> None:
    _check("zero_ctrl_init", _lib.zero_ctrl_init(_ptr(ctrl), loss_scale, _stream()))


def zero_reduce_grads(contrib, dtype: int, nranks: int, stride: int, valid_len: int, ctrl, g,
                      ws) -> None:
    _check("zero_reduce_grads", _lib.zero_reduce_grads(
        _ptr(contrib), dtype, nranks, stride, valid_len, _ptr(ctrl), _ptr(g), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))


def zero_reduce_grads_rows(rows, dtype: int, valid_len: int, ctrl, g, ws) -> None:
    arr, n = _rows(rows)
    _check("zero_reduce_grads_rows", _lib.zero_reduce_grads_rows(
        arr, dtype, n, valid_len, _ptr(ctrl), _ptr(g), _ptr(ws), ws.numel() * ws.element_size(),
        _stream()))


def zero_grad_norm_overflow(ws_list, valid_lens, ctrls, hp: Hparams, pingpong: bool) -> None:
    n = len(ctrls)
    ws_arr = (_vp * n)(*[t.data_ptr() if t is not None else None for t in ws_list])
    len_arr = (_i64 * n)(*valid_lens)
    ctrl_arr = (_vp * n)(*[t.data_ptr() for t in ctrls])
    _check("zero_grad_norm_overflow", _lib.zero_grad_norm_overflow(
        n, ws_arr, len_arr, ctrl_arr, ctypes.byref(hp), int(bool(pingpong)), _stream()))


def zero_adam_step(state, g, valid_len: int, hp: Hparams, ctrl, gather=None,
                   gather_dtype: int = F16, offset: int = 0) -> None:
    st = _state(state)
    _check("zero_adam_step", _lib.zero_adam_step(
        ctypes.byref(st), _ptr(g), valid_len, ctypes.byref(hp), _ptr(ctrl), _ptr(gather),
        gather_dtype, offset, _stream()))


def zero_cast_to_gather(master, valid_len: int, gather, dtype: int, offset: int) -> None:
    _check("zero_cast_to_gather", _lib.zero_cast_to_gather(
        _ptr(master), valid_len, _ptr(gather), dtype, offset, _stream()))


def zero_fused_step(contrib, contrib_dtype: int, nranks: int, stride: int, pair,
                    valid_len: int, gather, gather_dtype: int, offset: int, hp: Hparams, ctrl,
                    ws) -> None:
    st = _state(pair)
    _check("zero_fused_step", _lib.zero_fused_step(
        _ptr(contrib), contrib_dtype, nranks, stride, ctypes.byref(st), valid_len, _ptr(gather),
        gather_dtype, offset, ctypes.byref(hp), _ptr(ctrl), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))


def zero_fused_step_noalloc(contrib, contrib_dtype: int, nranks: int, stride: int, pair,
                            valid_len: int, gather, gather_dtype: int, offset: int, hp: Hparams,
                            ctrl) -> None:
    """One rank's whole fused step (pass, decision, restore) with no workspace:
    the library keeps the partials in its own device array."""
    st = _state(pair)
    _check("zero_fused_step_noalloc", _lib.zero_fused_step_noalloc(
        _ptr(contrib), contrib_dtype, nranks, stride, ctypes.byref(st), valid_len, _ptr(gather),
        gather_dtype, offset, ctypes.byref(hp), _ptr(ctrl), _stream()))


def zero_fused_step_rows(rows, contrib_dtype: int, pair, valid_len: int, gather,
                         gather_dtype: int, offset: int, hp: Hparams, ctrl, ws) -> None:
    arr, n = _rows(rows)
    st = _state(pair)
    _check("zero_fused_step_rows", _lib.zero_fused_step_rows(
        arr, contrib_dtype, n, ctypes.byref(st), valid_len, _ptr(gather), gather_dtype, offset,
        ctypes.byref(hp), _ptr(ctrl), _ptr(ws), ws.numel() * ws.element_size(), _stream()))


def zero_fused_restore(pair, valid_len: int, gather, dtype: int, offset: int, ctrl) -> None:
    st = _state(pair)
    _check("zero_fused_restore", _lib.zero_fused_restore(
        ctypes.byref(st), valid_len, _ptr(gather), dtype, offset, _ptr(ctrl), _stream()))


def shard_table(shards) -> ctypes.Array:
    """The host array of zero_shard descriptors the batched calls take, from
    (contrib, stride, pair, valid_len, offset, ctrl, ws, state, g) per shard:
    contrib the [N, stride] rows, pair the paired state's (master, m, v) views
    (fused path, else None), ws the shard's workspace tensor, state the flat
    (master, m, v) and g the gradient buffer (two-pass path, else None)."""
    table = (Shard * len(shards))()
    for d, (contrib, stride, pair, valid_len, offset, ctrl, ws, state, g) in zip(table, shards):
        d.contrib, d.stride = _ptr(contrib), stride
        d.pair = _ptr(pair[0]) if pair is not None else None
        d.valid_len, d.offset, d.ctrl = valid_len, offset, _ptr(ctrl)
        d.ws, d.ws_bytes = _ptr(ws), ws.numel() * ws.element_size()
        if state is not None:
            d.state = _state(state)
        d.g = _ptr(g) if g is not None else None
    return table


def zero_fused_step_shards(table, contrib_dtype: int, nranks: int, gather, gather_dtype: int,
                           hp: Hparams) -> None:
    _check("zero_fused_step_shards", _lib.zero_fused_step_shards(
        table, len(table), contrib_dtype, nranks, _ptr(gather), gather_dtype, ctypes.byref(hp),
        _stream()))


def zero_fused_restore_shards(table, gather, gather_dtype: int) -> None:
    _check("zero_fused_restore_shards", _lib.zero_fused_restore_shards(
        table, len(table), _ptr(gather), gather_dtype, _stream()))


def zero_reduce_grads_shards(table, contrib_dtype: int, nranks: int) -> None:
    _check("zero_reduce_grads_shards", _lib.zero_reduce_grads_shards(
        table, len(table), contrib_dtype, nranks, _stream()))


def zero_adam_step_shards(table, hp: Hparams, gather, gather_dtype: int) -> None:
    _check("zero_adam_step_shards", _lib.zero_adam_step_shards(
        table, len(table), ctypes.byref(hp), _ptr(gather), gather_dtype, _stream()))


def zero_pair_store(flat, pair, valid_len: int, ctrl) -> None:
    f, p = _state(flat), _state(pair)
    _check("zero_pair_store", _lib.zero_pair_store(ctypes.byref(f), ctypes.byref(p), valid_len,
                                                   _ptr(ctrl), _stream()))


def zero_pair_load(pair, flat, valid_len: int, ctrl) -> None:
    p, f = _state(pair), _state(flat)
    _check("zero_pair_load", _lib.zero_pair_load(ctypes.byref(p), ctypes.byref(f), valid_len,
                                                 _ptr(ctrl), _stream()))


def zero_qblock_count(length: int) -> int:
    return _lib.zero_qblock_count(length)


def zero_qcode_bytes(length: int, bits: int) -> int:
    return _lib.zero_qcode_bytes(length, bits)


def zero_quantize_blocks(src, dtype: int, length: int, bits: int, codes, blocks) -> None:
    _check("zero_quantize_blocks", _lib.zero_quantize_blocks(
        _ptr(src), dtype, length, bits, _ptr(codes), _ptr(blocks), _stream()))


def zero_dequantize_blocks(codes, blocks, bits: int, length: int, dst, dtype: int) -> None:
    _check("zero_dequantize_blocks", _lib.zero_dequantize_blocks(
        _ptr(codes), _ptr(blocks), bits, length, _ptr(dst), dtype, _stream()))


class QuantRows:
    """N block-quantised contribution rows: ``rows`` is a list of (codes,
    blocks) device tensors (or integer addresses), all of ``bits`` bits."""

    def __init__(self, rows, bits: int):
        self.rows, self.bits = list(rows), bits

    def tables(self):
        c, n = _rows([r[0] for r in self.rows])
        b, _ = _rows([r[1] for r in self.rows])
        return c, b, n

    @staticmethod
    def alloc(nranks: int, length: int, bits: int, device):
        """Code and block buffers for nranks rows of `length` elements."""
        import torch
        nbytes = max((zero_qcode_bytes(length, bits) + 15) // 16 * 16, 16)
        nblk = max(zero_qblock_count(length), 1)
        return QuantRows([(torch.empty(nbytes, dtype=torch.uint8, device=device),
                           torch.empty(nblk * 8, dtype=torch.uint8, device=device))
                          for _ in range(nranks)], bits)


def zero_reduce_grads_q(q: QuantRows, valid_len: int, ctrl, g, ws) -> None:
    c, b, n = q.tables()
    _check("zero_reduce_grads_q", _lib.zero_reduce_grads_q(
        c, b, q.bits, n, valid_len, _ptr(ctrl), _ptr(g), _ptr(ws), ws.numel() * ws.element_size(),
        _stream()))


def zero_fused_step_q(q: QuantRows, pair, valid_len: int, gather, gather_dtype: int, offset: int,
                      hp: Hparams, ctrl, ws) -> None:
    c, b, n = q.tables()
    st = _state(pair)
    _check("zero_fused_step_q", _lib.zero_fused_step_q(
        c, b, q.bits, n, ctypes.byref(st), valid_len, _ptr(gather), gather_dtype, offset,
        ctypes.byref(hp), _ptr(ctrl), _ptr(ws), ws.numel() * ws.element_size(), _stream()))


class QGather:
    """A rank's quantised all-gather payload: ``codes`` and ``blocks`` device
    tensors holding ``bits``-bit block codes of ``length`` 16-bit parameters."""

    def __init__(self, codes, blocks, bits: int, length: int):
        self.codes, self.blocks, self.bits, self.length = codes, blocks, bits, length

    @staticmethod
    def alloc(length: int, bits: int, device):
        (codes, blocks), = QuantRows.alloc(1, length, bits, device).rows
        return QGather(codes, blocks, bits, length)

    def at(self, b0: int):
        """The payload from element b0 on (b0 a multiple of TILE)."""
        return QGather(_at(self.codes, b0 * self.bits // 8), _at(self.blocks, b0 // QBLOCK * 8),
                       self.bits, self.length - b0)


def zero_fused_step_qgather(contrib, contrib_dtype: int, nranks: int, stride: int, pair,
                            valid_len: int, gather, gather_dtype: int, offset: int, q: QGather,
                            hp: Hparams, ctrl, ws) -> None:
    st = _state(pair)
    _check("zero_fused_step_qgather", _lib.zero_fused_step_qgather(
        _ptr(contrib), contrib_dtype, nranks, stride, ctypes.byref(st), valid_len, _ptr(gather),
        gather_dtype, offset, q.bits, _ptr(q.codes), _ptr(q.blocks), ctypes.byref(hp), _ptr(ctrl),
        _ptr(ws), ws.numel() * ws.element_size(), _stream()))


def zero_fused_step_rows_qgather(rows, contrib_dtype: int, pair, valid_len: int, gather,
                                 gather_dtype: int, offset: int, q: QGather, hp: Hparams, ctrl,
                                 ws) -> None:
    arr, n = _rows(rows)
    st = _state(pair)
    _check("zero_fused_step_rows_qgather", _lib.zero_fused_step_rows_qgather(
        arr, contrib_dtype, n, ctypes.byref(st), valid_len, _ptr(gather), gather_dtype, offset,
        q.bits, _ptr(q.codes), _ptr(q.blocks), ctypes.byref(hp), _ptr(ctrl), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))


def zero_fused_step_q_qgather(qr: QuantRows, pair, valid_len: int, gather, gather_dtype: int,
                              offset: int, q: QGather, hp: Hparams, ctrl, ws) -> None:
    c, b, n = qr.tables()
    st = _state(pair)
    _check("zero_fused_step_q_qgather", _lib.zero_fused_step_q_qgather(
        c, b, qr.bits, n, ctypes.byref(st), valid_len, _ptr(gather), gather_dtype, offset, q.bits,
        _ptr(q.codes), _ptr(q.blocks), ctypes.byref(hp), _ptr(ctrl), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))


def zero_fused_restore_q(pair, valid_len: int, gather, dtype: int, offset: int, q: QGather,
                         ctrl) -> None:
    st = _state(pair)
    _check("zero_fused_restore_q", _lib.zero_fused_restore_q(
        ctypes.byref(st), valid_len, _ptr(gather), dtype, offset, q.bits, _ptr(q.codes),
        _ptr(q.blocks), _ptr(ctrl), _stream()))


def zero_adam_step_qgather(state, g, valid_len: int, hp: Hparams, ctrl, gather,
                           gather_dtype: int, offset: int, q: QGather) -> None:
    st = _state(state)
    _check("zero_adam_step_qgather", _lib.zero_adam_step_qgather(
        ctypes.byref(st), _ptr(g), valid_len, ctypes.byref(hp), _ptr(ctrl), _ptr(gather),
        gather_dtype, offset, q.bits, _ptr(q.codes), _ptr(q.blocks), _stream()))


def zero_last_error() -> str:
    return _lib.zero_last_error().decode()


def read_ctrl(ctrl) -> dict:
    """Copies a ctrl block back to the host (synchronises) and decodes it."""
    raw = bytes(ctrl.detach().cpu().numpy().tobytes())
    return Ctrl.from_buffer_copy(raw).as_dict()


# ----------------------------------------------------------------------------- sequencing helpers
class ShardStep:
    """One rank's shard step over caller-provided device buffers.

    contrib: [N, stride] 16-bit tensor, a list of N row tensors (or device
    addresses) taken by the row-table calls, or a QuantRows of block-quantised
    rows taken by the *_q calls; gather: the full 16-bit parameter buffer, this
    rank's slot at ``offset``.  ``state`` is the flat
    (master, m, v) fp32 state of valid_len elements.  The two-pass path
    (clipping on) updates it in place through ``g``; the fused path keeps
    its double-buffered copy in ``pair`` (one interleaved buffer allocated
    here by paired_state(), loaded from ``state``) and ``current()`` copies
    the current set back out.

    ``bucket`` (a multiple of TILE elements; 0 for none): the shard's gradient
    arrives in consecutive pieces of that many elements, and each piece is
    reduced (two-pass) or fully stepped (fused) by its own calls before the
    decision over the whole shard; bit-identical to one call per step.
    """

    def __init__(self, nranks, stride, valid_len, offset, dtype, gather_dtype, hp: Hparams,
                 state, g=None, loss_scale=1.0, bucket: int = 0):
        import torch
        if bucket < 0 or bucket % TILE:
            raise ValueError(f"bucket must be a multiple of {TILE} elements")
        self.bucket = bucket
        self.nranks, self.stride, self.valid_len, self.offset = nranks, stride, valid_len, offset
        self.dtype, self.gather_dtype, self.hp = dtype, gather_dtype, hp
        self.state, self.g = state, g
        self.fused = hp.max_grad_norm <= 0
        if not self.fused and g is None:
            raise ValueError("the two-pass path needs a g buffer")
        dev = state[0].device
        self.ctrl = torch.empty(zero_ctrl_bytes(), dtype=torch.uint8, device=dev)
        self.ws = torch.empty(zero_workspace_bytes(valid_len), dtype=torch.uint8, device=dev)
        zero_ctrl_init(self.ctrl, loss_scale)
        self.pair = None
        if self.fused:
            self.pair = paired_state(valid_len, dev)
            zero_pair_store(state, self.pair, valid_len, self.ctrl)

    def pieces(self):
        """(first element, length) of each piece one step is issued in."""
        b, n = self.bucket, self.valid_len
        if not b or n <= b:
            return [(0, n)]
        return [(b0, min(b, n - b0)) for b0 in range(0, n, b)]

    @staticmethod
    def _contrib_at(contrib, b0: int):
        if isinstance(contrib, QuantRows):
            return QuantRows([(_at(c, b0 * contrib.bits // 8), _at(k, b0 // QBLOCK * 8))
                              for c, k in contrib.rows], contrib.bits)
        if isinstance(contrib, (list, tuple)):
            return [_at(r, 2 * b0) for r in contrib]
        return contrib[:, b0:]

    def step(self, contrib, gather, qgather: QGather = None) -> None:
        """One step.  With ``qgather`` the step also writes the quantised
        all-gather payload of the new parameters, and ``gather`` may be None
        (no 16-bit slot written)."""
        self.run_pieces(contrib, gather, qgather)
        self.decide()
        self.complete(gather, qgather)

    def run_pieces(self, contrib, gather, qgather: QGather = None) -> None:
        """The per-element launches of a step, one per piece: the reduce
        (two-pass) or the whole fused step (fused path)."""
        quant = isinstance(contrib, QuantRows)
        table = isinstance(contrib, (list, tuple))
        if (table and len(contrib) != self.nranks) or (quant and len(contrib.rows) != self.nranks):
            raise ValueError(f"contribution rows do not match {self.nranks} ranks")
        hp, ctrl = self.hp, self.ctrl
        pieces = self.pieces()
        for b0, ln in pieces:
            if len(pieces) == 1:
                c, ws, off, q = contrib, self.ws, self.offset, qgather
            else:
                c, ws = self._contrib_at(contrib, b0), _at(self.ws, b0 // TILE * PARTIAL_BYTES)
                off, q = self.offset + b0, None if qgather is None else qgather.at(b0)
            if self.fused:
                pair = self.pair if b0 == 0 else tuple(_at(t, 4 * 6 * b0) for t in self.pair)
                if q is not None and quant:
                    zero_fused_step_q_qgather(c, pair, ln, gather, self.gather_dtype, off, q, hp,
                                              ctrl, ws)
                elif q is not None and table:
                    zero_fused_step_rows_qgather(c, self.dtype, pair, ln, gather,
                                                 self.gather_dtype, off, q, hp, ctrl, ws)
                elif q is not None:
                    zero_fused_step_qgather(c, self.dtype, self.nranks, self.stride, pair, ln,
                                            gather, self.gather_dtype, off, q, hp, ctrl, ws)
                elif quant:
                    zero_fused_step_q(c, pair, ln, gather, self.gather_dtype, off, hp, ctrl, ws)
                elif table:
                    zero_fused_step_rows(c, self.dtype, pair, ln, gather, self.gather_dtype, off,
                                         hp, ctrl, ws)
                else:
                    zero_fused_step(c, self.dtype, self.nranks, self.stride, pair, ln, gather,
                                    self.gather_dtype, off, hp, ctrl, ws)
            else:
                g = self.g if b0 == 0 else _at(self.g, 4 * b0)
                if quant:
                    zero_reduce_grads_q(c, ln, ctrl, g, ws)
                elif table:
                    zero_reduce_grads_rows(c, self.dtype, ln, ctrl, g, ws)
                else:
                    zero_reduce_grads(c, self.dtype, self.nranks, self.stride, ln, ctrl, g, ws)

    def decide(self) -> None:
        """Norm, overflow and the step's decisions over the whole shard."""
        zero_grad_norm_overflow([self.ws], [self.valid_len], [self.ctrl], self.hp, self.fused)

    def complete(self, gather, qgather: QGather = None) -> None:
        """The rest of the step: the Adam pass (two-pass path), or the restore
        of slot and payload after a skipped fused step."""
        if self.fused and qgather is not None:
            zero_fused_restore_q(self.pair, self.valid_len, gather, self.gather_dtype, self.offset,
                                 qgather, self.ctrl)
        elif self.fused:
            zero_fused_restore(self.pair, self.valid_len, gather, self.gather_dtype, self.offset,
                               self.ctrl)
        elif qgather is not None:
            zero_adam_step_qgather(self.state, self.g, self.valid_len, self.hp, self.ctrl, gather,
                                   self.gather_dtype, self.offset, qgather)
        else:
            zero_adam_step(self.state, self.g, self.valid_len, self.hp, self.ctrl, gather,
                           self.gather_dtype, self.offset)

    def capture(self, contrib, gather, qgather: QGather = None):
        """Records one step (its two or three launches) into a HIP graph and
        returns it (a torch.cuda.CUDAGraph); ``graph.replay()`` then runs a
        step.  Every step-to-step scalar lives in the device ctrl block and every
        argument is a fixed pointer, so the same graph serves every later step:
        the caller refills ``contrib`` in place between replays.  Capturing
        runs nothing."""
        import torch
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.step(contrib, gather, qgather)
        torch.cuda.current_stream().wait_stream(side)
        return graph

    def current(self):
        """(master, m, v): the current state, flat (the fused path copies it
        out of the paired buffers into ``state``)."""
        if self.fused:
            zero_pair_load(self.pair, self.state, self.valid_len, self.ctrl)
        return self.state

    def ctrl_dict(self) -> dict:
        return read_ctrl(self.ctrl)


class MultiShardStep:
    """Several ranks' shard steps on one GPU whose norm and overflow decisions
    are combined across the ranks (the scalar all-reduce between ranks).  The
    ranks share one path and one set of hyperparameters; each takes its own
    contributions (any form ShardStep takes) and optional payload.

    With ``batched`` (the default), a step whose ranks all take one [N, stride]
    contribution tensor, write no quantised payload, come in one piece and fit
    one launch goes through the batched calls, one launch per 32 ranks and
    pass: zero_fused_step_shards, the decision, zero_fused_restore_shards on
    the fused path (which also needs the 16-bit slot); zero_reduce_grads_shards,
    the decision, zero_adam_step_shards on the two-pass path.  Bit-identical to
    every rank's own calls."""

    def __init__(self, steps: list, batched: bool = True):
        if not 1 <= len(steps) <= MAX_RANKS:
            raise ValueError("between 1 and 64 ranks")
        first = bytes(steps[0].hp)
        if any(bytes(s.hp) != first for s in steps):
            raise ValueError("the ranks of one decision share their hyperparameters")
        self.steps = steps
        self.fused = steps[0].fused
        self.batched = batched
        self._table = None  # (contribution addresses, shard_table)

    def _batch_table(self, contribs, gather, qgathers):
        """The shard table of a step the batched calls can take, or None."""
        ss, s0 = self.steps, self.steps[0]
        if not self.batched or any(q is not None for q in qgathers):
            return None
        if self.fused and gather is None:
            return None
        cap = launch_tiles(s0.nranks) * TILE
        if any(s.bucket or s.valid_len > cap or s.nranks != s0.nranks or s.dtype != s0.dtype
               or s.gather_dtype != s0.gather_dtype for s in ss):
            return None
        if any(isinstance(c, (list, tuple, QuantRows)) for c in contribs):
            return None
        key = tuple(c.data_ptr() for c in contribs)
        if self._table is None or self._table[0] != key:
            self._table = (key, shard_table([
                (c, s.stride, s.pair, s.valid_len, s.offset, s.ctrl, s.ws,
                 None if self.fused else s.state, s.g) for s, c in zip(ss, contribs)]))
        return self._table[1]

    def step(self, contribs, gather, qgathers=None, branches: list | None = None) -> None:
        """One step of every rank.  With ``branches`` (streams) and a step
        the batched calls do not take, rank i's launches go to
        branches[i % len(branches)], forked from and joined back into the
        current stream around each phase; the ranks touch disjoint buffers,
        so only the shared decision orders them."""
        qgathers = self._payloads(contribs, qgathers)
        self.run_passes(contribs, gather, qgathers, branches)
        self.decide()
        self.complete(contribs, gather, qgathers, branches)

    def takes_batched(self, contribs, gather, qgathers=None) -> bool:
        """Whether a step on these buffers goes through the batched calls."""
        return self._batch_table(contribs, gather, self._payloads(contribs, qgathers)) is not None

    def _payloads(self, contribs, qgathers):
        n = len(self.steps)
        qgathers = [None] * n if qgathers is None else list(qgathers)
        if len(contribs) != n or len(qgathers) != n:
            raise ValueError(f"one contribution set and payload per rank ({n})")
        return qgathers

    def _per_rank(self, fn, branches) -> None:
        import torch
        if not branches:
            for i in range(len(self.steps)):
                fn(i)
            return
        main = torch.cuda.current_stream()
        for b in branches:
            b.wait_stream(main)
        for i in range(len(self.steps)):
            with torch.cuda.stream(branches[i % len(branches)]):
                fn(i)
        for b in branches:
            main.wait_stream(b)

    def run_passes(self, contribs, gather, qgathers=None, branches=None) -> None:
        """The per-element launches of a step: every rank's fused pass or
        reduce pass (one batched launch per 32 ranks when the step allows)."""
        ss = self.steps
        qgathers = self._payloads(contribs, qgathers)
        table = self._batch_table(contribs, gather, qgathers)
        s0 = ss[0]
        if table is not None and self.fused:
            zero_fused_step_shards(table, s0.dtype, s0.nranks, gather, s0.gather_dtype, s0.hp)
        elif table is not None:
            zero_reduce_grads_shards(table, s0.dtype, s0.nranks)
        else:
            self._per_rank(lambda i: ss[i].run_pieces(contribs[i], gather, qgathers[i]), branches)

    def decide(self) -> None:
        """One decision over every rank's partials, written to every rank's ctrl."""
        ss = self.steps
        zero_grad_norm_overflow([s.ws for s in ss], [s.valid_len for s in ss],
                                [s.ctrl for s in ss], ss[0].hp, self.fused)

    def complete(self, contribs, gather, qgathers=None, branches=None) -> None:
        """The rest of the step: every rank's restore check or Adam pass
        (batched when the passes were)."""
        ss = self.steps
        qgathers = self._payloads(contribs, qgathers)
        table = self._batch_table(contribs, gather, qgathers)
        if table is not None and self.fused:
            zero_fused_restore_shards(table, gather, ss[0].gather_dtype)
        elif table is not None:
            zero_adam_step_shards(table, ss[0].hp, gather, ss[0].gather_dtype)
        else:
            self._per_rank(lambda i: ss[i].complete(gather, qgathers[i]), branches)

    def capture(self, contribs, gather, qgathers=None, branches: int = 4):
        """Records one step of all the ranks (every rank's launches, the
        shared decision, every rank's completion) into a HIP graph, as
        ShardStep.capture does for one rank; ``graph.replay()`` runs a step.
        The ranks' launches are recorded on ``branches`` parallel branches
        of the graph (0 or 1: one chain), so that the small launches of
        different ranks can run at the same time."""
        import torch
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        pool = [torch.cuda.Stream() for _ in range(branches)] if branches > 1 else None
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.step(contribs, gather, qgathers, pool)
        torch.cuda.current_stream().wait_stream(side)
        return graph
