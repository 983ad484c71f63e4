"""The C ABI without a GPU: symbols, the pure-host partition, argument checks.

Every call below either needs no device (zero_partition, the size queries) or
is rejected by argument validation before anything reaches the HIP runtime.
Fake non-null device addresses are only ever passed to calls that must fail
validation.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_shard.h")


@pytest.fixture(scope="module")
def Z():
    import zero_partitioned_mixed_amd as Z
    return Z


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(zero_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(Z):
    names = declared_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", Z.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(Z.EXPORTS) == set(names)


def test_struct_sizes_match_header(Z):
    assert Z.zero_ctrl_bytes() == 128 == ctypes.sizeof(Z.Ctrl)
    assert ctypes.sizeof(Z.Hparams) == 36
    assert ctypes.sizeof(Z.State) == 24
    assert ctypes.sizeof(Z.Shard) == 96


def test_partition_matches_oracle(Z, O):
    for psi in list(range(1, 130)) + [637_824, 637_825, 124_439_808, 13_000_000_000]:
        for n in (1, 2, 3, 7, 8, 17, 32, 64):
            for r in range(n):
                assert Z.zero_partition(psi, n, r) == O.partition(psi, n, r)


@pytest.mark.parametrize("args", [(0, 4, 0), (10, 0, 0), (10, 4, 4), (10, 4, -1)])
def test_partition_rejects(Z, args):
    with pytest.raises(Z.ZeroError) as e:
        Z.zero_partition(*args)
    assert e.value.code == -1


def test_workspace_and_pair_sizes(Z):
    # one 16-byte partial per 2048-element tile plus 256 second-level slots
    assert Z.zero_workspace_bytes(0) == 256 * 16
    assert Z.zero_workspace_bytes(1) == 257 * 16
    assert Z.zero_workspace_bytes(2048) == 257 * 16
    assert Z.zero_workspace_bytes(2049) == 258 * 16
    assert Z.zero_workspace_bytes(1_625_000_000) == (793_458 + 256) * 16
    # one buffer: per tile two sets of master, m and v
    assert Z.zero_pair_elems(0) == 0
    assert Z.zero_pair_elems(1) == 6 * 2048
    assert Z.zero_pair_elems(4096) == 12 * 2048
    assert Z.zero_pair_elems(4097) == 18 * 2048


FAKE = 1 << 20  # a 16-byte aligned non-null address, never dereferenced


def _pair(Z):
    """A well-formed paired state at FAKE: m and v 2048 floats apart."""
    return Z.State(FAKE, FAKE + 4 * 2048, FAKE + 8 * 2048)


def _reduce(Z, contrib=FAKE, dtype=1, n=8, stride=64, valid=64, ctrl=FAKE, g=FAKE, ws=FAKE,
            wsb=1 << 16):
    return Z._lib.zero_reduce_grads(contrib, dtype, n, stride, valid, ctrl, g, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), -1), (dict(n=0), -1), (dict(n=1025), -1), (dict(stride=60), -1),
    (dict(stride=68, valid=64), -2), (dict(contrib=FAKE + 2), -2), (dict(g=FAKE + 4), -2),
    (dict(contrib=0), -1), (dict(g=0), -1), (dict(ctrl=0), -1), (dict(ws=0), -1),
    (dict(wsb=4096), -4), (dict(valid=-1), -3), (dict(ctrl=FAKE + 4), -2),
])
def test_reduce_validation(Z, kw, code):
    assert _reduce(Z, **kw) == code
    assert Z.zero_last_error() != ""


def test_fused_rejects_clipping_and_a_bad_paired_state(Z):
    pair = _pair(Z)
    hp = Z.hparams(max_grad_norm=1.0)
    rc = Z._lib.zero_fused_step(FAKE, 1, 8, 64, ctypes.byref(pair), 64, FAKE, 1, 0,
                                ctypes.byref(hp), FAKE, FAKE, 1 << 20, None)
    assert rc == -1 and "two-pass" in Z.zero_last_error()
    hp = Z.hparams()
    # a paired state is one buffer: m and v one and two tiles of 2048 floats past master
    for bad in (Z.State(FAKE, FAKE, FAKE + 16384), Z.State(FAKE, FAKE + 65536, FAKE + 131072),
                Z.State(FAKE, FAKE + 8192, FAKE + 8192), Z.State(FAKE, FAKE + 8192, 0)):
        rc = Z._lib.zero_fused_step(FAKE, 1, 8, 64, ctypes.byref(bad), 64, FAKE, 1, 0,
                                    ctypes.byref(hp), FAKE, FAKE, 1 << 20, None)
        assert rc == -1 and "one buffer" in Z.zero_last_error()
    odd = Z.State(FAKE + 4, FAKE + 4 + 8192, FAKE + 4 + 16384)
    rc = Z._lib.zero_fused_step(FAKE, 1, 8, 64, ctypes.byref(odd), 64, FAKE, 1, 0,
                                ctypes.byref(hp), FAKE, FAKE, 1 << 20, None)
    assert rc == -2
    rc = Z._lib.zero_fused_step(FAKE, 1, 8, 64, ctypes.byref(pair), 64, FAKE, 1, 0,
                                ctypes.byref(hp), FAKE, FAKE, 16, None)
    assert rc == -4  # workspace too small


def test_fused_noalloc_validation(Z):
    """The allocation-free step rejects its arguments before it looks up its
    scratch array or enqueues anything: sizes beyond the array, clipping, a
    bad paired state, null ctrl and gather."""
    pair, hp = _pair(Z), Z.hparams()

    def call(valid=64, stride=64, hp=hp, pair=pair, ctrl=FAKE, gather=FAKE):
        return Z._lib.zero_fused_step_noalloc(FAKE, 1, 8, stride, ctypes.byref(pair), valid, gather,
                                              1, 0, ctypes.byref(hp), ctrl, None)

    big = Z.NOALLOC_MAX_LEN + 8
    assert call(valid=big, stride=big) == -3
    assert "ZERO_NOALLOC_MAX_LEN" in Z.zero_last_error()
    assert call(hp=Z.hparams(max_grad_norm=1.0)) == -1 and "two-pass" in Z.zero_last_error()
    assert call(pair=Z.State(FAKE, FAKE, FAKE + 16384)) == -1
    assert call(ctrl=0) == -1
    assert call(gather=0) == -1
    assert call(stride=60) == -1


def _shard(Z, **kw):
    """A well-formed zero_shard of 64 elements at fake addresses, with changes."""
    d = dict(contrib=FAKE, stride=64, pair=FAKE, valid_len=64, offset=0, ctrl=FAKE, ws=FAKE,
             ws_bytes=Z.zero_workspace_bytes(64), state=(FAKE, FAKE + 256, FAKE + 512),
             g=FAKE + 768)
    d.update(kw)
    return Z.Shard(d["contrib"], d["stride"], d["pair"], d["valid_len"], d["offset"], d["ctrl"],
                   d["ws"], d["ws_bytes"], Z.State(*d["state"]), d["g"])


def test_batched_shards_validation(Z):
    """The batched fused step and restore check every shard before anything
    is enqueued: the shard count, each shard's rows, state, workspace, ctrl
    and slot, and that each shard fits one launch."""
    hp = Z.hparams()

    def fused(shards, n=8, hp=hp, gather=FAKE, table=True):
        arr = (Z.Shard * max(len(shards), 1))(*shards)
        return Z._lib.zero_fused_step_shards(arr if table else None, len(shards), 1, n, gather, 1,
                                             ctypes.byref(hp), None)

    def restore(shards, gather=FAKE):
        arr = (Z.Shard * max(len(shards), 1))(*shards)
        return Z._lib.zero_fused_restore_shards(arr, len(shards), gather, 1, None)

    good = _shard(Z)
    assert fused([good], table=False) == -1
    assert fused([]) == -1 and fused([good] * 65) == -1
    assert fused([good], hp=Z.hparams(max_grad_norm=1.0)) == -1
    assert "two-pass" in Z.zero_last_error()
    assert fused([good], gather=0) == -1
    # each shard at most one launch of tiles: 32,768 at N = 8, 2,048 at N = 64
    for n in (8, 64):
        top = Z.launch_tiles(n) * Z.TILE
        big = _shard(Z, valid_len=top + 1, stride=top + 8,
                     ws_bytes=Z.zero_workspace_bytes(top + 1))
        assert fused([good, big], n=n) == -3 and "shard 1" in Z.zero_last_error()
    bad = [_shard(Z, contrib=0), _shard(Z, contrib=FAKE + 8), _shard(Z, stride=68),
           _shard(Z, stride=32), _shard(Z, pair=0), _shard(Z, pair=FAKE + 4), _shard(Z, ctrl=0),
           _shard(Z, ctrl=FAKE + 4), _shard(Z, ws=0), _shard(Z, ws_bytes=16),
           _shard(Z, offset=-1), _shard(Z, valid_len=-1)]
    codes = [fused([good, b, good]) for b in bad]
    assert codes == [-1, -2, -2, -1, -1, -1, -1, -2, -1, -4, -3, -3], codes
    # the restore: at most ZERO_LAUNCH_TILES tiles a shard, and its state, slot and ctrl
    top = Z.LAUNCH_TILES * Z.TILE
    assert restore([good, _shard(Z, valid_len=top + 1)]) == -3
    assert restore([_shard(Z, pair=0)]) == -1 and restore([_shard(Z, ctrl=0)]) == -1
    assert restore([good], gather=0) == -1 and restore([good] * 65) == -1


def test_batched_two_pass_validation(Z):
    """The batched reduce and Adam passes check every shard before anything is
    enqueued: rows, workspace and g for the reduce, flat state and g for the
    Adam pass, ctrl and the slot (the Adam pass may write none), and that
    each shard fits one launch."""
    hp = Z.hparams(max_grad_norm=1.0)

    def reduce(shards, n=8):
        arr = (Z.Shard * max(len(shards), 1))(*shards)
        return Z._lib.zero_reduce_grads_shards(arr, len(shards), 1, n, None)

    def adam(shards, gather=FAKE, hp=hp, gdt=1):
        arr = (Z.Shard * max(len(shards), 1))(*shards)
        return Z._lib.zero_adam_step_shards(arr, len(shards), ctypes.byref(hp), gather, gdt, None)

    good = _shard(Z)
    assert reduce([]) == -1 and reduce([good] * 65) == -1
    top = Z.launch_tiles(64) * Z.TILE
    big = _shard(Z, valid_len=top + 1, stride=top + 8, ws_bytes=Z.zero_workspace_bytes(top + 1))
    assert reduce([good, big], n=64) == -3
    codes = [reduce([good, b]) for b in (_shard(Z, contrib=0), _shard(Z, contrib=FAKE + 8),
                                         _shard(Z, stride=68), _shard(Z, ws=0),
                                         _shard(Z, ws_bytes=16), _shard(Z, g=0),
                                         _shard(Z, g=FAKE + 4), _shard(Z, ctrl=0))]
    assert codes == [-1, -2, -2, -1, -4, -1, -1, -1], codes
    assert adam([good] * 65) == -1
    assert adam([good], hp=Z.hparams(beta1=1.0)) == -1
    assert adam([good, _shard(Z, valid_len=Z.LAUNCH_TILES * Z.TILE + 1)]) == -3
    codes = [adam([good, b]) for b in (_shard(Z, g=0), _shard(Z, state=(0, FAKE, FAKE + 256)),
                                       _shard(Z, state=(FAKE, FAKE, FAKE + 256)),
                                       _shard(Z, state=(FAKE + 4, FAKE + 256, FAKE + 512)),
                                       _shard(Z, ctrl=0), _shard(Z, offset=-1))]
    assert codes == [-1, -1, -1, -2, -1, -3], codes
    assert adam([_shard(Z, g=0)], gather=None) == -1   # no slot: the rest still checked
    assert adam([good], gather=None, gdt=7) == -1


def test_hparam_validation(Z):
    s0 = Z.State(FAKE, FAKE + 256, FAKE + 512)
    for hp in (Z.hparams(beta1=1.0), Z.hparams(eps=-1.0), Z.hparams(scaler=7),
               Z.hparams(scaler=2, growth_interval=0)):
        rc = Z._lib.zero_adam_step(ctypes.byref(s0), FAKE, 64, ctypes.byref(hp), FAKE, None, 1, 0,
                                   None)
        assert rc == -1


def test_norm_overflow_validation(Z):
    hp = Z.hparams()
    arr = (ctypes.c_void_p * 1)(FAKE)
    lens = (ctypes.c_int64 * 1)(64)
    assert Z._lib.zero_grad_norm_overflow(0, arr, lens, arr, ctypes.byref(hp), 0, None) == -1
    assert Z._lib.zero_grad_norm_overflow(65, arr, lens, arr, ctypes.byref(hp), 0, None) == -1
    nul = (ctypes.c_void_p * 1)(None)
    assert Z._lib.zero_grad_norm_overflow(1, arr, lens, nul, ctypes.byref(hp), 0, None) == -1


def test_slot_and_ctrl_validation(Z):
    assert Z._lib.zero_cast_to_gather(FAKE, 64, FAKE + 1, 1, 0, None) == -2  # odd gather address
    assert Z._lib.zero_cast_to_gather(FAKE, 64, FAKE, 1, -5, None) == -3
    assert Z._lib.zero_cast_to_gather(FAKE, 64, FAKE, 9, 0, None) == -1
    assert Z._lib.zero_ctrl_init(FAKE, ctypes.c_float(0.0), None) == -1
    assert Z._lib.zero_ctrl_init(FAKE, ctypes.c_float(float("inf")), None) == -1
    assert Z._lib.zero_ctrl_init(None, ctypes.c_float(1.0), None) == -1


def test_binding_refuses_cpu_tensors(Z):
    import torch
    with pytest.raises(ValueError):
        Z.zero_cast_to_gather(torch.zeros(8), 8, torch.zeros(8, dtype=torch.int16), Z.F16, 0)


def _rows_call(Z, fused, rows, n=None, dtype=1, valid=64, ctrl=FAKE, g=FAKE, wsb=1 << 16):
    n = len(rows) if n is None else n
    arr = (ctypes.c_void_p * max(len(rows), 1))(*rows) if rows is not None else None
    if not fused:
        return Z._lib.zero_reduce_grads_rows(arr, dtype, n, valid, ctrl, g, FAKE, wsb, None)
    pair = _pair(Z)
    hp = Z.hparams()
    return Z._lib.zero_fused_step_rows(arr, dtype, n, ctypes.byref(pair), valid, FAKE, 1, 0,
                                       ctypes.byref(hp), ctrl, FAKE, wsb, None)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("rows,kw,code,msg", [
    (None, dict(n=8), -1, "null row table"),
    ([FAKE] * 8, dict(n=0), -1, "outside"),
    ([FAKE] * 65, dict(), -1, "outside"),                   # more rows than a table holds
    ([FAKE, FAKE, 0, FAKE], dict(), -1, "row 2 is null"),
    ([FAKE, FAKE + 4], dict(), -2, "row 1 not 8-byte"),      # 4-byte aligned only
    ([FAKE] * 4, dict(dtype=5), -1, "dtype"),
    ([FAKE] * 4, dict(valid=-3), -3, "out of range"),
    ([FAKE] * 4, dict(wsb=16), -4, "workspace"),
    ([FAKE] * 4, dict(ctrl=0), -1, "ctrl"),
])
def test_row_table_validation(Z, fused, rows, kw, code, msg):
    assert _rows_call(Z, fused, rows, **kw) == code
    assert msg in Z.zero_last_error()


def test_row_table_accepts_8_byte_aligned_rows(Z):
    # 8-byte aligned rows (a peer slice at an odd multiple of 4 elements) pass
    # every check; only a misaligned g then stops the call before any launch.
    assert _rows_call(Z, False, [FAKE + 8, FAKE + 24, FAKE], g=FAKE + 4) == -2
    assert "g not 16-byte" in Z.zero_last_error()


def test_quant_sizes(Z):
    assert Z.zero_qblock_count(0) == 0 and Z.zero_qblock_count(1) == 1
    assert Z.zero_qblock_count(2048) == 1 and Z.zero_qblock_count(2049) == 2
    assert Z.zero_qcode_bytes(5, 8) == 5 and Z.zero_qcode_bytes(5, 4) == 3
    assert Z.zero_qcode_bytes(4, 4) == 2 and Z.zero_qcode_bytes(-1, 8) == 0
    assert ctypes.sizeof(ctypes.c_float) + ctypes.sizeof(ctypes.c_int32) == 8  # zero_qblock


def test_quantize_validation(Z):
    L = Z._lib
    assert L.zero_quantize_blocks(FAKE, 1, 64, 3, FAKE, FAKE, None) == -1          # bits
    assert L.zero_quantize_blocks(FAKE, 7, 64, 8, FAKE, FAKE, None) == -1          # dtype
    assert L.zero_quantize_blocks(0, 1, 64, 8, FAKE, FAKE, None) == -1
    assert L.zero_quantize_blocks(FAKE + 1, 1, 64, 8, FAKE, FAKE, None) == -2      # odd src
    assert L.zero_quantize_blocks(FAKE + 2, 1, 64, 8, FAKE + 4, FAKE, None) == -2  # codes
    assert L.zero_quantize_blocks(FAKE, 1, 64, 4, FAKE + 4, FAKE, None) == -2
    assert L.zero_quantize_blocks(FAKE, 1, -5, 8, FAKE, FAKE, None) == -3
    assert L.zero_dequantize_blocks(FAKE, FAKE, 4, 64, FAKE + 7, 1, None) == -2    # odd dst
    assert L.zero_dequantize_blocks(FAKE, FAKE + 2, 4, 64, FAKE + 6, 1, None) == -2  # blocks
    assert L.zero_dequantize_blocks(FAKE, FAKE, 2, 64, FAKE, 1, None) == -1
    assert L.zero_dequantize_blocks(FAKE, None, 8, 64, FAKE, 2, None) == -1


def _q_call(Z, fused, codes, blocks, bits=8, n=None, valid=64, g=FAKE, wsb=1 << 16):
    n = len(codes) if n is None else n
    ca = (ctypes.c_void_p * max(len(codes), 1))(*codes) if codes is not None else None
    ba = (ctypes.c_void_p * max(len(blocks), 1))(*blocks) if blocks is not None else None
    if not fused:
        return Z._lib.zero_reduce_grads_q(ca, ba, bits, n, valid, FAKE, g, FAKE, wsb, None)
    pair = _pair(Z)
    hp = Z.hparams()
    return Z._lib.zero_fused_step_q(ca, ba, bits, n, ctypes.byref(pair), valid, FAKE, 1, 0,
                                    ctypes.byref(hp), FAKE, FAKE, wsb, None)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("codes,blocks,kw,code,msg", [
    ([FAKE] * 2, [FAKE] * 2, dict(bits=2), -1, "bits"),
    (None, [FAKE], dict(n=1), -1, "null row table"),
    ([FAKE] * 2, None, dict(n=2), -1, "null row table"),
    ([FAKE] * 65, [FAKE] * 65, dict(), -1, "outside"),
    ([FAKE, 0], [FAKE, FAKE], dict(), -1, "row 1 is null"),
    ([FAKE, FAKE], [FAKE, 0], dict(), -1, "row 1 is null"),
    ([FAKE, FAKE + 4], [FAKE, FAKE], dict(), -2, "row 1 not 8-byte"),
    ([FAKE, FAKE], [FAKE + 4, FAKE], dict(), -2, "row 0 not 8-byte"),
    ([FAKE] * 2, [FAKE] * 2, dict(valid=-1), -3, "out of range"),
    ([FAKE] * 2, [FAKE] * 2, dict(wsb=16), -4, "workspace"),
])
def test_quant_rows_validation(Z, fused, codes, blocks, kw, code, msg):
    assert _q_call(Z, fused, codes, blocks, **kw) == code
    assert msg in Z.zero_last_error()


def _qg_call(Z, form="strided", contrib_dtype=1, valid=64, gather=FAKE, gdt=1, bits=8,
             codes=FAKE, blocks=FAKE, clip=0.0, wsb=1 << 16, ctrl=FAKE, table=None, qbits=8):
    pair = _pair(Z)
    hp = Z.hparams(max_grad_norm=clip)
    tail = (gather, gdt, 0, bits, codes, blocks, ctypes.byref(hp), ctrl, FAKE, wsb, None)
    if form == "strided":
        return Z._lib.zero_fused_step_qgather(FAKE, contrib_dtype, 8, 64, ctypes.byref(pair),
                                              valid, *tail)
    rows = [FAKE] * 4 if table is None else table
    arr = (ctypes.c_void_p * max(len(rows), 1))(*rows)
    if form == "rows":
        return Z._lib.zero_fused_step_rows_qgather(arr, contrib_dtype, len(rows),
                                                   ctypes.byref(pair), valid, *tail)
    blk = (ctypes.c_void_p * max(len(rows), 1))(*([FAKE] * len(rows)))
    return Z._lib.zero_fused_step_q_qgather(arr, blk, qbits, len(rows), ctypes.byref(pair), valid,
                                            *tail)


@pytest.mark.parametrize("form", ["strided", "rows", "q"])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(bits=3), -1, "bits"),
    (dict(bits=16), -1, "bits"),
    (dict(codes=0), -1, "null codes"),
    (dict(blocks=0), -1, "null codes"),
    (dict(codes=FAKE + 4), -2, "8-byte"),
    (dict(blocks=FAKE + 2), -2, "8-byte"),
    (dict(gather=FAKE + 1), -2, "2-byte"),
    (dict(gather=None, gdt=9), -1, "gather dtype"),
    (dict(gdt=0), -1, "gather dtype"),
    (dict(clip=1.0), -1, "two-pass"),
    (dict(contrib_dtype=3), -1, "dtype"),
    (dict(valid=-1), -3, "out of range"),
    (dict(ctrl=0), -1, "null ctrl"),
    (dict(wsb=16), -4, "workspace"),
    # a NULL gather is accepted: validation runs on to the workspace check
    (dict(gather=None, wsb=16), -4, "workspace"),
])
def test_fused_qgather_validation(Z, form, kw, code, msg):
    if form == "q" and "contrib_dtype" in kw:
        pytest.skip("quantised contributions carry no 16-bit dtype")
    assert _qg_call(Z, form, **kw) == code
    assert msg in Z.zero_last_error()


@pytest.mark.parametrize("form,kw,code,msg", [
    ("rows", dict(table=[FAKE, 0, FAKE]), -1, "row 1 is null"),
    ("rows", dict(table=[FAKE, FAKE + 4]), -2, "row 1 not 8-byte"),
    ("rows", dict(table=[FAKE] * 65), -1, "outside"),
    ("q", dict(qbits=2), -1, "bits"),
    ("q", dict(table=[FAKE, FAKE + 4]), -2, "row 1 not 8-byte"),
    ("q", dict(table=[0, FAKE]), -1, "row 0 is null"),
])
def test_fused_qgather_source_validation(Z, form, kw, code, msg):
    """The row-table and quantised-row forms check their source as the
    corresponding plain fused calls do."""
    assert _qg_call(Z, form, **kw) == code
    assert msg in Z.zero_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(bits=5), -1, "bits"),
    (dict(codes=0), -1, "null codes"),
    (dict(blocks=FAKE + 4), -2, "8-byte"),
    (dict(gather=None, dtype=9), -1, "gather dtype"),
    (dict(gather=FAKE + 1), -2, "2-byte"),
    (dict(ctrl=0), -1, "null ctrl"),
    (dict(valid=-3), -3, "out of range"),
])
def test_fused_restore_q_validation(Z, kw, code, msg):
    a = dict(valid=64, gather=FAKE, dtype=1, bits=8, codes=FAKE, blocks=FAKE, ctrl=FAKE)
    a.update(kw)
    pair = _pair(Z)
    rc = Z._lib.zero_fused_restore_q(ctypes.byref(pair), a["valid"], a["gather"], a["dtype"], 0,
                                     a["bits"], a["codes"], a["blocks"], a["ctrl"], None)
    assert rc == code
    assert msg in Z.zero_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(bits=2), -1, "bits"),
    (dict(codes=0), -1, "null codes"),
    (dict(blocks=FAKE + 4), -2, "8-byte"),
    (dict(gather=None, gdt=0), -1, "gather dtype"),
    (dict(gather=FAKE + 1), -2, "2-byte"),
    (dict(g=0), -1, "null g"),
    (dict(g=FAKE + 8), -2, "g not 16-byte"),
    (dict(ctrl=0), -1, "null ctrl"),
    (dict(valid=-2), -3, "out of range"),
])
def test_adam_qgather_validation(Z, kw, code, msg):
    a = dict(valid=64, g=FAKE, gather=FAKE, gdt=1, bits=8, codes=FAKE, blocks=FAKE, ctrl=FAKE)
    a.update(kw)
    s0 = Z.State(FAKE, FAKE + 256, FAKE + 512)
    hp = Z.hparams(max_grad_norm=1.0)
    rc = Z._lib.zero_adam_step_qgather(ctypes.byref(s0), a["g"], a["valid"], ctypes.byref(hp),
                                       a["ctrl"], a["gather"], a["gdt"], 0, a["bits"], a["codes"],
                                       a["blocks"], None)
    assert rc == code
    assert msg in Z.zero_last_error()
