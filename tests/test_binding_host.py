"""Host-side logic of the Python binding, without a GPU: the constants that
mirror include/zero_shard.h, the number of launches a pass is issued as, and
the pieces and pointer advances of a bucketed step (the header's bucket
contract: every per-element pointer advanced by the piece's first element,
codes by bytes, block records by whole blocks)."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def Z():
    import zero_partitioned_mixed_amd as Z
    return Z


def _header_define(name):
    text = open(os.path.join(ROOT, "include", "zero_shard.h")).read()
    m = re.search(rf"^#define {name} (\d+)", text, re.M)
    assert m, name
    return int(m.group(1))


def test_constants_match_header(Z):
    assert Z.TILE == _header_define("ZERO_TILE")
    assert Z.QBLOCK == _header_define("ZERO_QBLOCK")
    assert Z.PARTIAL_BYTES == _header_define("ZERO_PARTIAL_BYTES")
    assert Z.LAUNCH_TILES == _header_define("ZERO_LAUNCH_TILES")
    assert Z.LAUNCH_ROW_TILES == _header_define("ZERO_LAUNCH_ROW_TILES")
    assert Z.LAUNCH_MIN_TILES == _header_define("ZERO_LAUNCH_MIN_TILES")
    assert Z.LAUNCH_PAYLOAD_TILES == _header_define("ZERO_LAUNCH_PAYLOAD_TILES")
    assert Z.MAX_RANKS == _header_define("ZERO_MAX_RANKS")
    assert Z.NOALLOC_MAX_LEN == _header_define("ZERO_NOALLOC_MAX_LEN")
    assert Z.BATCH_SHARDS == _header_define("ZERO_BATCH_SHARDS")
    # one workspace partial per tile: the workspace grows by PARTIAL_BYTES per tile
    assert Z.zero_workspace_bytes(3 * Z.TILE) - Z.zero_workspace_bytes(Z.TILE) == 2 * Z.PARTIAL_BYTES


@pytest.mark.parametrize("valid,nranks,expected", [
    (0, 0, 0), (1, 0, 1), (2048, 0, 1), (32768 * 2048, 0, 1), (32768 * 2048 + 1, 0, 2),
    (1_625_000_000, 0, 25), (1_625_000_000, 8, 25), (875_000_000, 8, 14),
    (15_554_976, 8, 1), (23_437_500, 64, 6), (23_437_500, 0, 1), (23_437_500, 32, 3),
    (5461 * 2048, 24, 1), (5461 * 2048 + 1, 24, 2), (2048 * 2048 + 1, 1024, 2),
    (14563 * 2048 + 1, 9, 2),
])
def test_launches_per_pass(Z, valid, nranks, expected):
    assert Z.launches(valid, nranks) == expected


@pytest.mark.parametrize("valid,nranks,expected", [
    (1_625_000_000, 8, 49), (16384 * 2048 + 1, 1, 2), (23_437_500, 64, 6), (8192 * 2048, 16, 1),
])
def test_launches_of_the_fused_payload_pass(Z, valid, nranks, expected):
    assert Z.launches(valid, nranks, payload=True) == expected


def test_launch_tiles_match_the_library(Z):
    """The binding's launch size (used for launch counts in profiles) is the
    library's own, for every row count a call accepts and beyond."""
    for n in list(range(-2, 1100)) + [4096, 1 << 20]:
        assert Z.launch_tiles(n) == Z._lib.zero_launch_tiles(n), n
    assert [Z.launch_tiles(n) for n in (0, 1, 8, 9, 16, 24, 32, 64, 65, 1024)] == \
        [32768, 32768, 32768, 14563, 8192, 5461, 4096, 2048, 2048, 2048]


def _step(Z, valid, bucket):
    st = object.__new__(Z.ShardStep)   # no device state: only the piece logic is used
    st.valid_len, st.bucket = valid, bucket
    return st


@pytest.mark.parametrize("valid,bucket", [
    (0, 0), (5, 0), (5, 2048), (2048, 2048), (2049, 2048), (100_003, 2048 * 3),
    (1_625_000_000, 499_998_720),
])
def test_pieces_cover_the_shard_in_order(Z, valid, bucket):
    pieces = _step(Z, valid, bucket).pieces()
    assert pieces[0][0] == 0
    assert sum(n for _, n in pieces) == valid
    for (b0, n), (b1, _) in zip(pieces, pieces[1:]):
        assert b1 == b0 + n and b0 % Z.TILE == 0 and b1 % Z.TILE == 0
    if bucket and valid > bucket:
        assert all(n == bucket for _, n in pieces[:-1]) and 0 < pieces[-1][1] <= bucket
    else:
        assert pieces == [(0, valid)]


def test_bucket_must_be_whole_tiles(Z):
    hp = Z.hparams()
    with pytest.raises(ValueError):
        Z.ShardStep(8, 64, 64, 0, Z.F16, Z.F16, hp, (None, None, None), bucket=1000)


def test_piece_pointer_advances(Z):
    b0 = 3 * Z.TILE
    rows = Z.ShardStep._contrib_at([1 << 20, 1 << 24], b0)
    assert rows == [(1 << 20) + 2 * b0, (1 << 24) + 2 * b0]        # 16-bit elements
    for bits, code_bytes in ((8, b0), (4, b0 // 2)):
        q = Z.ShardStep._contrib_at(Z.QuantRows([(1 << 20, 1 << 22)], bits), b0)
        assert q.bits == bits
        assert q.rows == [((1 << 20) + code_bytes, (1 << 22) + 8 * (b0 // Z.QBLOCK))]
        g = Z.QGather(1 << 20, 1 << 22, bits, 100_000).at(b0)
        assert (g.codes, g.blocks, g.bits, g.length) == \
            ((1 << 20) + code_bytes, (1 << 22) + 8 * (b0 // Z.QBLOCK), bits, 100_000 - b0)


def test_one_hip_runtime_whatever_the_import_order():
    """Imported before torch, the binding and the device input generator still
    leave one HIP runtime in the process (torch's): with two, the library's
    runtime finds no device."""
    code = ("import zero_partitioned_mixed_amd, synth; synth.gpu(); import torch; "
            "import json; print(json.dumps(sorted({l.split()[-1] for l in open('/proc/self/maps') "
            "if 'libamdhip64' in l})))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    paths = json.loads(r.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths


ENTRY_POINTS = ["zero_fused_step", "zero_fused_step_rows", "zero_fused_step_q",
                "zero_fused_step_qgather", "zero_fused_step_rows_qgather",
                "zero_fused_step_q_qgather", "zero_reduce_grads", "zero_reduce_grads_rows",
                "zero_reduce_grads_q", "zero_grad_norm_overflow", "zero_fused_restore",
                "zero_fused_restore_q", "zero_adam_step", "zero_adam_step_qgather",
                "zero_fused_step_shards", "zero_fused_restore_shards", "zero_reduce_grads_shards",
                "zero_adam_step_shards"]


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("source", ["strided", "rows", "quant"])
@pytest.mark.parametrize("payload", [False, True])
def test_shard_step_routes_each_form_to_its_call(Z, monkeypatch, fused, source, payload):
    """ShardStep.step issues, for every contribution form, payload choice and
    path, the calls the header pairs with them: the per-element pass, the
    decision, then the restore (fused) or the Adam pass (two-pass)."""
    calls = []
    for name in ENTRY_POINTS:
        monkeypatch.setattr(Z, name, lambda *a, _n=name, **k: calls.append(_n))
    st = _fake_step(Z, fused)
    contrib = {"strided": object(), "rows": [1 << 20, 1 << 21],
               "quant": Z.QuantRows([(1 << 20, 1 << 22), (1 << 21, 1 << 23)], 8)}[source]
    qg = Z.QGather(1 << 24, 1 << 25, 8, 4096) if payload else None
    st.step(contrib, "gather", qg)
    suffix = {"strided": "", "rows": "_rows", "quant": "_q"}[source]
    if fused:
        first = "zero_fused_step" + suffix + ("_qgather" if payload else "")
        last = "zero_fused_restore_q" if payload else "zero_fused_restore"
    else:
        first = "zero_reduce_grads" + suffix
        last = "zero_adam_step_qgather" if payload else "zero_adam_step"
    assert calls == [first, "zero_grad_norm_overflow", last]


def test_shard_step_rejects_a_row_count_mismatch(Z):
    st = object.__new__(Z.ShardStep)
    st.nranks, st.fused = 3, True
    with pytest.raises(ValueError):
        st.run_pieces([1 << 20, 1 << 21], "gather")
    with pytest.raises(ValueError):
        st.run_pieces(Z.QuantRows([(1 << 20, 1 << 22)], 4), "gather")


def _fake_step(Z, fused, clip=1.0):
    st = object.__new__(Z.ShardStep)
    st.bucket, st.nranks, st.stride, st.valid_len, st.offset = 0, 2, 4096, 4096, 0
    st.dtype = st.gather_dtype = Z.F16
    st.hp = Z.hparams(max_grad_norm=0.0 if fused else clip)
    st.fused = fused
    st.state, st.g, st.ctrl, st.ws = ("m0", "m1", "m2"), "g", "ctrl", "ws"
    st.pair = ("p0", "p1", "p2") if fused else None
    return st


def test_multi_shard_step_runs_every_rank_then_one_decision(Z, monkeypatch):
    """Each rank's per-element pass (its own form and payload), one combined
    decision, then each rank's restore."""
    calls = []
    for name in ENTRY_POINTS:
        monkeypatch.setattr(Z, name, lambda *a, _n=name, **k: calls.append(_n))
    multi = Z.MultiShardStep([_fake_step(Z, True), _fake_step(Z, True)])
    qrows = Z.QuantRows([(1 << 20, 1 << 22), (1 << 21, 1 << 23)], 8)
    multi.step([object(), qrows], "gather", [None, Z.QGather(1 << 24, 1 << 25, 8, 4096)])
    assert calls == ["zero_fused_step", "zero_fused_step_q_qgather", "zero_grad_norm_overflow",
                     "zero_fused_restore", "zero_fused_restore_q"]


class _FakeRows:
    """Stands in for a [N, stride] contribution tensor (only its address is read)."""

    def data_ptr(self):
        return id(self)


def test_multi_shard_step_batches_small_fused_shards(Z, monkeypatch):
    """Ranks with one [N, stride] tensor each, no payload, no buckets and
    shards of at most one launch go through the batched calls, on the fused
    path (with a 16-bit slot) and on the two-pass path: three launches a step
    whatever the rank count; any other step, or batched=False, through every
    rank's own calls."""
    calls = []
    for name in ENTRY_POINTS:
        monkeypatch.setattr(Z, name, lambda *a, _n=name, **k: calls.append(_n))
    monkeypatch.setattr(Z, "shard_table", lambda shards: list(shards))
    ranks = [_fake_step(Z, True) for _ in range(5)]
    rows = [_FakeRows() for _ in ranks]
    multi = Z.MultiShardStep(ranks)
    assert multi.takes_batched(rows, "gather")
    multi.step(rows, "gather")
    assert calls == ["zero_fused_step_shards", "zero_grad_norm_overflow",
                     "zero_fused_restore_shards"]
    per_rank = ["zero_fused_step"] * 5 + ["zero_grad_norm_overflow"] + ["zero_fused_restore"] * 5
    calls.clear()
    Z.MultiShardStep(ranks, batched=False).step(rows, "gather")
    assert calls == per_rank
    calls.clear()
    Z.MultiShardStep([_fake_step(Z, False) for _ in range(5)]).step(rows, "gather")
    assert calls == ["zero_reduce_grads_shards", "zero_grad_norm_overflow",
                     "zero_adam_step_shards"]
    for change in ("table", "bucket", "long", "payload"):
        calls.clear()
        rs = [_fake_step(Z, True) for _ in range(5)]
        contribs, qgs = list(rows), None
        if change == "table":
            contribs[2] = [1 << 20, 1 << 21]
        elif change == "bucket":
            rs[3].bucket = Z.TILE
        elif change == "long":
            rs[4].valid_len = Z.launch_tiles(2) * Z.TILE + 1
        elif change == "payload":
            qgs = [None] * 4 + [Z.QGather(1 << 24, 1 << 25, 8, 4096)]
        multi = Z.MultiShardStep(rs)
        assert not multi.takes_batched(contribs, "gather", qgs), change
        if change in ("bucket", "long"):
            continue  # the fake ranks would issue pieces; the routing is what is checked
        multi.step(contribs, "gather", qgs)
        assert "zero_fused_step_shards" not in calls and "zero_grad_norm_overflow" in calls, change


def test_multi_shard_step_validation(Z):
    with pytest.raises(ValueError):
        Z.MultiShardStep([])
    with pytest.raises(ValueError):  # one decision, one set of hyperparameters
        Z.MultiShardStep([_fake_step(Z, False, 1.0), _fake_step(Z, False, 0.5)])
    multi = Z.MultiShardStep([_fake_step(Z, True), _fake_step(Z, True)])
    with pytest.raises(ValueError):
        multi.step([object()], "gather")
    with pytest.raises(ValueError):
        multi.step([object(), object()], "gather", [None])
