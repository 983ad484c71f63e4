"""Every compiled form of the fused step, each against the oracle.

The fused kernels are instantiated per 16-bit slot format, slot store width
(8-, 4- or 2-byte aligned slot: 4, 2 or 1 values per store), row count (the
N = 8 kernel and the one for any N) and contribution source (fp16 or bf16
rows, strided or through a row table; INT8 or INT4 blocks), and the ones
that also write the quantised all-gather payload per slot format, row count,
source and payload width.  Each case here selects one instantiation by its
arguments and runs two steps of a small shard (two whole tiles and a ragged
one) against the oracle; a kernel trace of the GPU suite lists every
instantiation of the library as launched.  Also the two-pass step without a
16-bit slot (the Adam pass then writes the state only).
"""
import itertools

import pytest

import harness as H
from harness import Case
from synth.workloads import BF16, F16, Workload

pytestmark = pytest.mark.gpu

# shard length per slot store width: rank 1's slot starts at element `shard`
# of the 256-byte aligned gather buffer, so 5000 -> 8-byte, 5002 -> 4-byte and
# 5001 -> 2-byte aligned
SHARD = {4: 5000, 2: 5002, 1: 5001}
# contribution source: (contribution format, layout, block bits)
SOURCES = {"f16": (F16, "strided", 0), "bf16": (BF16, "strided", 0),
           "f16_table": (F16, "rows", 0), "bf16_table": (BF16, "rows", 0),
           "int8": (F16, "strided", 8), "int4": (BF16, "strided", 4)}
FORMATS = {"f16": F16, "bf16": BF16}


def _case(src, slot_fmt, n, shard):
    dt, layout, qbits = SOURCES[src]
    w = Workload(name="inst", psi=n * shard, nranks=n, ranks=(1,), dtype=dt, steps=2,
                 gather_dtype=FORMATS[slot_fmt])
    return Case(w, 1, 2, qbits=qbits), layout


@pytest.mark.parametrize("src,slot_fmt,gw,n", list(itertools.product(SOURCES, FORMATS,
                                                                        (4, 2, 1), (8, 3))))
def test_fused_instantiation(src, slot_fmt, gw, n):
    c, layout = _case(src, slot_fmt, n, SHARD[gw])
    slot_byte = 2 * c.part[1]  # from the 256-byte aligned start of the gather buffer
    assert gw == (4 if slot_byte % 8 == 0 else 2 if slot_byte % 4 == 0 else 1)
    H.run_and_compare(c, f"fused {src} -> {slot_fmt} gw{gw} n{n}", layout=layout)


@pytest.mark.parametrize("src,slot_fmt,n,bits", list(itertools.product(SOURCES, FORMATS, (8, 3),
                                                                         (8, 4))))
def test_fused_payload_instantiation(src, slot_fmt, n, bits):
    c, layout = _case(src, slot_fmt, n, SHARD[1 if n == 3 else 4])
    H.run_and_compare(c, f"fused payload{bits} {src} -> {slot_fmt} n{n}", layout=layout,
                      qgather=bits, write_slot=(n == 8))


@pytest.mark.parametrize("dt", [F16, BF16])
def test_two_pass_without_slot(dt):
    """zero_adam_step with no gather buffer: the state only, the whole gather
    buffer untouched."""
    w = Workload(name="noslot", psi=8 * 5001, nranks=8, ranks=(1,), dtype=dt, steps=3,
                 max_grad_norm=0.05)
    H.run_and_compare(Case(w, 1, 3), f"two-pass without slot dtype {dt}", write_slot=False)
