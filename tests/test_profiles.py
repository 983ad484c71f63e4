"""The committed rocprofv3 summaries describe the library as built from these
sources: every counter summary names a kernel of libzero_shard.so whose
machine code (SHA-256 of its gfx950 assembly, written by the build) is the
one the counters were taken on, and every summary gives the command that
made it.  bench.py reports the measured traffic only under the same digest
check, so a kernel changed without new counters shows up here first."""
import glob
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def _fields(path):
    out = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            out[k.strip()] = v.strip().strip("`")
    return out


@pytest.fixture(scope="module")
def isa():
    from zero_partitioned_mixed_amd import build as zb
    if not os.path.exists(zb.ISA_JSON):
        pytest.skip("the library's digests are written by __graft_entry__.build()")
    return json.load(open(zb.ISA_JSON))


def test_there_are_profiles():
    assert any(p.endswith("_pmc.md") for p in PROFILES)
    assert any(p.endswith("_kernel_stats.md") for p in PROFILES)


@pytest.mark.parametrize("path", [p for p in PROFILES if p.endswith("_pmc.md")],
                         ids=os.path.basename)
def test_counter_summary_matches_the_built_kernel(isa, path):
    f = _fields(path)
    assert f["kernel"] in isa, f"{f['kernel']} is not a kernel of the built library"
    assert f["isa_sha256"] == isa[f["kernel"]], "counters taken on other machine code"
    assert int(f["traffic_bytes_per_pass"]) > 0


@pytest.mark.parametrize("path", PROFILES, ids=os.path.basename)
def test_summary_gives_its_command(path):
    text = open(path).read()
    assert "rocprofv3" in text and "```" in text, "no command"
    assert "_work" not in text, "a summary's command runs committed files only"
