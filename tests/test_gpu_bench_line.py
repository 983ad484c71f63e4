"""bench.py keeps its contract: one JSON line with the fields the benchmark
report needs, on a small workload (the GPT-2-sized shard, a few steps, a
small CPU sample), run as a child process exactly as a user would."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_complete_json_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "gpt2_psi124439808_n8",
           "--steps", "5", "--warmup", "1", "--cpu-sample", str(1 << 20), "--no-copy"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "pct_hbm_peak", "elements_per_s"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["value"] > 0
    assert d["config"]["workload"] == "gpt2_psi124439808_n8"
    ro = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in ro, key
    assert ro["bound"] == "hbm" and ro["peak"] == 8000.0 and 0 < ro["frac"] < 1
    assert abs(ro["frac"] - ro["achieved"] / ro["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0 and cb["sample"]


def test_bench_refuses_more_than_one_gpu():
    # checked before anything touches the GPU, so this runs without one
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "ONE GPU" in r.stderr


@pytest.mark.gpu
def test_bench_skip_step_timing_restores_its_input():
    """bench.timed_skip_steps on a small fused workload with an injected +inf:
    every timed step is skipped (the decision halves the scale each time),
    the parts are timed, and the contribution element is put back after."""
    import torch
    import bench
    import synth
    import zero_partitioned_mixed_amd as Z
    from synth.workloads import F16, Workload
    synth.gpu()
    w = Workload(name="skipbench", psi=8 * 300_001, nranks=8, ranks=(7,), dtype=F16, steps=5,
                 contrib_scale=2.0 ** 10, scaler=2, loss_scale=2.0 ** 10,
                 inject_inf=((2, 3, 150_000),))
    b = bench.setup(w, torch, synth, Z)
    before = b["contrib"].clone()
    bench.timed_steps(b, 3, 1, torch, Z)
    scale0 = b["step"].ctrl_dict()["loss_scale"]
    out = bench.timed_skip_steps(b, w, torch, reps=3)
    assert torch.equal(b["contrib"].view(torch.int16), before.view(torch.int16))
    assert out["steps"] == 3 and out["ms"] > 0 and out["restore_ms"] > 0
    assert out["loss_scales_after"] == [scale0 / 2, scale0 / 4, scale0 / 8]
    assert out["restore_bytes"] == 6 * b["valid"]


@pytest.mark.gpu
def test_stream_reference_lines():
    """The plain streams the bench reports beside the kernels: each kind runs
    over the buffers and gives a positive rate; the copy leaves the copied
    values and the mixed streams their sums."""
    import torch
    import bench
    import synth
    synth.gpu()
    rates = bench.stream_rates(torch, synth, nbytes=64 << 20, reps=2)
    assert set(rates) == {"read", "write", "copy", "mix_2r1w", "mix_4r1w"}
    assert min(rates.values()) > 0
    n = (8 << 20) // 4
    a = torch.arange(n, dtype=torch.float32, device="cuda")
    b = torch.full((n,), 0.5, device="cuda")
    d = torch.zeros(n, device="cuda")
    synth.gpu_stream("copy", a, None, d, 8 << 20, 65536, 48 * 1024)
    assert torch.equal(d, a)
    synth.gpu_stream("mix_2r1w", a, b, d, 8 << 20, 100, 0)  # several launches of 100 workgroups
    assert torch.equal(d, a + b)
    d.zero_()
    m = n // 2  # four reads per write: each half of a and of b, into the first half of d
    synth.gpu_stream("mix_4r1w", a, b, d, 4 << 20, 100, 0)
    assert torch.equal(d[:m], (a[:m] + a[m:]) + (b[:m] + b[m:]))
    assert not d[m:].any()
