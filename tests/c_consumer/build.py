"""Compiles shard_step_demo.c (a plain C consumer of the shard-step C ABI)
against the built libzero_shard.so and libsynth_cpu.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "shard_step_demo.c")
BIN = os.path.join(HERE, "shard_step_demo")
ROCM = "/opt/rocm"


def build() -> str:
    tmp = BIN + ".tmp"
    subprocess.run(
        ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
         "-o", tmp, SRC,
         "-L", os.path.join(ROOT, "zero_partitioned_mixed_amd"), "-lzero_shard",
         "-L", os.path.join(ROOT, "synth"), "-lsynth_cpu",
         "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
         "-Wl,-rpath,$ORIGIN/../../zero_partitioned_mixed_amd:$ORIGIN/../../synth:"
         + os.path.join(ROCM, "lib")],
        check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
