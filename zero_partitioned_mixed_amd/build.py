"""Builds libzero_shard.so (gfx950) next to this file with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "zero_shard.hip")
LIB = os.path.join(HERE, "libzero_shard.so")
INCLUDE = os.path.join(ROOT, "include")

# -ffp-contract=off: every fp32 operation of the step is rounded on its own.
# -packed-fp32-ops: no packed fp32 instructions in any generated code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-I", INCLUDE]


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", *HIPCC_FLAGS, "-o", tmp, SRC], check=True,
                   stderr=subprocess.PIPE)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
