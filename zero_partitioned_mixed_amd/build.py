"""Builds libzero_shard.so (gfx950) next to this file with hipcc.

Besides the library it writes libzero_shard.isa.json: for every kernel, a
SHA-256 of its gfx950 machine code as the compiler prints it (instructions
only; comments, directives and label numbers dropped), keyed by the kernel's
readable name (e.g. ``fused_kernel<1, 4, 8, Src16<1, StridedRows> >``, the
form profilers print).  A measurement of a kernel stays attributable to the
current build exactly as long as that kernel's digest is unchanged.
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "zero_shard.hip")
LIB = os.path.join(HERE, "libzero_shard.so")
ISA_JSON = os.path.join(HERE, "libzero_shard.isa.json")
INCLUDE = os.path.join(ROOT, "include")

# -ffp-contract=off: every fp32 operation of the step is rounded on its own.
# -packed-fp32-ops: no packed fp32 instructions in any generated code.
CODEGEN_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HIPCC_FLAGS = CODEGEN_FLAGS + ["-fPIC", "-shared", "-Wall", "-Wextra", "-I", INCLUDE]


def kernel_name(demangled: str) -> str:
    """Readable kernel name: namespaces, return type and parameters dropped."""
    s = demangled.replace("(anonymous namespace)::", "")
    if s.startswith("void "):
        s = s[5:]
    return s.split("(")[0].strip()


def isa_digests(asm: str) -> dict:
    """{mangled symbol: sha256 of its normalised instruction stream}."""
    out = {}
    functions = set(re.findall(r"^\s*\.type\s+(_Z\S+),@function", asm, re.M))
    for m in re.finditer(r"^(_Z\S+):", asm, re.M):
        if m.group(1) not in functions:  # device data (the no-alloc scratch array)
            continue
        end = asm.find(".Lfunc_end", m.end())
        lines = []
        for line in asm[m.end():end].splitlines():
            t = line.split(";")[0].strip()
            if t and not t.startswith("."):
                lines.append(t)
        body = re.sub(r"\.LBB\d+_\d+", "L", "\n".join(lines))
        out[m.group(1)] = hashlib.sha256(body.encode()).hexdigest()
    return out


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    return r


def build() -> str:
    tmp = LIB + ".tmp"
    _run(["hipcc", *HIPCC_FLAGS, "-o", tmp, SRC])
    asm = ISA_JSON + ".s.tmp"
    try:
        _run(["hipcc", *CODEGEN_FLAGS, "-I", INCLUDE, "--cuda-device-only", "-S", "-o", asm, SRC])
        digests = isa_digests(open(asm).read())
    finally:
        if os.path.exists(asm):
            os.remove(asm)
    names = subprocess.run(["c++filt"], input="\n".join(digests), stdout=subprocess.PIPE,
                           text=True, check=True).stdout.splitlines()
    table = {kernel_name(d): h for d, h in zip(names, digests.values())}
    with open(ISA_JSON + ".tmp", "w") as f:
        json.dump(table, f, indent=0, sort_keys=True)
    os.replace(tmp, LIB)
    os.replace(ISA_JSON + ".tmp", ISA_JSON)
    return LIB


if __name__ == "__main__":
    print(build())
