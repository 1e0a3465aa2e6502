"""Compile the fp64 CPU oracle (plain C) into a shared library.

Test infrastructure only.  ``build()`` writes ``oracle/_lib/liblora_oracle.so``;
``build(mutant=k)`` writes a copy with planted mistake ``k`` (see
``ORC_MUTANT`` in lora_oracle.c) to a caller-chosen directory, for the tests
that check the pins would catch such a mistake.
"""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "lora_oracle.c"
LIB_DIR = HERE / "_lib"
LIB = LIB_DIR / "liblora_oracle.so"

# No -ffast-math, no FMA contraction: every product and sum is the plain one.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(out: Path | None = None, mutant: int = 0) -> Path:
    out = Path(out) if out is not None else LIB
    out.parent.mkdir(parents=True, exist_ok=True)
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", *CFLAGS, f"-DORC_MUTANT={int(mutant)}", str(SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
