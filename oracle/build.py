"""Build the CPU oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure: the product library never links or loads this.
Usage: ``python oracle/build.py`` or ``build(src=..., out=..., defines=...)``.
"""

from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"


def build(src: Path = SRC, out: Path = LIB, extra_flags=()) -> Path:
    out = Path(out)
    tmp = out.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-I", str(HERE), str(src), "-o", str(tmp), "-lm", *extra_flags]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
    sys.exit(0)
