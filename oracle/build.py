"""Build the CPU oracle shared library (test infrastructure only).

The oracle is plain C compiled with gcc; it is built next to its source as
``oracle/liboracle.so``.  ``build(defines=...)`` also produces the
planted-mistake variants that the test suite uses to show that its pins catch
plausible mistakes; those go to a caller-chosen directory.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gemm_coll_oracle.c")
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

# Portable x86-64 code (no -march=native: the library may run on another host),
# no fast-math and no contraction, so the arithmetic is exactly what the source
# says.
CFLAGS = ["-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(out_path: str | None = None, defines: tuple[str, ...] = ()) -> str:
    """Compile the oracle; returns the path of the shared library."""
    out_path = out_path or DEFAULT_LIB
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = ["gcc", *CFLAGS, *[f"-D{d}" for d in defines], "-o", tmp, SOURCE, "-lm"]
    try:
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        os.replace(tmp, out_path)
    except subprocess.CalledProcessError as e:
        os.unlink(tmp)
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{e.stderr}") from e
    return out_path


if __name__ == "__main__":
    print(build())
