"""Build the HIP library ``libgemm_coll.so`` for gfx950, in-tree.

    python -m tensor_bf16_gemm_amd.build

Compiles csrc/gemm_coll.hip (host C ABI + device kernels) with hipcc into
``tensor_bf16_gemm_amd/libgemm_coll.so``.  Packed-fp32 VALU instructions are
disabled for device code (-packed-fp32-ops); hipcc's host pass warns that it
does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgemm_coll.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def build(out_path: str = LIB, extra: tuple[str, ...] = ()) -> str:
    """Compile the library (always); returns its path."""
    src = os.path.join(CSRC, "gemm_coll.hip")
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = [hipcc(), *compile_flags(), "-shared", *extra, "-o", tmp, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"HIP build failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build())
