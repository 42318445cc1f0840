"""tensor_bf16_gemm_amd -- fused tensor-parallel BF16 GEMM + reduction on MI355X.

Thin Python binding of ``libgemm_coll.so`` (C ABI: include/gemm_coll.h).  It
only marshals arguments: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the stream.

    out = gemm_ar(A, B, partials, R=8, rank=0)            # GEMM-AR
    out = gemm_rs(A, B, partials, ws, R=8, rank=5)        # GEMM-RS
    out = ag_gemm(A, B, shards, flags, status, R=8, rank=3, epoch=1)

Tensors are bf16, contiguous, on the current CUDA (HIP) device.  A failed
call raises RuntimeError with the library's message.  If the library is not
built, the first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gemm_ar", "gemm_rs", "ag_gemm", "should_run", "strerror", "lib", "GcPeers",
           "LIB_PATH", "GC_OK", "GC_EINVAL", "GC_ENOTSUP", "GC_EIO", "GC_TIMEOUT_BASE"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm_coll.so")

GC_OK = 0
GC_EINVAL = -22
GC_ENOTSUP = -95
GC_EIO = -5
GC_TIMEOUT_BASE = 1000


class GcPeers(ctypes.Structure):
    """Mirror of ``gc_peers`` in include/gemm_coll.h."""
    _fields_ = [
        ("partials", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("shards", ctypes.c_void_p),
        ("flags", ctypes.c_void_p),
        ("epoch", ctypes.c_uint32),
        ("status", ctypes.c_void_p),
        ("max_spins", ctypes.c_uint32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tensor_bf16_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        sig = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(GcPeers), vp, vp]
        for name in ("gemm_ar", "gemm_rs", "ag_gemm"):
            f = getattr(L, name)
            f.argtypes = sig
            f.restype = ctypes.c_int
        L.gemm_coll_should_run.argtypes = [i64]
        L.gemm_coll_should_run.restype = ctypes.c_int
        L.gemm_coll_strerror.argtypes = [ctypes.c_int]
        L.gemm_coll_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().gemm_coll_strerror(int(code)).decode()


def should_run(M: int) -> bool:
    """Dispatch gate: True when the fused path should serve M tokens (M >= 128)."""
    return bool(lib().gemm_coll_should_run(int(M)))


def _check(code: int, what: str):
    if code != GC_OK:
        raise RuntimeError(f"{what}: {strerror(code)} (code {code})")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _bf16(name, t, shape=None):
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def gemm_ar(A, B, partials, out=None, *, R: int, rank: int, stream=None):
    """GEMM-AR: out [M,N] = bf16(A.B + sum of partials [R-1,M,N])."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    _bf16("A", A)
    _bf16("B", B, (K, N))
    _bf16("partials", partials, (R - 1, M, N))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _bf16("out", out, (M, N))
    peers = GcPeers(partials=_ptr(partials))
    _check(lib().gemm_ar(_ptr(A), _ptr(B), M, N, K, R, rank, ctypes.byref(peers), _ptr(out),
                         _stream(stream)), "gemm_ar")
    return out


def gemm_rs(A, B, partials, ws, out=None, *, R: int, rank: int, stream=None):
    """GEMM-RS: out [ceil(M/R), N] = this rank's rows of bf16(A.B + sum of partials);
    ws [M,N] receives bf16(A.B) on the rows this rank does not own."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    P = (M + R - 1) // R
    _bf16("A", A)
    _bf16("B", B, (K, N))
    _bf16("partials", partials, (R - 1, M, N))
    _bf16("ws", ws, (M, N))
    if out is None:
        out = torch.empty((P, N), dtype=torch.bfloat16, device=A.device)
    _bf16("out", out, (P, N))
    peers = GcPeers(partials=_ptr(partials), ws=_ptr(ws))
    _check(lib().gemm_rs(_ptr(A), _ptr(B), M, N, K, R, rank, ctypes.byref(peers), _ptr(out),
                         _stream(stream)), "gemm_rs")
    return out


def ag_gemm(A, B, shards, flags, status, out=None, *, R: int, rank: int, epoch: int,
            max_spins: int = 0, stream=None):
    """AG-GEMM: out [R*Ms, N] = bf16(concat(shards).B), A = this rank's shard [Ms,K].
    flags: int32 tensor [R] in device memory or pinned host memory (the kernel
    polls it with system-scope loads); status: int32 device tensor [1]."""
    import torch
    Ms, K = A.shape
    N = B.shape[1]
    _bf16("A", A)
    _bf16("B", B, (K, N))
    _bf16("shards", shards, (R, Ms, K))
    if (flags.numel() != R or flags.element_size() != 4 or not flags.is_contiguous()
            or not (flags.is_cuda or flags.is_pinned())):
        raise ValueError("flags must be R 4-byte elements in device or pinned host memory")
    if status.numel() < 1 or status.element_size() != 4 or not status.is_cuda:
        raise ValueError("status must be a 4-byte device tensor")
    if out is None:
        out = torch.empty((R * Ms, N), dtype=torch.bfloat16, device=A.device)
    _bf16("out", out, (R * Ms, N))
    peers = GcPeers(shards=_ptr(shards), flags=_ptr(flags), epoch=int(epoch) & 0xFFFFFFFF,
                    status=_ptr(status), max_spins=int(max_spins))
    _check(lib().ag_gemm(_ptr(A), _ptr(B), Ms, N, K, R, rank, ctypes.byref(peers), _ptr(out),
                         _stream(stream)), "ag_gemm")
    return out
