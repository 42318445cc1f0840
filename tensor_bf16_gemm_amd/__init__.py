"""tensor_bf16_gemm_amd -- fused tensor-parallel BF16 GEMM + reduction on MI355X.

Thin Python binding of ``libgemm_coll.so`` (C ABI: include/gemm_coll.h).  It
only marshals arguments: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the stream.

    out = gemm_ar(A, B, partials, R=8, rank=0)            # GEMM-AR
    out = gemm_rs(A, B, partials, ws, R=8, rank=5)        # GEMM-RS
    out = ag_gemm(A, B, shards, flags, status, R=8, rank=3, epoch=1)

Tensors are bf16, contiguous, on the current CUDA (HIP) device.  By default
each call uses a workspace that lets the kernel split leftover tiles along
K, allocated once per (device, stream) pair, so that calls in flight on
different streams never share one; pass workspace=False to compute every
tile whole, or a zero-filled uint8 tensor of workspace_bytes() of your own.  A failed
call raises RuntimeError with the library's message.  If the library is not
built, the first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gemm_ar", "gemm_ar_noalloc", "gemm_rs", "gemm_ar_two_shot", "ag_gemm", "ag_push_shards", "peer_sum",
           "should_run", "strerror", "plan",
           "lib", "GcPeers", "GcPlan",
           "workspace_bytes", "default_workspace",
           "LIB_PATH", "GC_OK", "GC_EINVAL", "GC_ENOTSUP", "GC_EIO", "GC_ENOSPC",
           "GC_TIMEOUT_BASE"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm_coll.so")

GC_OK = 0
GC_EINVAL = -22
GC_ENOTSUP = -95
GC_EIO = -5
GC_ENOSPC = -28
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
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
        ("tile_rows", ctypes.c_uint32),
        ("peer_out", ctypes.c_void_p),
        ("split_wait_spins", ctypes.c_uint32),
    ]


class GcPlan(ctypes.Structure):
    """Mirror of ``gc_plan`` in include/gemm_coll.h."""
    _fields_ = [
        ("tile_rows", ctypes.c_uint32),
        ("tiles", ctypes.c_int32),
        ("whole_tiles", ctypes.c_int32),
        ("split_tiles", ctypes.c_int32),
        ("chunks", ctypes.c_int32),
        ("chunk_steps", ctypes.c_int32),
        ("units", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("peer_nt", ctypes.c_int32),
    ]


MODES = {"ar": 0, "rs": 1, "ag": 2}

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
        for name in ("gemm_ar", "gemm_ar_noalloc", "gemm_rs", "gemm_ar_two_shot", "ag_gemm"):
            f = getattr(L, name)
            f.argtypes = sig
            f.restype = ctypes.c_int
        L.gemm_coll_should_run.argtypes = [i64]
        L.gemm_coll_should_run.restype = ctypes.c_int
        L.gemm_coll_strerror.argtypes = [ctypes.c_int]
        L.gemm_coll_strerror.restype = ctypes.c_char_p
        L.gemm_coll_workspace_bytes.argtypes = []
        L.gemm_coll_workspace_bytes.restype = ctypes.c_int64
        L.gemm_coll_peer_sum.argtypes = [vp, vp, i64, i64, ctypes.c_int, i64, vp, vp]
        L.gemm_coll_peer_sum.restype = ctypes.c_int
        L.ag_push_shards.argtypes = [vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.ag_push_shards.restype = ctypes.c_int
        L.gemm_coll_plan.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                     ctypes.POINTER(GcPlan)]
        L.gemm_coll_plan.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().gemm_coll_strerror(int(code)).decode()


def should_run(M: int) -> bool:
    """Dispatch gate: True when the fused path should serve M tokens (M >= 128)."""
    return bool(lib().gemm_coll_should_run(int(M)))


def plan(mode: str, M: int, N: int, K: int, R: int, rank: int = 0, *, cus: int = 256,
         workspace: bool = True, tile_rows: int = 0) -> dict:
    """The launch plan a call would make (``gemm_coll_plan``; no GPU needed).
    ``mode`` is "ar", "rs" (also the two-shot AR) or "ag" (M = shard rows)."""
    out = GcPlan()
    rc = lib().gemm_coll_plan(MODES[mode], int(M), int(N), int(K), int(R), int(rank), int(cus),
                              int(bool(workspace)), int(tile_rows), ctypes.byref(out))
    if rc != GC_OK:
        raise RuntimeError(f"gemm_coll_plan failed: {strerror(rc)} ({rc})")
    return {name: int(getattr(out, name)) for name, _ in GcPlan._fields_}


_workspaces: dict = {}


def workspace_bytes() -> int:
    """Bytes of workspace that lets calls on the current device split tiles along K."""
    n = lib().gemm_coll_workspace_bytes()
    if n < 0:
        raise RuntimeError(f"gemm_coll_workspace_bytes: {strerror(n)}")
    return n


def _workspace_key(device, stream) -> tuple[int, int]:
    """(device index, hipStream_t handle) that a default workspace serves."""
    import torch
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    with torch.cuda.device(idx):
        return idx, _stream(stream)


def default_workspace(device=None, stream=None):
    """The zero-filled workspace of (device, stream), allocated on first use
    and reused by every later call on that stream.  Calls on one stream run
    one after another, so they never use it at the same time; a call on
    another stream gets a workspace of its own.  The zero fill is complete
    before this returns (a device synchronization, once per workspace), so
    the first call may be on any stream."""
    import torch
    key = _workspace_key(device, stream)

    def make():
        with torch.cuda.device(key[0]):
            ws = torch.zeros(workspace_bytes(), dtype=torch.uint8, device=f"cuda:{key[0]}")
            torch.cuda.synchronize(key[0])
        return ws
    return _cached_workspace(key, make)


def _cached_workspace(key: tuple[int, int], make):
    """The workspace cached under key = (device, stream), made by make() on
    first use."""
    ws = _workspaces.get(key)
    if ws is None:
        ws = make()
        _workspaces[key] = ws
    return ws


def _ws_fields(workspace, device, stream):
    """(pointer, bytes) for gc_peers: workspace=None -> the default one of
    (device, stream), False -> none (every tile computed whole), else a uint8
    device tensor."""
    if workspace is False:
        return None, 0
    if workspace is None:
        workspace = default_workspace(device, stream)
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


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


def gemm_ar(A, B, partials, out=None, *, R: int, rank: int, stream=None, workspace=None,
            status=None, tile_rows: int = 0, split_wait_spins: int = 0):
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
    wp, wb = _ws_fields(workspace, A.device, stream)
    peers = GcPeers(partials=_ptr(partials), workspace=wp, workspace_bytes=wb,
                    status=_ptr(status), tile_rows=int(tile_rows),
                    split_wait_spins=int(split_wait_spins))
    _check(lib().gemm_ar(_ptr(A), _ptr(B), M, N, K, R, rank, ctypes.byref(peers), _ptr(out),
                         _stream(stream)), "gemm_ar")
    return out


def gemm_ar_noalloc(A, B, partials, out, *, R: int, rank: int, stream=None, status=None,
                    tile_rows: int = 0):
    """GEMM-AR that allocates nothing (gemm_ar_noalloc in the C ABI): as
    gemm_ar, with the K-split state in the library's static per-device
    scratch instead of a workspace.  `out` [M,N] is required (this wrapper
    allocates nothing either).  Calls on one device share that scratch: do
    not run two at the same time."""
    M, K = A.shape
    N = B.shape[1]
    _bf16("A", A)
    _bf16("B", B, (K, N))
    _bf16("partials", partials, (R - 1, M, N))
    _bf16("out", out, (M, N))
    peers = GcPeers(partials=_ptr(partials), status=_ptr(status), tile_rows=int(tile_rows))
    _check(lib().gemm_ar_noalloc(_ptr(A), _ptr(B), M, N, K, R, rank, ctypes.byref(peers),
                                 _ptr(out), _stream(stream)), "gemm_ar_noalloc")
    return out


def gemm_rs(A, B, partials, ws, out=None, *, R: int, rank: int, stream=None, workspace=None,
            status=None, tile_rows: int = 0, split_wait_spins: int = 0):
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
    wp, wb = _ws_fields(workspace, A.device, stream)
    peers = GcPeers(partials=_ptr(partials), ws=_ptr(ws), workspace=wp, workspace_bytes=wb,
                    status=_ptr(status), tile_rows=int(tile_rows),
                    split_wait_spins=int(split_wait_spins))
    _check(lib().gemm_rs(_ptr(A), _ptr(B), M, N, K, R, rank, ctypes.byref(peers), _ptr(out),
                         _stream(stream)), "gemm_rs")
    return out


def gemm_ar_two_shot(A, B, partials, ws, peer_out, out=None, *, R: int, rank: int, stream=None,
                     workspace=None, status=None, tile_rows: int = 0, split_wait_spins: int = 0):
    """GEMM-AR, two-shot: this rank's rows [r*P, min((r+1)*P, M)) of
    bf16(A.B + sum of partials) go to out [M,N] and to every slot of
    peer_out [R-1,M,N]; ws [M,N] receives bf16(A.B) on the other rows.  Rows
    of out and peer_out outside the slice are left untouched."""
    import torch
    M, K = A.shape
    N = B.shape[1]
    _bf16("A", A)
    _bf16("B", B, (K, N))
    _bf16("partials", partials, (R - 1, M, N))
    _bf16("ws", ws, (M, N))
    _bf16("peer_out", peer_out, (R - 1, M, N))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _bf16("out", out, (M, N))
    wp, wb = _ws_fields(workspace, A.device, stream)
    peers = GcPeers(partials=_ptr(partials), ws=_ptr(ws), workspace=wp, workspace_bytes=wb,
                    status=_ptr(status), tile_rows=int(tile_rows), peer_out=_ptr(peer_out),
                    split_wait_spins=int(split_wait_spins))
    _check(lib().gemm_ar_two_shot(_ptr(A), _ptr(B), M, N, K, R, rank, ctypes.byref(peers),
                                  _ptr(out), _stream(stream)), "gemm_ar_two_shot")
    return out


def ag_gemm(A, B, shards, flags, status, out=None, *, R: int, rank: int, epoch: int,
            max_spins: int = 0, stream=None, workspace=None, tile_rows: int = 0,
            split_wait_spins: int = 0):
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
    wp, wb = _ws_fields(workspace, A.device, stream)
    peers = GcPeers(shards=_ptr(shards), flags=_ptr(flags), epoch=int(epoch) & 0xFFFFFFFF,
                    status=_ptr(status), max_spins=int(max_spins), workspace=wp,
                    workspace_bytes=wb, tile_rows=int(tile_rows),
                    split_wait_spins=int(split_wait_spins))
    _check(lib().ag_gemm(_ptr(A), _ptr(B), Ms, N, K, R, rank, ctypes.byref(peers), _ptr(out),
                         _stream(stream)), "ag_gemm")
    return out


def peer_sum(local, partials, out=None, *, stream=None):
    """Reduction step of the unfused baseline: out [rows,N] = bf16(local +
    sum over p of partials[p]), fp32 sum in the order local, peer 0, 1, ...
    local: [rows,N] bf16, contiguous; partials: [npeers,rows,N] bf16 with
    contiguous rows (stride(0) may be larger, e.g. a row slice of [R-1,M,N]
    partials); out may be local."""
    import torch
    rows, N = local.shape
    _bf16("local", local, (rows, N))
    if not partials.is_cuda:
        raise ValueError("partials must be a device tensor")
    if partials.dtype != torch.bfloat16 or partials.dim() != 3 or tuple(partials.shape[1:]) != (rows, N):
        raise ValueError(f"partials: expected bf16 [npeers, {rows}, {N}], got "
                         f"{partials.dtype} {tuple(partials.shape)}")
    if partials.shape[0] > 0 and rows * N > 0 and (partials.stride(2) != 1 or partials.stride(1) != N):
        raise ValueError("partials: rows must be contiguous")
    if out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=local.device)
    _bf16("out", out, (rows, N))
    npeers = partials.shape[0]
    stride = partials.stride(0) if npeers > 0 else 0
    _check(lib().gemm_coll_peer_sum(_ptr(local), _ptr(partials) if npeers else None, rows, N, npeers,
                                    stride, _ptr(out), _stream(stream)), "gemm_coll_peer_sum")
    return out


def ag_push_shards(src, dst, flags, epoch_word, *, R: int, rank: int, stream=None):
    """The other ranks' side of AG-GEMM, emulated: on `stream`, in ring order,
    copy shard q of src [R,Ms,K] into dst [R,Ms,K] (ag_gemm's shards) and then
    raise flags[q] to epoch_word[0], all through the DMA engines.  flags:
    int32 [R] device tensor; epoch_word: int32 [1] device tensor."""
    import torch
    Rr, Ms, K = src.shape
    if Rr != R:
        raise ValueError(f"src has {Rr} shards, R={R}")
    _bf16("src", src, (R, Ms, K))
    _bf16("dst", dst, (R, Ms, K))
    for name, t, n in (("flags", flags, R), ("epoch_word", epoch_word, 1)):
        if t.dtype not in (torch.int32, torch.uint32) or tuple(t.shape) != (n,) or not t.is_cuda:
            raise ValueError(f"{name}: expected a 32-bit device tensor of shape ({n},)")
    _check(lib().ag_push_shards(_ptr(src), _ptr(dst), Ms, K, R, rank, _ptr(flags), _ptr(epoch_word),
                                _stream(stream)), "ag_push_shards")

