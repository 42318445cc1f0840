"""ctypes front end of the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  It takes and returns numpy ``uint16`` arrays holding raw bf16
bits, and never touches the GPU library.

Every function follows the plain definition written out in
``gemm_coll_oracle.c``:

* GEMM-AR  out = bf16(A.B + sum of the R-1 peer partials)      (all rows)
* GEMM-RS  rank r keeps rows [r*P, (r+1)*P) of that sum, P = ceil(M/R),
  with the rows past M zero; its non-owned rows publish bf16(A.B) into ws
* AG-GEMM  out = bf16(concat(shards).B)

(sources: the test reference in "[Kimi-K3] Extend GEMM-RS to GEMM-AR",
section 关键源码片段; "[Kimi-K3] AG-GEMM for Sequence Parallelism", Purpose.)

The sum runs k ascending, then peers ascending, in a binary32 accumulator
(``acc="fp32"``, the default: fp32 accumulation over bf16 inputs, the
contract of the fused kernels) or a binary64 one (``acc="fp64"``, nearly
exact, which the pins use to check the fp32 one from outside); one
round-to-nearest-even to bf16 at the end.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64 = ctypes.c_int64
_i64p = ctypes.POINTER(ctypes.c_int64)


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.dtype == np.uint16 and a.flags["C_CONTIGUOUS"], (a.dtype, a.flags)
    return a.ctypes.data_as(_u16p)


def _check(err: int, what: str):
    if err != 0:
        raise RuntimeError(f"oracle {what} failed with code {err}")


ACC_CODES = {"fp32": 32, "fp64": 64}


class Oracle:
    """One loaded build of the oracle library, with one accumulation
    precision (``acc``: "fp32" or "fp64")."""

    def __init__(self, lib_path: str, acc: str = "fp32"):
        if acc not in ACC_CODES:
            raise ValueError(f"acc must be one of {sorted(ACC_CODES)}, got {acc!r}")
        self.path = lib_path
        self.acc = acc
        self._acc = ACC_CODES[acc]
        lib = ctypes.CDLL(lib_path)
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        ci = ctypes.c_int
        lib.oracle_ar_rows.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, ci, ci, _u16p]
        lib.oracle_ar_rows.restype = ctypes.c_int
        lib.oracle_rs_slice.argtypes = [_i64, ctypes.c_int, ctypes.c_int, _i64p, _i64p, _i64p]
        lib.oracle_rs_slice.restype = ctypes.c_int
        lib.oracle_gemm_ar.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, ci, ci, _u16p]
        lib.oracle_gemm_ar.restype = ctypes.c_int
        lib.oracle_gemm_rs.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, ci, ci, ci,
                                       _u16p, _u16p]
        lib.oracle_gemm_rs.restype = ctypes.c_int
        lib.oracle_ag_source.argtypes = [_i64, ctypes.c_int, _i64, ctypes.POINTER(ctypes.c_int), _i64p]
        lib.oracle_ag_source.restype = ctypes.c_int
        lib.oracle_ag_gemm.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, _i64, ci, ci, ci,
                                       _u16p]
        lib.oracle_ag_gemm.restype = ctypes.c_int
        self.lib = lib

    # -- scalars ---------------------------------------------------------
    def round_bf16(self, x: float) -> int:
        """Nearest bf16 (ties to even) of a double, as raw bits."""
        return int(self.lib.oracle_round_bf16(float(x)))

    def bf16_to_float(self, h: int) -> float:
        return float(self.lib.oracle_bf16_to_double(int(h)))

    # -- matrices --------------------------------------------------------
    def ar_rows(self, A_rows: np.ndarray, B: np.ndarray, peer_rows: np.ndarray | None) -> np.ndarray:
        """out[t] = bf16(A_rows[t].B + sum_p peer_rows[p, t]); peer_rows [npeers, nrows, N]."""
        nrows, K = A_rows.shape
        K2, N = B.shape
        assert K == K2
        npeers = 0
        if peer_rows is not None:
            npeers, pr, pn = peer_rows.shape
            assert (pr, pn) == (nrows, N)
            if npeers == 0:
                peer_rows = None
        out = np.empty((nrows, N), dtype=np.uint16)
        _check(self.lib.oracle_ar_rows(_ptr(A_rows), _ptr(B), _ptr(peer_rows), nrows, N, K,
                                       npeers, self._acc, _ptr(out)), "ar_rows")
        return out

    def gemm_ar(self, A: np.ndarray, B: np.ndarray, peers: np.ndarray, R: int) -> np.ndarray:
        """GEMM-AR: peers [R-1, M, N]; returns out [M, N]."""
        M, K = A.shape
        N = B.shape[1]
        if R > 1:
            assert peers.shape == (R - 1, M, N)
        out = np.empty((M, N), dtype=np.uint16)
        _check(self.lib.oracle_gemm_ar(_ptr(A), _ptr(B), _ptr(peers if R > 1 else None), M, N, K,
                                       R, self._acc, _ptr(out)), "gemm_ar")
        return out

    def rs_slice(self, M: int, R: int, r: int) -> tuple[int, int, int]:
        """(P, lo, hi): slice height and the valid global rows rank r owns."""
        P, lo, hi = _i64(), _i64(), _i64()
        _check(self.lib.oracle_rs_slice(M, R, r, ctypes.byref(P), ctypes.byref(lo), ctypes.byref(hi)),
               "rs_slice")
        return P.value, lo.value, hi.value

    def gemm_rs(self, A: np.ndarray, B: np.ndarray, peers: np.ndarray, R: int, r: int,
                ws: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray | None]:
        """GEMM-RS: returns (out [P, N], ws).  ws (if given, [M, N]) is updated in place
        on the non-owned rows and left untouched on the owned rows."""
        M, K = A.shape
        N = B.shape[1]
        P, _, _ = self.rs_slice(M, R, r)
        out = np.empty((P, N), dtype=np.uint16)
        if ws is not None:
            assert ws.shape == (M, N)
        _check(self.lib.oracle_gemm_rs(_ptr(A), _ptr(B), _ptr(peers if R > 1 else None), M, N, K,
                                       R, r, self._acc, _ptr(out), _ptr(ws)), "gemm_rs")
        return out, ws

    def ag_source(self, Ms: int, R: int, g: int) -> tuple[int, int]:
        """(shard q, row t) that output row g of AG-GEMM comes from."""
        q, t = ctypes.c_int(), _i64()
        _check(self.lib.oracle_ag_source(Ms, R, g, ctypes.byref(q), ctypes.byref(t)), "ag_source")
        return q.value, t.value

    def ag_gemm(self, A_local: np.ndarray, B: np.ndarray, shards: np.ndarray, R: int, r: int) -> np.ndarray:
        """AG-GEMM: shards [R, Ms, K] (slot r unused, A_local is read); out [R*Ms, N]."""
        Ms, K = A_local.shape
        N = B.shape[1]
        assert shards.shape == (R, Ms, K)
        out = np.empty((R * Ms, N), dtype=np.uint16)
        _check(self.lib.oracle_ag_gemm(_ptr(A_local), _ptr(B), _ptr(shards), Ms, N, K, R, r,
                                       self._acc, _ptr(out)), "ag_gemm")
        return out


_DEFAULT: dict = {}


def load(lib_path: str | None = None, acc: str = "fp32") -> Oracle:
    """Load the oracle library (building it first only if nothing is built),
    accumulating in `acc` ("fp32", the default, or "fp64")."""
    if lib_path is not None:
        return Oracle(lib_path, acc)
    if acc not in _DEFAULT:
        if not os.path.exists(_build.DEFAULT_LIB):
            _build.build()
        _DEFAULT[acc] = Oracle(_build.DEFAULT_LIB, acc)
    return _DEFAULT[acc]
