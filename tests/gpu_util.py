"""Helpers shared by the GPU parity tests (comparison and sampling only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from workloads import bits, from_bits

RTOL = 1e-2
ATOL = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return bits(t.detach().to("cpu"))


def values(b: np.ndarray) -> np.ndarray:
    return from_bits(b).to(torch.float64).numpy()


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    """|gpu - ref| <= 1e-2 * |ref| + 1e-2, elementwise (bf16 bit arrays)."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g, r = values(got), values(ref)
    err = np.abs(g - r)
    bad = err > RTOL * np.abs(r) + ATOL
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: gpu={g[tuple(i)]!r} ref={r[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {detail}")
    nz = np.abs(r) > 0
    rel = float((err[nz] / np.abs(r[nz])).max()) if nz.any() else 0.0
    log(f"  {what}: max|err|={float(err.max()) if err.size else 0.0:.3g} max rel={rel:.3g} "
        f"exact={float((got == ref).mean()) if got.size else 1.0:.4f}")


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} differ; first {i}: "
                             f"gpu={got[i]:#06x} ref={ref[i]:#06x}")
