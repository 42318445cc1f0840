"""Seeded synthetic workloads for the fused TP GEMM + reduction.

This module holds no arithmetic of the method: it only names the workloads
and draws their inputs.  Both sides of every parity check (the HIP library and
the CPU oracle) receive the same bf16 bits from here.

The shapes are those of the projections the pages benchmark: the KDA and MLA
output projections of "[Kimi-K3] AG-GEMM for Sequence Parallelism"
(Microbenchmark results table: N = 6288 / 3648, K = 7168, TP8) and the
"[Kimi-K3] Extend GEMM-RS to GEMM-AR" dispatch (M >= 128).  The pages' real
activations and weights are not available; Gaussian stand-ins of the same
shapes take their place.

Draw order (one ``torch.Generator`` seeded per workload): A, B, then the R-1
peer partials in ascending slot order.  For AG: the R shards in rank order,
then B.  Values are drawn in float32 from N(0, 1), scaled, then rounded to
bf16 (round-to-nearest-even, torch's conversion).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "ar" | "rs" | "ag" | "ar2" (GEMM-AR by the two-shot flow)
    M: int               # rows (AG: rows per shard, Ms)
    N: int
    K: int
    R: int               # emulated tensor-parallel ranks
    rank: int            # the rank this GPU plays
    a_scale: float = 1.0
    b_scale: float = 1.0
    peer_scale: float = 1.0
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        rows = self.M * self.R if self.mode == "ag" else self.M
        return 2 * rows * self.N * self.K

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


def _isqrt(k: int) -> float:
    return 1.0 / math.sqrt(k)


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_ar", "ar", 128, 256, 512, 2, 0, _isqrt(512), _isqrt(512), 1.0, 0,
                 "GEMM-AR tiny, 1 peer"),
        Workload("mla_ar", "ar", 256, 3648, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "MLA projection, one rank's share, GEMM-AR"),
        Workload("mla_rs", "rs", 256, 3648, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "MLA projection, one rank's share, GEMM-RS"),
        Workload("kda512_ar", "ar", 512, 6288, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "KDA projection M=512, GEMM-AR"),
        Workload("kda1024_ar", "ar", 1024, 6288, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "KDA projection M=1024, GEMM-AR"),
        Workload("kda4096_ar", "ar", 4096, 6288, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "KDA projection M=4096, GEMM-AR (headline)"),
        Workload("kda4096_ar2", "ar2", 4096, 6288, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "KDA projection M=4096, GEMM-AR by the two-shot flow (rank 0's share)"),
        Workload("kda64_ar", "ar", 64, 6288, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "KDA decode size M=64, below the dispatch gate: GEMM-AR, tiles split along K"),
        Workload("kda16_ar", "ar", 16, 6288, 7168, 8, 0, 1.0, _isqrt(7168), 1.0, 0,
                 "KDA decode size M=16, below the dispatch gate: GEMM-AR, tiles split along K"),
        Workload("kda4096_k0", "ar", 4096, 6288, 0, 8, 0, 1.0, 1.0, 1.0, 0,
                 "KDA M=4096 with K=0: the fused kernel reduces to the peer sum (epilogue bandwidth)"),
        Workload("ag_kda", "ag", 4096, 6288, 7168, 8, 3, 1.0, _isqrt(7168), 1.0, 0,
                 "AG-GEMM KDA, 8 shards of 4096 rows, ring from rank 3"),
        Workload("rs_odd", "rs", 32768 + 37, 7168, 896, 8, 5, _isqrt(896), _isqrt(896), 1.0, 0,
                 "GEMM-RS odd M, rank 5"),
    ]
}

HEADLINE = "kda4096_ar"


def _draw(g: torch.Generator, shape, scale: float, device) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu") -> dict[str, torch.Tensor]:
    """Draw the workload's inputs (bf16 tensors on ``device``).

    AR / RS: {"A": [M,K], "B": [K,N], "peers": [R-1,M,N]}
    AG:      {"A": [Ms,K] (= shards[rank]), "B": [K,N], "shards": [R,Ms,K]}
    """
    g = torch.Generator(device=device)
    g.manual_seed(w.seed)
    if w.mode == "ag":
        shards = _draw(g, (w.R, w.M, w.K), w.a_scale, device)
        B = _draw(g, (w.K, w.N), w.b_scale, device)
        return {"A": shards[w.rank].clone(), "B": B, "shards": shards}
    A = _draw(g, (w.M, w.K), w.a_scale, device)
    B = _draw(g, (w.K, w.N), w.b_scale, device)
    peers = _draw(g, (max(w.R - 1, 0), w.M, w.N), w.peer_scale, device)
    return {"A": A, "B": B, "peers": peers}


def integer_inputs(mode: str, M: int, N: int, K: int, R: int, rank: int = 0, seed: int = 0,
                   ab_range: int = 2, peer_range: int = 64, device="cpu") -> dict[str, torch.Tensor]:
    """Small-integer inputs (exact in bf16).  With |A|,|B| <= ab_range and
    |peer| <= peer_range every partial sum is an integer far below 2^24, so
    any summation order gives the same value before the final rounding."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def ints(shape, lim):
        return torch.randint(-lim, lim + 1, shape, generator=g, device=device,
                             dtype=torch.int32).to(torch.bfloat16)

    if mode == "ag":
        shards = ints((R, M, K), ab_range)
        B = ints((K, N), ab_range)
        return {"A": shards[rank].clone(), "B": B, "shards": shards}
    A = ints((M, K), ab_range)
    B = ints((K, N), ab_range)
    peers = ints((max(R - 1, 0), M, N), peer_range)
    return {"A": A, "B": B, "peers": peers}


def bits(t: torch.Tensor):
    """Raw bf16 bits of a CPU tensor as a numpy uint16 array (no copy of values)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def from_bits(a) -> torch.Tensor:
    """bf16 tensor from a numpy uint16 array of raw bits."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
