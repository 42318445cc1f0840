"""224-row output tiles (tile_rows=224; the host picks them by itself where
they fill the last round of tiles better): on integer inputs, where every
partial sum is exact in fp32, the results equal the oracle's bit for bit in
all three modes -- ragged M, N and K, a last row tile that is mostly empty,
K shorter than the peer items (their drain after the K loop), and every RS
rank.  Also: the automatic choice at M=4096 against forced 256-row tiles on
float inputs, and the argument check."""

import numpy as np
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, host_bits, log
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FC1


@pytest.fixture(scope="module")
def orc():
    return load_oracle()


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def filled(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


SHAPES = [
    (300, 520, 512, 4),      # 2 row tiles, the second 76 rows; 16 K-steps, 3 peers
    (4133, 1040, 256, 8),    # 19 row tiles (the last 101 rows) x 5: 95 tiles
    (224, 264, 96, 2),       # exactly one row tile; ragged N
    (1000, 776, 72, 8),      # 3 K-steps: 56 peer items, 53 of them after the K loop
]


@pytest.mark.parametrize("M,N,K,R", SHAPES)
def test_ar_224(orc, M, N, K, R):
    log(f"224-row AR M={M} N={N} K={K} R={R}")
    xc = wl.integer_inputs("ar", M, N, K, R, seed=7 * M + N + K)
    x = to_dev(xc)
    out = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=1,
                     workspace=False, tile_rows=224)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), orc.gemm_ar(host_bits(xc["A"]), host_bits(xc["B"]),
                                                  host_bits(xc["peers"]), R), "AR 224")


@pytest.mark.parametrize("M,N,K,R", [SHAPES[0], SHAPES[1], SHAPES[3]])
def test_rs_224_all_ranks(orc, M, N, K, R):
    log(f"224-row RS M={M} N={N} K={K} R={R}")
    xc = wl.integer_inputs("rs", M, N, K, R, seed=3 * M + K)
    x = to_dev(xc)
    A, B, peers = (host_bits(xc[k]) for k in ("A", "B", "peers"))
    for rank in range(R):
        ws = filled((M, N))
        out = gc.gemm_rs(x["A"], x["B"], x["peers"], ws, R=R, rank=rank, workspace=False,
                         tile_rows=224)
        torch.cuda.synchronize()
        ws_ref = np.full((M, N), SENTINEL, np.uint16)
        ref, ws_ref = orc.gemm_rs(A, B, peers, R, rank, ws_ref)
        assert_bits_equal(host_bits(out), ref, f"RS 224 rank {rank}")
        assert_bits_equal(host_bits(ws), ws_ref, f"RS 224 ws rank {rank}")


@pytest.mark.parametrize("Ms,N,K,R", [(300, 520, 256, 4), (600, 1040, 72, 8)])
def test_ag_224(orc, Ms, N, K, R):
    log(f"224-row AG Ms={Ms} N={N} K={K} R={R}")
    rank = 2
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=Ms + 5 * K)
    x = to_dev(xc)
    flags = torch.ones(R, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, R=R, rank=rank, epoch=1,
                     workspace=False, tile_rows=224)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    sh = host_bits(xc["shards"])
    assert_bits_equal(host_bits(out), orc.ag_gemm(sh[rank].copy(), host_bits(xc["B"]), sh, R, rank),
                      "AG 224")


def test_auto_choice_matches_256_float(orc):
    """At M=4096, N=6288 the host picks 224-row tiles; on float inputs the
    result differs from forced 256-row tiles only by fp32 summation order."""
    w = wl.WORKLOADS["kda4096_ar"]
    x = wl.make_inputs(w, device=DEV)
    a = gc.gemm_ar(x["A"], x["B"], x["peers"], R=w.R, rank=w.rank)
    b = gc.gemm_ar(x["A"], x["B"], x["peers"], R=w.R, rank=w.rank, tile_rows=256)
    torch.cuda.synchronize()
    assert_close(host_bits(a), host_bits(b), "auto vs 256-row tiles")


def test_tile_rows_rejected():
    """Heights other than 0, 64, 128, 224 and 256 are refused before any launch."""
    A = torch.zeros((256, 64), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((1, 256, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="invalid argument"):
        gc.gemm_ar(A, B, P, R=2, rank=0, tile_rows=96)
