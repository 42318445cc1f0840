"""64- and 128-row output tiles (tile_rows=64 / 128; the host picks them by
itself when a shard has at most 64 / 128 rows): on integer inputs, where every
partial sum is exact in fp32, the results equal the oracle's bit for bit in
all three modes -- several row tiles with a ragged last one, ragged N and K,
peer items after the K loop, every RS rank (slice edges inside a tile), and
tiles split along K (the hand-over then has 4 or 8 segments per wave, fewer
than a tile's units at 16 chunks).  Also: the automatic choice at decode
sizes against forced 256-row tiles on float inputs."""
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


# (M, N, K, R, tile_rows, workspace)
AR_CASES = [
    (300, 520, 512, 4, 64, False),    # 5 row tiles (the last 44 rows) x 3, whole
    (300, 520, 512, 4, 128, False),   # 3 row tiles (the last 44 rows) x 3, whole
    (1000, 776, 72, 8, 64, False),    # 3 K-steps: 53 of the 56 peer items after the K loop
    (130, 264, 96, 2, 128, False),    # 2 row tiles, the second 2 rows
    (300, 520, 4096, 4, 64, True),    # 15 tiles split along K, 3 peers
    (64, 264, 4096, 4, 0, True),      # automatic: 64 rows, 2 tiles in 16 chunks
    (16, 1040, 2048, 8, 0, True),     # automatic: 64 rows, 5 tiles split, 7 peers
    (100, 1040, 3072, 8, 0, True),    # automatic: 128 rows, 5 tiles split, 7 peers
    (128, 256, 512, 2, 0, True),      # automatic: 128 rows, one tile in 2 chunks
]


@pytest.mark.parametrize("M,N,K,R,rows,ws", AR_CASES)
def test_ar_short(orc, M, N, K, R, rows, ws):
    log(f"short-tile AR M={M} N={N} K={K} R={R} tile_rows={rows} workspace={ws}")
    xc = wl.integer_inputs("ar", M, N, K, R, seed=11 * M + N + K + rows)
    x = to_dev(xc)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kw = {} if ws else {"workspace": False}
    out = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=1, status=status,
                     tile_rows=rows, **kw)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_bits_equal(host_bits(out), orc.gemm_ar(host_bits(xc["A"]), host_bits(xc["B"]),
                                                  host_bits(xc["peers"]), R), "AR short tiles")


@pytest.mark.parametrize("M,N,K,R,rows,ws", [
    (300, 520, 512, 4, 64, False),    # slices of 75 rows: edges inside 64-row tiles
    (300, 520, 512, 4, 128, False),
    (60, 264, 2048, 4, 0, True),      # automatic: 64 rows, split; slices of 15 rows
    (300, 520, 4096, 4, 128, True),   # 9 tiles split along K
])
def test_rs_short_all_ranks(orc, M, N, K, R, rows, ws):
    log(f"short-tile RS M={M} N={N} K={K} R={R} tile_rows={rows} workspace={ws}")
    xc = wl.integer_inputs("rs", M, N, K, R, seed=5 * M + K + rows)
    x = to_dev(xc)
    A, B, peers = (host_bits(xc[k]) for k in ("A", "B", "peers"))
    kw = {} if ws else {"workspace": False}
    for rank in range(R):
        wsb = filled((M, N))
        out = gc.gemm_rs(x["A"], x["B"], x["peers"], wsb, R=R, rank=rank, tile_rows=rows, **kw)
        torch.cuda.synchronize()
        ws_ref = np.full((M, N), SENTINEL, np.uint16)
        ref, ws_ref = orc.gemm_rs(A, B, peers, R, rank, ws_ref)
        assert_bits_equal(host_bits(out), ref, f"RS short rank {rank}")
        assert_bits_equal(host_bits(wsb), ws_ref, f"RS short ws rank {rank}")


@pytest.mark.parametrize("Ms,N,K,R,rows,ws", [
    (100, 520, 256, 4, 64, False),    # 2 row tiles per shard
    (40, 520, 1024, 8, 0, True),      # automatic: 64 rows, 8 shards x 3 tiles split
    (100, 520, 1024, 4, 0, True),     # automatic: 128 rows
])
def test_ag_short(orc, Ms, N, K, R, rows, ws):
    log(f"short-tile AG Ms={Ms} N={N} K={K} R={R} tile_rows={rows} workspace={ws}")
    rank = 2
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=Ms + 3 * K + rows)
    x = to_dev(xc)
    flags = torch.ones(R, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    kw = {} if ws else {"workspace": False}
    out = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, filled((R * Ms, N)), R=R,
                     rank=rank, epoch=1, tile_rows=rows, **kw)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    sh = host_bits(xc["shards"])
    assert_bits_equal(host_bits(out), orc.ag_gemm(sh[rank].copy(), host_bits(xc["B"]), sh, R, rank),
                      "AG short tiles")


@pytest.mark.parametrize("name", ["kda64_ar", "kda16_ar"])
def test_decode_auto_matches_256_float(orc, name):
    """At decode sizes the host picks 64-row tiles; on float inputs the result
    differs from forced 256-row tiles only by fp32 summation order."""
    w = wl.WORKLOADS[name]
    x = wl.make_inputs(w, device=DEV)
    a = gc.gemm_ar(x["A"], x["B"], x["peers"], R=w.R, rank=w.rank)
    b = gc.gemm_ar(x["A"], x["B"], x["peers"], R=w.R, rank=w.rank, tile_rows=256)
    torch.cuda.synchronize()
    assert_close(host_bits(a), host_bits(b), f"{name}: auto vs 256-row tiles")
