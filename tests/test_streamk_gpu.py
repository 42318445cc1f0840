"""Work split along K: tiles shared by several workgroups (each finishing its
share of the tile from the others' partials) must give exactly what whole
tiles give on integer inputs (every partial sum exact in fp32), in all three
modes, across shapes that exercise the split: 2 to 16 chunks per tile, a last
chunk shorter than the others, chunks taking no, one or two peers' items,
shapes the host does not split (too few K-steps, peer items past the K loop),
and back-to-back launches (arrival counters, flags and claims carry a
per-launch epoch and are never reset).  The split tests run with 256-row tiles
(tile_rows=256) and with the host's own choice, which takes 64- or 128-row
tiles for most of these shapes (4 or 8 hand-over segments per wave instead of
16)."""
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


# Comments: the plan with 256-row tiles.
SHAPES = [
    (300, 1040, 1024, 4),    # 10 tiles, 32 K-steps, 3 peers: 4 chunks of 8 steps
    (64, 264, 4096, 4),      # 2 tiles, 128 K-steps: each tile in 16 chunks
    (513, 520, 896, 2),      # 9 tiles, 28 K-steps: chunks of 8, 8, 8 and 4 steps
    (1024, 4096, 2048, 4),   # 64 tiles in 2 chunks of 32 steps, 3 peers: 2, 1
    (1000, 776, 72, 8),      # 3 K-steps: not split
    (2304, 2560, 256, 4),    # 90 tiles, 8 K-steps: not split
    (1000, 776, 1024, 8),    # 7 peers need 56 item steps, more than 32: not split
    (256, 3648, 7168, 8),    # 15 tiles in 10 chunks of 24 steps, 7 peers: one each for 7
    (512, 6400, 3072, 8),    # 50 tiles in 3 chunks of 32 steps, 7 peers: 3, 2, 2
    (300, 1040, 4096, 4),    # 10 tiles in 8 chunks of 16 steps, 3 peers
    (200, 600, 2560, 8),     # 3 ragged tiles, 10 chunks, 7 peers
]


@pytest.mark.parametrize("rows", [256, 0])
@pytest.mark.parametrize("M,N,K,R", SHAPES)
def test_ar_split_equals_whole(orc, M, N, K, R, rows):
    log(f"stream-K AR M={M} N={N} K={K} R={R} tile_rows={rows}")
    xc = wl.integer_inputs("ar", M, N, K, R, seed=M + N + K)
    x = to_dev(xc)
    whole = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=1, workspace=False)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    split = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=1, status=status,
                       tile_rows=rows)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_bits_equal(host_bits(split), host_bits(whole), "split vs whole")
    assert_bits_equal(host_bits(split), orc.gemm_ar(host_bits(xc["A"]), host_bits(xc["B"]),
                                                    host_bits(xc["peers"]), R), "split vs oracle")


@pytest.mark.parametrize("rows", [256, 0])
@pytest.mark.parametrize("M,N,K,R", SHAPES[:3] + SHAPES[-2:])
def test_rs_split_all_ranks(orc, M, N, K, R, rows):
    log(f"stream-K RS M={M} N={N} K={K} R={R} tile_rows={rows}")
    xc = wl.integer_inputs("rs", M, N, K, R, seed=M + 2 * K)
    x = to_dev(xc)
    A, B, peers = (host_bits(xc[k]) for k in ("A", "B", "peers"))
    for rank in range(R):
        ws = filled((M, N))
        out = gc.gemm_rs(x["A"], x["B"], x["peers"], ws, R=R, rank=rank, tile_rows=rows)
        torch.cuda.synchronize()
        ws_ref = np.full((M, N), SENTINEL, np.uint16)
        ref, ws_ref = orc.gemm_rs(A, B, peers, R, rank, ws_ref)
        assert_bits_equal(host_bits(out), ref, f"RS split rank {rank}")
        assert_bits_equal(host_bits(ws), ws_ref, f"RS split ws rank {rank}")


@pytest.mark.parametrize("rows", [256, 0])
@pytest.mark.parametrize("Ms,N,K,R", [(100, 520, 1024, 4), (512, 1040, 896, 8)])
def test_ag_split(orc, Ms, N, K, R, rows):
    log(f"stream-K AG Ms={Ms} N={N} K={K} R={R} tile_rows={rows}")
    rank = R - 1
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=Ms + K)
    x = to_dev(xc)
    flags = torch.ones(R, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, R=R, rank=rank, epoch=1,
                     tile_rows=rows)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    sh = host_bits(xc["shards"])
    assert_bits_equal(host_bits(out), orc.ag_gemm(sh[rank].copy(), host_bits(xc["B"]), sh, R, rank),
                      "AG split")


def test_back_to_back_launches(orc):
    """Many launches on one workspace: each must see only its own partials."""
    M, N, K, R = 300, 520, 2048, 4
    outs = []
    inputs = []
    for i in range(6):
        xc = wl.integer_inputs("ar", M, N, K, R, seed=100 + i)
        x = to_dev(xc)
        inputs.append(xc)
        outs.append(gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=0))
    torch.cuda.synchronize()
    for i, (xc, o) in enumerate(zip(inputs, outs)):
        assert_bits_equal(host_bits(o), orc.gemm_ar(host_bits(xc["A"]), host_bits(xc["B"]),
                                                    host_bits(xc["peers"]), R), f"launch {i}")


def test_split_float_inputs_close(orc):
    """Float inputs: the split changes only the fp32 summation order."""
    w = wl.Workload("sk", "ar", 512, 6288, 7168, 8, 0, 1.0, 1 / np.sqrt(7168))
    x = wl.make_inputs(w, device=DEV)
    a = gc.gemm_ar(x["A"], x["B"], x["peers"], R=8, rank=0)
    b = gc.gemm_ar(x["A"], x["B"], x["peers"], R=8, rank=0, workspace=False)
    torch.cuda.synchronize()
    assert_close(host_bits(a), host_bits(b), "split vs whole (float)")


@pytest.mark.parametrize("mode,M,N,K,R", [
    ("ar", 4352, 4096, 64, 2),   # 17 x 16 = 272 tiles: one full round of 256, then 16
    ("rs", 4352, 4104, 40, 4),   # 17 x 17 = 289 tiles, ragged N and K
    ("ag", 600, 4096, 72, 8),    # 8 shards x 3 x 16 = 384 tiles
])
def test_whole_tiles_partial_last_round(orc, mode, M, N, K, R):
    """Whole tiles only (no workspace) with more tiles than compute units and a
    last round that leaves workgroups idle: every tile exactly once."""
    log(f"whole tiles {mode} M={M} N={N} K={K} R={R}")
    rank = 1
    xc = wl.integer_inputs(mode, M, N, K, R, rank=rank, seed=M + N)
    x = to_dev(xc)
    Bh = host_bits(xc["B"])
    if mode == "ar":
        out = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=rank,
                         workspace=False)
        torch.cuda.synchronize()
        ref = orc.gemm_ar(host_bits(xc["A"]), Bh, host_bits(xc["peers"]), R)
        assert_bits_equal(host_bits(out), ref, "AR whole tiles")
    elif mode == "rs":
        ws = filled((M, N))
        out = gc.gemm_rs(x["A"], x["B"], x["peers"], ws, R=R, rank=rank, workspace=False)
        torch.cuda.synchronize()
        ws_ref = np.full((M, N), SENTINEL, np.uint16)
        ref, ws_ref = orc.gemm_rs(host_bits(xc["A"]), Bh, host_bits(xc["peers"]), R, rank, ws_ref)
        assert_bits_equal(host_bits(out), ref, "RS whole tiles")
        assert_bits_equal(host_bits(ws), ws_ref, "RS whole tiles ws")
    else:
        flags = torch.ones(R, dtype=torch.int32, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, filled((R * M, N)), R=R,
                         rank=rank, epoch=1, workspace=False)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        sh = host_bits(xc["shards"])
        assert_bits_equal(host_bits(out), orc.ag_gemm(sh[rank].copy(), Bh, sh, R, rank),
                          "AG whole tiles")


@pytest.mark.parametrize("mode,M,N,K,R", [
    ("ar", 8448, 2048, 4096, 4),   # 33 x 8 = 264 tiles: a full round, then 8 tiles in 8 chunks
    ("rs", 8448, 2048, 4096, 4),   # the same; rank 3's slice reaches into the split tiles
    ("ag", 1024, 2304, 4096, 8),   # 8 shards x 4 x 9 = 288 tiles: a full round, then 32 in 4 chunks
])
def test_tail_round_split_equals_whole(orc, mode, M, N, K, R):
    """More tiles than CUs: the full rounds run as whole tiles and the tiles
    of the last partial round are split along K in a second launch.  Bit-exact
    against whole tiles on integer inputs, and sampled rows (the last ones,
    in the split tiles, and some before) against the oracle."""
    log(f"tail split {mode} M={M} N={N} K={K} R={R}")
    rank = R - 1
    xc = wl.integer_inputs(mode, M, N, K, R, rank=rank, seed=M + 3 * K)
    x = to_dev(xc)
    Bh = host_bits(xc["B"])
    rows = np.r_[0:64, M // 2:M // 2 + 64, M - 320:M]
    if mode == "ar":
        whole = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=rank, workspace=False)
        split = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=rank)
        torch.cuda.synchronize()
        assert_bits_equal(host_bits(split), host_bits(whole), "AR tail split vs whole")
        Ah, Ph = host_bits(xc["A"]), host_bits(xc["peers"])
        ref = orc.ar_rows(Ah[rows].copy(), Bh, Ph[:, rows].copy())
        assert_bits_equal(host_bits(split)[rows], ref, "AR tail split vs oracle rows")
    elif mode == "rs":
        ws_w, ws_s = filled((M, N)), filled((M, N))
        whole = gc.gemm_rs(x["A"], x["B"], x["peers"], ws_w, R=R, rank=rank, workspace=False)
        split = gc.gemm_rs(x["A"], x["B"], x["peers"], ws_s, R=R, rank=rank)
        torch.cuda.synchronize()
        assert_bits_equal(host_bits(split), host_bits(whole), "RS tail split vs whole")
        assert_bits_equal(host_bits(ws_s), host_bits(ws_w), "RS tail split ws vs whole")
    else:
        flags = torch.ones(R, dtype=torch.int32, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        whole = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, R=R, rank=rank, epoch=1,
                           workspace=False)
        split = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, filled((R * M, N)), R=R,
                           rank=rank, epoch=1)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert_bits_equal(host_bits(split), host_bits(whole), "AG tail split vs whole")
        sh = host_bits(xc["shards"]).reshape(R * M, K)
        arows = np.r_[0:64, R * M - 320:R * M]
        ref = orc.ar_rows(sh[arows].copy(), Bh, None)
        assert_bits_equal(host_bits(split)[arows], ref, "AG tail split vs oracle rows")


@pytest.mark.parametrize("rows", [256, 0])
@pytest.mark.parametrize("mode,M,N,K,R", [
    ("ar", 256, 3648, 7168, 8),    # 15 tiles, 10 chunks each (128 rows: 30 tiles, 7 chunks)
    ("rs", 300, 1040, 4096, 4),    # 10 tiles, 8 chunks each (64 rows: 25 tiles, 8 chunks)
    ("ag", 100, 520, 1024, 4),     # 12 tiles, 4 chunks each (64 rows: 24 tiles, 4 chunks)
])
def test_split_units_that_give_up(orc, mode, M, N, K, R, rows):
    """The split hand-over's fallback, forced from the host: with the units'
    wait limited to one poll, nearly every unit that is not the last to
    arrive leaves its share, and the last one finishes it.  The result must
    not change (bit-exact on integer inputs)."""
    log(f"split units giving up: {mode} M={M} N={N} K={K} R={R}")
    rank = 1
    xc = wl.integer_inputs(mode, M, N, K, R, rank=rank, seed=M + 7 * K)
    x = to_dev(xc)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    if mode == "ar":
        split = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=rank, status=status,
                           tile_rows=rows, split_wait_spins=1)
        torch.cuda.synchronize()
        whole = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=rank, workspace=False)
    elif mode == "rs":
        ws_s = filled((M, N))
        split = gc.gemm_rs(x["A"], x["B"], x["peers"], ws_s, R=R, rank=rank, status=status,
                           tile_rows=rows, split_wait_spins=1)
        torch.cuda.synchronize()
        ws_w = filled((M, N))
        whole = gc.gemm_rs(x["A"], x["B"], x["peers"], ws_w, R=R, rank=rank, workspace=False)
        torch.cuda.synchronize()
        assert_bits_equal(host_bits(ws_s), host_bits(ws_w), "RS ws, units giving up")
    else:
        flags = torch.ones(R, dtype=torch.int32, device=DEV)
        split = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, filled((R * M, N)), R=R,
                           rank=rank, epoch=1, tile_rows=rows, split_wait_spins=1)
        torch.cuda.synchronize()
        st2 = torch.zeros(1, dtype=torch.int32, device=DEV)
        whole = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, st2, R=R, rank=rank, epoch=1,
                           workspace=False)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert_bits_equal(host_bits(split), host_bits(whole), f"{mode} split with units giving up")
