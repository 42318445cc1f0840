"""GEMM-AR by the two-shot flow (gemm_ar_two_shot): the owned slice rows of
out and of every peer output slot equal the oracle's GEMM-RS slice bit for
bit on integer inputs, ws equals the oracle's published partial, and every
other row of out and peer_out is left as it was.  All ranks of ragged
shapes, including a slice that runs past M and an empty slice, at both tile
heights; and, on float inputs at M=4096, the same bits as gemm_rs."""
import numpy as np
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, host_bits, log
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FC1


@pytest.fixture(scope="module")
def orc():
    return load_oracle()


def filled(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def check_rank(orc, xc, x, M, N, R, rank, tile_rows):
    P = -(-M // R)
    lo, hi = min(rank * P, M), min(rank * P + P, M)
    ws = filled((M, N))
    out = filled((M, N))
    peer_out = filled((R - 1, M, N))
    gc.gemm_ar_two_shot(x["A"], x["B"], x["peers"], ws, peer_out, out, R=R, rank=rank,
                        workspace=False, tile_rows=tile_rows)
    torch.cuda.synchronize()
    ws_ref = np.full((M, N), SENTINEL, np.uint16)
    slice_ref, ws_ref = orc.gemm_rs(host_bits(xc["A"]), host_bits(xc["B"]), host_bits(xc["peers"]),
                                    R, rank, ws_ref)
    want = np.full((M, N), SENTINEL, np.uint16)
    want[lo:hi] = slice_ref[:hi - lo]
    assert_bits_equal(host_bits(out), want, f"two-shot out rank {rank}")
    po = host_bits(peer_out)
    for q in range(R - 1):
        assert_bits_equal(po[q], want, f"two-shot peer_out[{q}] rank {rank}")
    assert_bits_equal(host_bits(ws), ws_ref, f"two-shot ws rank {rank}")


@pytest.mark.parametrize("tile_rows", [256, 224])
@pytest.mark.parametrize("M,N,K,R", [
    (1001, 520, 256, 8),     # P = 126: the last slice runs past M
    (300, 264, 96, 4),       # ragged N, 3 K-steps (peer items after the K loop)
    (10, 256, 64, 8),        # P = 2: ranks 5..7 own no rows
])
def test_two_shot_all_ranks(orc, M, N, K, R, tile_rows):
    log(f"two-shot AR M={M} N={N} K={K} R={R} tile_rows={tile_rows}")
    xc = wl.integer_inputs("rs", M, N, K, R, seed=M + 3 * N + K)
    x = {k: v.to(DEV) for k, v in xc.items()}
    for rank in range(R):
        check_rank(orc, xc, x, M, N, R, rank, tile_rows)


def test_two_shot_matches_rs_float():
    """Float inputs at M=4096: the slice and ws equal gemm_rs's bits (same
    kernel arithmetic), and the peer slots equal the slice."""
    w = wl.WORKLOADS["kda4096_ar2"]
    x = wl.make_inputs(w, device=DEV)
    M, N, R = w.M, w.N, w.R
    P = -(-M // R)
    for rank in (0, 5):
        ws_a, ws_b = filled((M, N)), filled((M, N))
        out = filled((M, N))
        peer_out = filled((R - 1, M, N))
        gc.gemm_ar_two_shot(x["A"], x["B"], x["peers"], ws_a, peer_out, out, R=R, rank=rank)
        rs = gc.gemm_rs(x["A"], x["B"], x["peers"], ws_b, R=R, rank=rank)
        torch.cuda.synchronize()
        lo, hi = rank * P, min(rank * P + P, M)
        o, r = host_bits(out), host_bits(rs)
        assert_bits_equal(o[lo:hi], r[:hi - lo], f"slice vs gemm_rs rank {rank}")
        assert (o[:lo] == SENTINEL).all() and (o[hi:] == SENTINEL).all()
        po = host_bits(peer_out)
        for q in range(R - 1):
            assert_bits_equal(po[q], o, f"peer slot {q} rank {rank}")
        assert_bits_equal(host_bits(ws_a), host_bits(ws_b), f"ws rank {rank}")
