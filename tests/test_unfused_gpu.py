"""The unfused baseline's reduction kernel (gemm_coll_peer_sum) against the
oracle, and the whole unfused pipeline (library GEMM, then that kernel)
against the fused entry point.

The oracle has no separate peer-sum routine; ar_rows(I, L, peers) with the
identity as A gives bf16(L + sum of peers) with the sum taken in fp32 in the
order local, peer 0, 1, ... (the identity adds only exact zeros), which is
the definition the kernel follows.  Cases: a
ragged element count (a tail of n % 8 elements), peer blocks farther apart
than one block (a row slice of [R-1][M][N] partials), in place (out =
local), no peers (a copy), and the largest peer count (15)."""
import numpy as np
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, host_bits, log
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def orc():
    return load_oracle()


def ident_bits(n):
    return np.where(np.eye(n, dtype=bool), np.uint16(0x3F80), np.uint16(0)).astype(np.uint16)


def int_bf16(shape, lo, hi, g):
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.bfloat16)


def expect(orc, local, peers):
    """bf16(local + sum of peers) from the oracle (local [rows,N], peers [np,rows,N])."""
    rows = local.shape[0]
    return orc.ar_rows(ident_bits(rows), host_bits(local), host_bits(peers.contiguous()))


@pytest.mark.parametrize("rows,N,npeers", [(64, 256, 7), (5, 13, 3), (33, 1000, 15), (17, 264, 0),
                                           (1, 8, 1)])
def test_peer_sum_integers_exact(orc, rows, N, npeers):
    log(f"peer_sum integers rows={rows} N={N} npeers={npeers}")
    g = torch.Generator().manual_seed(rows * 131 + N + npeers)
    local = int_bf16((rows, N), -64, 64, g)
    n = rows * N
    stride = (n + 7) // 8 * 8 + 8          # blocks apart by more than one block
    big = int_bf16((max(npeers, 1), stride), -64, 64, g)
    peers_h = torch.as_strided(big, (npeers, rows, N), (stride, N, 1))
    ld, bd = local.to(DEV), big.to(DEV)
    pd = torch.as_strided(bd, (npeers, rows, N), (stride, N, 1))
    out = gc.peer_sum(ld, pd)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), expect(orc, local, peers_h), "peer_sum")


def test_peer_sum_float_and_in_place(orc):
    g = torch.Generator().manual_seed(3)
    rows, N, npeers = 96, 520, 7
    local = torch.randn(rows, N, generator=g).to(torch.bfloat16)
    peers = torch.randn(npeers, rows, N, generator=g).to(torch.bfloat16)
    ref = expect(orc, local, peers)
    ld = local.to(DEV)
    out = gc.peer_sum(ld, peers.to(DEV), ld)        # in place
    torch.cuda.synchronize()
    assert out.data_ptr() == ld.data_ptr()
    assert_close(host_bits(ld), ref, "peer_sum float, in place")


def test_peer_sum_row_slice(orc):
    """RS's use: rows [lo, hi) of [R-1][M][N] partials, block stride M*N."""
    g = torch.Generator().manual_seed(11)
    R, M, N = 8, 300, 264
    P = (M + R - 1) // R
    lo, hi = 2 * P, 3 * P
    local = int_bf16((M, N), -32, 32, g)
    peers = int_bf16((R - 1, M, N), -32, 32, g)
    ld, pd = local.to(DEV), peers.to(DEV)
    out = gc.peer_sum(ld[lo:hi], pd[:, lo:hi])
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), expect(orc, local[lo:hi], peers[:, lo:hi]), "peer_sum slice")


def test_unfused_pipeline_matches_fused():
    """Library GEMM (bf16 local product) then peer_sum, against gemm_ar on
    the MLA shape: the unfused path rounds the local product to bf16 before
    the sum, so the two agree to the tolerance, not bit for bit."""
    w = wl.WORKLOADS["mla_ar"]
    x = wl.make_inputs(w, device=DEV)
    fused = gc.gemm_ar(x["A"], x["B"], x["peers"], R=w.R, rank=w.rank)
    local = torch.matmul(x["A"], x["B"])
    unfused = gc.peer_sum(local, x["peers"])
    torch.cuda.synchronize()
    assert_close(host_bits(unfused), host_bits(fused), "unfused vs fused (MLA)")
