"""AG-GEMM with the shards arriving while the kernel runs: ag_push_shards
copies the other ranks' shards into the receive buffer on a side stream
through the DMA engines and raises each shard's flag after its copy, while
ag_gemm, launched first on the main stream, holds every compute unit and
polls the flags.  The output must equal the oracle's bit for bit on integer
inputs, with no time-out, in two rounds on the same receive buffer (new
shard contents and a new epoch: a stale cached copy of the first round's
shards would show)."""
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, host_bits, log
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def orc():
    return load_oracle()


def test_push_alone():
    R, rank, Ms, K = 8, 3, 40, 264
    g = torch.Generator().manual_seed(1)
    src = torch.randint(-8, 9, (R, Ms, K), generator=g).to(torch.bfloat16).to(DEV)
    dst = torch.zeros_like(src)
    flags = torch.zeros(R, dtype=torch.int32, device=DEV)
    ew = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    gc.ag_push_shards(src, dst, flags, ew, R=R, rank=rank)
    torch.cuda.synchronize()
    for q in range(R):
        if q == rank:
            assert bool((dst[q] == 0).all())
        else:
            assert torch.equal(dst[q], src[q]), q
    want = [0 if q == rank else 5 for q in range(R)]
    assert flags.cpu().tolist() == want


@pytest.mark.parametrize("Ms,N,K,R,rank", [(256, 520, 512, 8, 5), (300, 1040, 256, 4, 0),
                                            (512, 2048, 512, 8, 2)])  # the last: 256 units, every CU
def test_kernel_consumes_shards_as_they_arrive(orc, Ms, N, K, R, rank):
    recv = torch.zeros((R, Ms, K), dtype=torch.bfloat16, device=DEV)
    flags = torch.zeros(R, dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for rnd, epoch in ((0, 1), (1, 2)):
        log(f"AG arrival Ms={Ms} N={N} K={K} R={R} rank={rank} round {rnd}")
        xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=17 * Ms + rnd)
        src = xc["shards"].to(DEV)
        A = xc["shards"][rank].contiguous().to(DEV)
        B = xc["B"].to(DEV)
        ew = torch.full((1,), epoch, dtype=torch.int32, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = torch.empty((R * Ms, N), dtype=torch.bfloat16, device=DEV)
        torch.cuda.synchronize()
        # the kernel first (it takes every compute unit and waits), then the pushes
        gc.ag_gemm(A, B, recv, flags, status, out, R=R, rank=rank, epoch=epoch, stream=main)
        gc.ag_push_shards(src, recv, flags, ew, R=R, rank=rank, stream=side)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"round {rnd}: status {int(status.item())}"
        sh = host_bits(xc["shards"])
        assert_bits_equal(host_bits(out), orc.ag_gemm(sh[rank].copy(), host_bits(xc["B"]), sh, R, rank),
                          f"AG with arriving shards, round {rnd}")
