"""gemm_ar_noalloc, the GEMM-AR entry point that allocates nothing (its K-split
state lives in the library's static per-device scratch), against gemm_ar with
a workspace, called through the C ABI: two calls in a row on shapes whose
tiles are split along K, the second smaller than the first (so it runs on the
state the first left in the scratch).  Integer inputs must agree bit for bit
with gemm_ar and with the oracle; the seeded float inputs of the same shapes
within |gpu - ref| <= 1e-2 * |ref| + 1e-2 of gemm_ar's result."""
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, host_bits, log
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FC1

# (M, N, K, R): the first larger than the second; both split along K
CALLS = [(512, 2064, 4096, 8), (200, 1040, 2048, 4)]


def filled(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


@pytest.mark.parametrize("kind", ["integer", "float"])
def test_noalloc_matches_gemm_ar(kind):
    orc = load_oracle()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for i, (M, N, K, R) in enumerate(CALLS):
        p = gc.plan("ar", M, N, K, R, cus=cus)
        log(f"call {i}: {kind} M={M} N={N} K={K} R={R} plan {p}")
        assert p["units"] > 0, "the shape must split along K (else the scratch is not used)"
        if kind == "integer":
            xc = wl.integer_inputs("ar", M, N, K, R, seed=100 + i)
        else:
            xc = wl.make_inputs(wl.Workload("noalloc", "ar", M, N, K, R, 0, 1.0, K ** -0.5,
                                            seed=100 + i))
        x = {k: v.to(DEV) for k, v in xc.items()}
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = filled((M, N))
        gc.gemm_ar_noalloc(x["A"], x["B"], x["peers"], out, R=R, rank=0, status=status)
        ref = gc.gemm_ar(x["A"], x["B"], x["peers"], filled((M, N)), R=R, rank=0)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        if kind == "integer":
            assert_bits_equal(host_bits(out), host_bits(ref), f"call {i}: noalloc vs gemm_ar")
            want = orc.gemm_ar(host_bits(xc["A"]), host_bits(xc["B"]), host_bits(xc["peers"]), R)
            assert_bits_equal(host_bits(out), want, f"call {i}: noalloc vs oracle")
        else:
            assert_close(host_bits(out), host_bits(ref), f"call {i}: noalloc vs gemm_ar")
