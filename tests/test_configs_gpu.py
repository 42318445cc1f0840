"""The named workloads at full size, in the launch configuration the
benchmark times, checked on sampled rows that the oracle computes one by one,
plus properties that hold at any size (every output element written, owned
ws rows untouched), and a bit-exact row-ID check of the RS slice selection
at the odd-M size.
"""
import numpy as np
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, host_bits, log, sample_rows
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FC1


@pytest.fixture(scope="module")
def orc():
    return load_oracle()


def filled(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def no_sentinel(t) -> bool:
    return not bool((t.view(torch.int16) == SENTINEL).any())


AR_RS = ["tiny_ar", "mla_ar", "mla_rs", "kda512_ar", "kda1024_ar", "kda4096_ar", "rs_odd"]


@pytest.mark.parametrize("name", AR_RS)
def test_workload_sampled(orc, name):
    w = wl.WORKLOADS[name]
    log(f"workload {name}: {w}")
    x = wl.make_inputs(w, device=DEV)
    B_h = host_bits(x["B"])
    if w.mode == "ar":
        out = filled((w.M, w.N))
        gc.gemm_ar(x["A"], x["B"], x["peers"], out, R=w.R, rank=w.rank)
        torch.cuda.synchronize()
        assert no_sentinel(out), "some output element was not written"
        rows = sample_rows(w.M, seed=w.M)
        idx = torch.tensor(rows, device=DEV)
        ref = orc.ar_rows(host_bits(x["A"][idx]), B_h, host_bits(x["peers"][:, idx]))
        assert_close(host_bits(out[idx]), ref, f"{name} rows {len(rows)}")
        return
    # RS
    P, lo, hi = orc.rs_slice(w.M, w.R, w.rank)
    ws = filled((w.M, w.N))
    out = filled((P, w.N))
    gc.gemm_rs(x["A"], x["B"], x["peers"], ws, out, R=w.R, rank=w.rank)
    torch.cuda.synchronize()
    assert no_sentinel(out), "some slice element was not written"
    assert bool((ws[lo:hi].view(torch.int16) == SENTINEL).all()), "owned ws rows were written"
    assert no_sentinel(ws[:lo]) and no_sentinel(ws[hi:]), "some ws row was not written"
    owned = hi - lo
    t_rows = sample_rows(owned, seed=1) if owned > 0 else []
    if t_rows:
        g = torch.tensor([lo + t for t in t_rows], device=DEV)
        ref = orc.ar_rows(host_bits(x["A"][g]), B_h, host_bits(x["peers"][:, g]))
        assert_close(host_bits(out[torch.tensor(t_rows, device=DEV)]), ref, f"{name} slice rows")
    if owned < P:
        assert bool((out[owned:].float() == 0).all()), "padding rows must be zero"
    others = [i for i in sample_rows(w.M, seed=2) if not lo <= i < hi]
    g = torch.tensor(others, device=DEV)
    ref = orc.ar_rows(host_bits(x["A"][g]), B_h, None)
    assert_close(host_bits(ws[g]), ref, f"{name} ws rows")


def test_ag_workload_sampled(orc):
    w = wl.WORKLOADS["ag_kda"]
    log(f"workload ag_kda: {w}")
    x = wl.make_inputs(w, device=DEV)
    flags = torch.ones(w.R, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = filled((w.R * w.M, w.N))
    gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, out, R=w.R, rank=w.rank, epoch=1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert no_sentinel(out), "some output element was not written"
    B_h = host_bits(x["B"])
    rows = sample_rows(w.R * w.M, seed=3, extra=12,
                       must=tuple(q * w.M + d for q in range(w.R) for d in (0, w.M - 1)))
    src = []
    for g in rows:
        q, t = orc.ag_source(w.M, w.R, g)
        src.append(x["A"][t] if q == w.rank else x["shards"][q][t])
    A_rows = host_bits(torch.stack(src))
    ref = orc.ar_rows(A_rows, B_h, None)
    assert_close(host_bits(out[torch.tensor(rows, device=DEV)]), ref, f"ag_kda rows {len(rows)}")


def test_rs_odd_row_ids_bit_exact(orc):
    """Row-ID encoding at the odd-M size: A[i,0] = i mod 128, A[i,1] = i div 128,
    B[0,0] = B[1,1] = 1 and zero elsewhere, zero peers.  Output column 0 and 1
    then spell the source row of every slice row and ws row exactly."""
    w = wl.WORKLOADS["rs_odd"]
    M, N, K, R, rank = w.M, w.N, w.K, w.R, w.rank
    i = torch.arange(M, device=DEV)
    A = torch.zeros(M, K, dtype=torch.bfloat16, device=DEV)
    A[:, 0] = (i % 128).to(torch.bfloat16)
    A[:, 1] = (i // 128).to(torch.bfloat16)
    B = torch.zeros(K, N, dtype=torch.bfloat16, device=DEV)
    B[0, 0] = 1
    B[1, 1] = 1
    peers = torch.zeros(R - 1, M, N, dtype=torch.bfloat16, device=DEV)
    for r in (0, rank, R - 1):
        P, lo, hi = orc.rs_slice(M, R, r)
        ws = filled((M, N))
        out = gc.gemm_rs(A, B, peers, ws, R=R, rank=r)
        torch.cuda.synchronize()
        src = (out[:, 0].float() + 128 * out[:, 1].float()).to("cpu").numpy().astype(np.int64)
        want = np.zeros(P, np.int64)
        want[: hi - lo] = np.arange(lo, hi)
        assert np.array_equal(src, want), f"RS row selection, rank {r}"
        assert bool((out[:, 2:].float() == 0).all())
        own = np.zeros(M, bool)
        own[lo:hi] = True
        # (the owned rows of ws keep the NaN sentinel: decode only the others)
        ids = (ws[:, 0].float() + 128 * ws[:, 1].float()).to("cpu").numpy()
        wsrc = ids[~own].astype(np.int64)
        assert np.array_equal(wsrc, np.arange(M)[~own]), f"ws rows, rank {r}"
        assert bool((ws[lo:hi].view(torch.int16) == SENTINEL).all())
        log(f"  rank {r}: slice [{lo},{hi}) P={P} row ids exact")
