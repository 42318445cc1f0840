"""The named workloads at full size, in the launch configuration the
benchmark times (default workspace, the host's own tile height), checked on
every output row against the oracle.

Two input sets per workload:
  * small integers (|A|, |B| <= 2, |peer| <= 64): every partial sum is an
    integer below 2^24, so fp32 sums are exact in any order and the result
    must equal the oracle's bit for bit.  This pins the GEMM part, the peer
    adds, RS row selection and AG shard placement exactly, including where
    the float inputs cannot: the tiny and odd-M configs scale both A and B
    by 1/sqrt(K), so their GEMM part is far below the tolerance of the peer
    sum;
  * the workload's own seeded Gaussian inputs: every element within
    |gpu - ref| <= 1e-2 * |ref| + 1e-2.
RS also checks that the owned rows of ws stay untouched, the padding rows
of the slice are zero, and (odd M) the row selection by a row-ID encoding,
for ranks 0, 5 and 7.  Each case logs the launch plan it runs, so the
kernel instance it covers (e.g. 224-row tiles with non-temporal peer loads
for the M=4096 GEMM-AR) is on record.
"""
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


def filled(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def plan_of(w, rank=None):
    mode = {"ar": "ar", "rs": "rs", "ar2": "rs", "ag": "ag"}[w.mode]
    p = gc.plan(mode, w.M, w.N, w.K, w.R, w.rank if rank is None else rank,
                cus=torch.cuda.get_device_properties(0).multi_processor_count)
    log(f"  plan: {p}")
    return p


def int_inputs(w):
    return wl.integer_inputs("ag" if w.mode == "ag" else "ar", w.M, w.N, w.K, w.R, rank=w.rank,
                             seed=w.M + w.N + w.K)


def check_ar(orc, w, xc, exact):
    x = {k: v.to(DEV) for k, v in xc.items()}
    plan_of(w)
    out = filled((w.M, w.N))
    gc.gemm_ar(x["A"], x["B"], x["peers"], out, R=w.R, rank=w.rank)
    torch.cuda.synchronize()
    got = host_bits(out)
    del x, out
    ref = orc.gemm_ar(host_bits(xc["A"]), host_bits(xc["B"]), host_bits(xc["peers"]), w.R)
    (assert_bits_equal if exact else assert_close)(got, ref, f"{w.name} AR, all {w.M} rows")


def check_rs(orc, w, xc, exact, ranks):
    x = {k: v.to(DEV) for k, v in xc.items()}
    A, B, peers = (host_bits(xc[k]) for k in ("A", "B", "peers"))
    cmp = assert_bits_equal if exact else assert_close
    for r in ranks:
        plan_of(w, r)
        P, lo, hi = orc.rs_slice(w.M, w.R, r)
        ws = filled((w.M, w.N))
        out = filled((P, w.N))
        gc.gemm_rs(x["A"], x["B"], x["peers"], ws, out, R=w.R, rank=r)
        torch.cuda.synchronize()
        got_out, got_ws = host_bits(out), host_bits(ws)
        ws_ref = np.full((w.M, w.N), SENTINEL, np.uint16)
        ref, ws_ref = orc.gemm_rs(A, B, peers, w.R, r, ws_ref)
        cmp(got_out, ref, f"{w.name} RS rank {r}: all {P} slice rows")
        assert np.all(got_out[hi - lo:] == 0), "padding rows of the slice must be zero"
        own = np.zeros(w.M, bool)
        own[lo:hi] = True
        assert np.all(got_ws[own] == SENTINEL), f"rank {r}: owned ws rows were written"
        cmp(got_ws[~own], ws_ref[~own], f"{w.name} RS rank {r}: all {int((~own).sum())} ws rows")


def check_ar2(orc, w, xc, exact):
    """Two-shot AR: the slice rows of out and of every peer output equal the
    RS slice; ws as RS; rows outside the slice untouched."""
    x = {k: v.to(DEV) for k, v in xc.items()}
    plan_of(w)
    P, lo, hi = orc.rs_slice(w.M, w.R, w.rank)
    ws = filled((w.M, w.N))
    out = filled((w.M, w.N))
    peer_out = filled((w.R - 1, w.M, w.N))
    gc.gemm_ar_two_shot(x["A"], x["B"], x["peers"], ws, peer_out, out, R=w.R, rank=w.rank)
    torch.cuda.synchronize()
    got_out, got_ws, got_po = host_bits(out), host_bits(ws), host_bits(peer_out)
    del x, out, ws, peer_out
    ws_ref = np.full((w.M, w.N), SENTINEL, np.uint16)
    ref, ws_ref = orc.gemm_rs(host_bits(xc["A"]), host_bits(xc["B"]), host_bits(xc["peers"]),
                              w.R, w.rank, ws_ref)
    cmp = assert_bits_equal if exact else assert_close
    cmp(got_out[lo:hi], ref[:hi - lo], f"{w.name} two-shot out slice")
    for q in range(w.R - 1):
        cmp(got_po[q, lo:hi], ref[:hi - lo], f"{w.name} two-shot peer_out[{q}] slice")
    own = np.zeros(w.M, bool)
    own[lo:hi] = True
    assert np.all(got_out[~own] == SENTINEL) and np.all(got_po[:, ~own] == SENTINEL)
    assert np.all(got_ws[own] == SENTINEL)
    cmp(got_ws[~own], ws_ref[~own], f"{w.name} two-shot ws")


def check_ag(orc, w, xc, exact):
    x = {k: v.to(DEV) for k, v in xc.items()}
    plan_of(w)
    flags = torch.ones(w.R, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = filled((w.R * w.M, w.N))
    gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, out, R=w.R, rank=w.rank, epoch=1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = host_bits(out)
    del x, out
    sh = host_bits(xc["shards"])
    ref = orc.ag_gemm(host_bits(xc["A"]), host_bits(xc["B"]), sh, w.R, w.rank)
    (assert_bits_equal if exact else assert_close)(got, ref, f"{w.name} AG, all {w.R * w.M} rows")


ALL = ["tiny_ar", "mla_ar", "mla_rs", "kda512_ar", "kda1024_ar", "kda4096_ar", "kda4096_ar2",
       "rs_odd", "ag_kda"]


def run(orc, name, exact):
    w = wl.WORKLOADS[name]
    log(f"workload {name} ({'integer, bit-exact' if exact else 'seeded floats, tolerance'}): {w}")
    xc = int_inputs(w) if exact else wl.make_inputs(w)
    if w.mode == "ar":
        check_ar(orc, w, xc, exact)
    elif w.mode == "rs":
        ranks = (0, w.rank, w.R - 1) if name == "rs_odd" else (w.rank,)
        check_rs(orc, w, xc, exact, ranks)
    elif w.mode == "ar2":
        check_ar2(orc, w, xc, exact)
    else:
        check_ag(orc, w, xc, exact)


@pytest.mark.parametrize("name", ALL)
def test_workload_integer_bit_exact(orc, name):
    run(orc, name, True)


@pytest.mark.parametrize("name", ALL)
def test_workload_float_every_row(orc, name):
    run(orc, name, False)


def test_headline_runs_the_224_row_nt_instance():
    """The M=4096 GEMM-AR launch is the 224-row, non-temporal-peer kernel
    instance in two rounds of whole tiles: the instance the two tests above
    check at that size."""
    w = wl.WORKLOADS["kda4096_ar"]
    p = plan_of(w)
    assert (p["tile_rows"], p["peer_nt"], p["units"]) == (224, 1, 0)
    w = wl.WORKLOADS["rs_odd"]
    p = plan_of(w)
    assert (p["tile_rows"], p["peer_nt"]) == (256, 1)


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
