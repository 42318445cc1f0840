"""GPU parity: the HIP library, through its C ABI, against the CPU oracle.

Floating-point results must satisfy |gpu - ref| <= 1e-2*|ref| + 1e-2 element
by element; row selection, slicing and indexing are checked bit-exactly with
integer-valued inputs and row-ID encodings.
"""
import ctypes

import numpy as np
import pytest
import torch

import tensor_bf16_gemm_amd as gc
import workloads as wl
from gpu_util import assert_bits_equal, assert_close, host_bits, log
from oracle.oracle import load as load_oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FC1  # a NaN pattern no kernel result can take


@pytest.fixture(scope="module")
def orc():
    return load_oracle()


def to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def npb(t):
    return host_bits(t)


def filled(shape, pattern=SENTINEL):
    return torch.full(shape, pattern, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def run_rs(x, R, rank, M, N):
    ws = filled((M, N))
    out = gc.gemm_rs(x["A"], x["B"], x["peers"], ws, R=R, rank=rank)
    return out, ws


def run_ag(x, R, rank, epoch=1, max_spins=0, flags=None, workspace=None):
    if flags is None:
        flags = torch.full((R,), epoch, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, R=R, rank=rank, epoch=epoch,
                     max_spins=max_spins, workspace=workspace)
    return out, status


def check_rs_full(orc, xc, out, ws, R, rank, M, N, exact=False):
    """Whole-matrix RS check: out against the oracle; ws non-owned rows
    against bf16(A.B); owned ws rows untouched."""
    A, B, peers = (npb(xc[k]) for k in ("A", "B", "peers"))
    ws_ref = np.full((M, N), SENTINEL, np.uint16)
    ref, ws_ref = orc.gemm_rs(A, B, peers, R, rank, ws_ref)
    P, lo, hi = orc.rs_slice(M, R, rank)
    got_out, got_ws = npb(out), npb(ws)
    cmp = assert_bits_equal if exact else assert_close
    cmp(got_out, ref, f"RS out rank {rank}")
    own = np.zeros(M, bool)
    own[lo:hi] = True
    assert_bits_equal(got_ws[own], ws_ref[own], f"RS ws owned rows untouched rank {rank}")
    cmp(got_ws[~own], ws_ref[~own], f"RS ws rank {rank}")
    assert np.all(got_out[hi - lo:] == 0), "RS padding rows must be zero"


# ---------------------------------------------------------------------------
def test_tiny_ar_full(orc):
    w = wl.WORKLOADS["tiny_ar"]
    log(f"tiny_ar {w}")
    xc = wl.make_inputs(w)
    x = to_dev(xc)
    out = gc.gemm_ar(x["A"], x["B"], x["peers"], R=w.R, rank=w.rank)
    torch.cuda.synchronize()
    ref = orc.gemm_ar(npb(xc["A"]), npb(xc["B"]), npb(xc["peers"]), w.R)
    assert_close(npb(out), ref, "tiny_ar")


RAGGED = [(300, 520, 200, 4), (257, 264, 72, 2), (513, 1040, 512, 8), (31, 40, 64, 16)]


@pytest.mark.parametrize("M,N,K,R", RAGGED)
def test_ragged_ar(orc, M, N, K, R):
    log(f"ragged AR M={M} N={N} K={K} R={R}")
    w = wl.Workload("ragged", "ar", M, N, K, R, 0, 1.0, 1 / np.sqrt(K), 1.0, seed=M + K)
    xc = wl.make_inputs(w)
    x = to_dev(xc)
    out = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=0)
    torch.cuda.synchronize()
    ref = orc.gemm_ar(npb(xc["A"]), npb(xc["B"]), npb(xc["peers"]), R)
    assert_close(npb(out), ref, f"AR {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,R", RAGGED)
def test_ragged_rs_all_ranks(orc, M, N, K, R):
    log(f"ragged RS M={M} N={N} K={K} R={R}")
    w = wl.Workload("ragged", "rs", M, N, K, R, 0, 1.0, 1 / np.sqrt(K), 1.0, seed=M + K + 1)
    xc = wl.make_inputs(w)
    x = to_dev(xc)
    for rank in range(R):
        out, ws = run_rs(x, R, rank, M, N)
        torch.cuda.synchronize()
        check_rs_full(orc, xc, out, ws, R, rank, M, N)


@pytest.mark.parametrize("Ms,N,K,R", [(150, 520, 200, 4), (64, 264, 72, 8), (257, 40, 64, 2),
                                     (37, 264, 136, 16)])
def test_ragged_ag_all_ranks(orc, Ms, N, K, R):
    log(f"ragged AG Ms={Ms} N={N} K={K} R={R}")
    w = wl.Workload("ragged", "ag", Ms, N, K, R, 0, 1.0, 1 / np.sqrt(K), seed=Ms + K)
    xc = wl.make_inputs(w)
    x = to_dev(xc)
    shards = npb(xc["shards"])
    ref = orc.ag_gemm(shards[0].copy(), npb(xc["B"]), shards, R, 0)
    for rank in range(R):
        xr = dict(x, A=x["shards"][rank].contiguous())
        out, status = run_ag(xr, R, rank)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert_close(npb(out), ref, f"AG rank {rank}")


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,R", [(513, 1040, 512, 8), (1000, 776, 1000, 4), (130, 256, 2048, 2)])
def test_integer_inputs_bit_exact(orc, M, N, K, R):
    """Integer-valued inputs: every partial sum is exact in fp32, so the GPU
    must equal the oracle bit for bit in all three modes, whatever its
    summation order."""
    log(f"integer bit-exact M={M} N={N} K={K} R={R}")
    xc = wl.integer_inputs("ar", M, N, K, R, seed=7)
    x = to_dev(xc)
    A, B, peers = npb(xc["A"]), npb(xc["B"]), npb(xc["peers"])
    out = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=0)
    torch.cuda.synchronize()
    assert_bits_equal(npb(out), orc.gemm_ar(A, B, peers, R), "integer AR")
    for rank in range(R):
        o, ws = run_rs(x, R, rank, M, N)
        torch.cuda.synchronize()
        check_rs_full(orc, xc, o, ws, R, rank, M, N, exact=True)
    Ms = M // 4 + 1
    xa = wl.integer_inputs("ag", Ms, N, K, R, rank=R - 1, seed=8)
    xad = to_dev(xa)
    out, status = run_ag(xad, R, R - 1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    sh = npb(xa["shards"])
    assert_bits_equal(npb(out), orc.ag_gemm(sh[R - 1].copy(), npb(xa["B"]), sh, R, R - 1),
                      "integer AG")


@pytest.mark.parametrize("M", [1, 7, 127, 128, 129, 255, 256, 257])
@pytest.mark.parametrize("N,K", [(8, 8), (264, 72), (136, 0)])
def test_edge_shapes(orc, M, N, K):
    """Tiny and boundary M, single-vector N, K = 0 (output = peer sum only)."""
    R = 8
    xc = wl.integer_inputs("ar", M, N, K, R, seed=M * 3 + K, peer_range=16)
    x = to_dev(xc)
    A, B, peers = npb(xc["A"]), npb(xc["B"]), npb(xc["peers"])
    out = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=3)
    torch.cuda.synchronize()
    assert_bits_equal(npb(out), orc.gemm_ar(A, B, peers, R), f"edge AR M={M} N={N} K={K}")
    for rank in (0, 5, 7):
        o, ws = run_rs(x, R, rank, M, N)
        torch.cuda.synchronize()
        check_rs_full(orc, xc, o, ws, R, rank, M, N, exact=True)


def test_lifetime_two_calls(orc):
    """The pages' lifetime check (M=257, K=768, seed 2500): a second call
    with -x must not disturb the first result (outputs are caller-owned)."""
    M, K, N, R = 257, 768, 512, 8
    g = torch.Generator().manual_seed(2500)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16)
    B = (torch.randn(K, N, generator=g) / np.sqrt(K)).to(torch.bfloat16)
    peers = torch.randn(R - 1, M, N, generator=g).to(torch.bfloat16)
    Ad, Bd, Pd = A.to(DEV), B.to(DEV), peers.to(DEV)
    first = gc.gemm_ar(Ad, Bd, Pd, R=R, rank=0)
    snap = first.clone()
    second = gc.gemm_ar((-Ad).contiguous(), Bd, Pd, R=R, rank=0)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), snap.view(torch.int16))
    assert_close(npb(first), orc.gemm_ar(npb(A), npb(B), npb(peers), R), "lifetime first")
    assert_close(npb(second), orc.gemm_ar(npb(-A), npb(B), npb(peers), R), "lifetime second")


def test_side_stream(orc):
    """Work goes on the stream the caller passes."""
    M, N, K, R = 256, 512, 256, 4
    xc = wl.integer_inputs("ar", M, N, K, R, seed=11)
    x = to_dev(xc)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=1, stream=s)
    s.synchronize()
    assert_bits_equal(npb(out), orc.gemm_ar(npb(xc["A"]), npb(xc["B"]), npb(xc["peers"]), R),
                      "side stream AR")


def test_default_stream_is_torch_current():
    """stream=None launches on torch's current stream, also inside a
    `with torch.cuda.stream(s)` block."""
    assert gc._stream(None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert gc._stream(None) == s.cuda_stream
    assert gc._stream(s) == s.cuda_stream


# ---------------------------------------------------------------------------
def test_invariants_between_modes():
    """RS rows == AR rows; AG == AR on the concatenated shards with zero
    peers; zero rows appended change no valid row (all bit-exact: same
    kernel arithmetic)."""
    M, N, K, R = 333, 392, 320, 4
    w = wl.Workload("inv", "ar", M, N, K, R, 0, 1.0, 1 / np.sqrt(K), seed=5)
    x = to_dev(wl.make_inputs(w))
    ar = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=0)
    P = (M + R - 1) // R
    for rank in range(R):
        out, _ = run_rs(x, R, rank, M, N)
        lo, hi = min(rank * P, M), min(rank * P + P, M)
        torch.cuda.synchronize()
        assert_bits_equal(npb(out[:hi - lo]), npb(ar[lo:hi]), f"RS == AR rows, rank {rank}")
    extra = 77
    A2 = torch.cat([x["A"], torch.zeros(extra, K, dtype=torch.bfloat16, device=DEV)])
    P2 = torch.cat([x["peers"], torch.zeros(R - 1, extra, N, dtype=torch.bfloat16, device=DEV)], 1)
    ar2 = gc.gemm_ar(A2, x["B"], P2.contiguous(), R=R, rank=0)
    torch.cuda.synchronize()
    assert_bits_equal(npb(ar2[:M]), npb(ar), "padding independence")
    assert bool((ar2[M:].float() == 0).all())
    # AG vs AR, both in whole tiles: where a tile is split along K depends on
    # the peer count (AR's peer items must fit in the K loop), and a split
    # changes the fp32 summation order
    Ms = 111
    g = torch.Generator().manual_seed(9)
    shards = torch.randn(R, Ms, K, generator=g).to(torch.bfloat16).to(DEV)
    cat = shards.reshape(R * Ms, K)
    zero_p = torch.zeros(R - 1, R * Ms, N, dtype=torch.bfloat16, device=DEV)
    ref = gc.gemm_ar(cat, x["B"], zero_p, R=R, rank=0, workspace=False)
    for rank in range(R):
        out, status = run_ag({"A": shards[rank].contiguous(), "B": x["B"], "shards": shards},
                             R, rank, workspace=False)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert_bits_equal(npb(out), npb(ref), f"AG == AR(cat), rank {rank}")


# ---------------------------------------------------------------------------
def test_ag_flags_withheld_times_out(orc):
    """A shard whose flag never reaches the epoch is skipped after max_spins
    polls; status names it; every other shard is still correct."""
    Ms, N, K, R, rank = 96, 264, 128, 8, 3
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=21)
    x = to_dev(xc)
    epoch = 5
    missing = 6
    flags = torch.full((R,), epoch, dtype=torch.int32, device=DEV)
    flags[missing] = epoch - 1
    out = filled((R * Ms, N))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, out, R=R, rank=rank, epoch=epoch,
               max_spins=200)
    torch.cuda.synchronize()
    assert int(status.item()) == gc.GC_TIMEOUT_BASE + missing
    sh = npb(xc["shards"])
    ref = orc.ag_gemm(sh[rank].copy(), npb(xc["B"]), sh, R, rank)
    got = npb(out)
    rows = np.arange(R * Ms) // Ms
    assert np.all(got[rows == missing] == SENTINEL), "skipped shard rows must be untouched"
    assert_bits_equal(got[rows != missing], ref[rows != missing], "AG other shards")


def test_ag_epochs_and_fresh_data(orc):
    """Flags are never reset: a later call with epoch+1 and new shard
    content must see the new content.  The new shards and the raised flags
    arrive through the DMA engines (ag_push_shards), not through kernels,
    so a cached copy of the first call's shards would show."""
    Ms, N, K, R, rank = 64, 136, 64, 4, 1
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=31)
    x = to_dev(xc)
    flags = torch.full((R,), 1, dtype=torch.int32, device=DEV)
    out1, st1 = run_ag(x, R, rank, epoch=1, flags=flags)
    torch.cuda.synchronize()
    assert int(st1.item()) == 0
    new_shards = (-xc["shards"]).contiguous()
    src = new_shards.to(DEV)
    ew = torch.full((1,), 2, dtype=torch.int32, device=DEV)
    gc.ag_push_shards(src, x["shards"], flags, ew, R=R, rank=rank)
    x["A"].copy_(new_shards[rank].to(DEV))
    out2, st2 = run_ag(x, R, rank, epoch=2, flags=flags)
    torch.cuda.synchronize()
    assert int(st2.item()) == 0
    sh = npb(new_shards)
    assert_bits_equal(npb(out2), orc.ag_gemm(sh[rank].copy(), npb(xc["B"]), sh, R, rank),
                      "AG after epoch bump")
    # epoch wrap-around: flag 0x00000001 is 'after' epoch 0xFFFFFFFF
    flags.fill_(1)
    out3, st3 = run_ag(x, R, rank, epoch=0xFFFFFFFF, flags=flags)
    torch.cuda.synchronize()
    assert int(st3.item()) == 0


def test_ag_flag_set_late_by_host(orc):
    """The kernel starts with one shard not ready; the host writes that
    shard's flag (in pinned host memory the kernel polls) while the kernel
    runs; the result must be complete and correct."""
    import time
    Ms, N, K, R, rank = 128, 264, 256, 8, 2
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=41)
    x = to_dev(xc)
    late = 5
    flags = torch.full((R,), 3, dtype=torch.int32).pin_memory()
    flags[late] = 0
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    out = gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, R=R, rank=rank, epoch=3,
                     max_spins=1 << 20)
    time.sleep(0.02)
    flags[late] = 3           # plain host store into the pinned page
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "late flag was not seen before the time-out"
    sh = npb(xc["shards"])
    assert_bits_equal(npb(out), orc.ag_gemm(sh[rank].copy(), npb(xc["B"]), sh, R, rank),
                      "AG with a late flag")


@pytest.mark.parametrize("Ms,N,K,R", [(40, 264, 128, 16), (300, 520, 512, 16)])
def test_ag_sixteen_ranks_integer_all_ranks(orc, Ms, N, K, R):
    """AG-GEMM with the largest rank count: every rank's ring order, integer
    inputs, bit-exact against the oracle."""
    log(f"AG R=16 Ms={Ms} N={N} K={K}")
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=0, seed=Ms + K)
    x = to_dev(xc)
    sh = npb(xc["shards"])
    ref = orc.ag_gemm(sh[0].copy(), npb(xc["B"]), sh, R, 0)
    for rank in range(R):
        xr = dict(x, A=x["shards"][rank].contiguous())
        out, status = run_ag(xr, R, rank)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert_bits_equal(npb(out), ref, f"AG R=16 rank {rank}")


@pytest.mark.parametrize("shards_null", [False, True])
def test_ag_k0_gives_zeros(shards_null):
    """AG-GEMM with K = 0: the output is all zeros, with the shards empty or
    passed as a NULL pointer (they hold no element); the flags are still
    waited on.  (A K = 0 call used to be refused when the empty shards
    tensor had no storage.)"""
    Ms, N, R, rank = 64, 56, 16, 13
    shards = torch.empty((R, Ms, 0), dtype=torch.bfloat16, device=DEV)
    A = torch.empty((Ms, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, N), dtype=torch.bfloat16, device=DEV)
    flags = torch.ones(R, dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.full((R * Ms, N), 7.0, dtype=torch.bfloat16, device=DEV)
    if shards_null:
        peers = gc.GcPeers()
        peers.shards = None
        peers.flags = flags.data_ptr()
        peers.status = status.data_ptr()
        peers.epoch = 1
        rc = gc.lib().ag_gemm(A.data_ptr(), B.data_ptr(), Ms, N, 0, R, rank, ctypes.byref(peers),
                              out.data_ptr(), None)
        assert rc == gc.GC_OK, gc.strerror(rc)
    else:
        gc.ag_gemm(A, B, shards, flags, status, out, R=R, rank=rank, epoch=1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert bool((out.float() == 0).all()), "K = 0 must give zeros on every row"


def test_ag_two_shards_withheld():
    """Two shards never become ready: status names one of them (their tiles
    are polled by different workgroups at the same time, and the first to
    time out records its shard), both are left unwritten, the rest is
    exact."""
    Ms, N, K, R, rank = 64, 264, 128, 8, 3
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=22)
    x = to_dev(xc)
    epoch = 9
    flags = torch.full((R,), epoch, dtype=torch.int32, device=DEV)
    flags[5] = epoch - 1           # ring order from rank 3: 3 2 1 0 7 6 5 4
    flags[6] = epoch - 1
    out = filled((R * Ms, N))
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, out, R=R, rank=rank, epoch=epoch,
               max_spins=2000)
    torch.cuda.synchronize()
    assert int(status.item()) in (gc.GC_TIMEOUT_BASE + 5, gc.GC_TIMEOUT_BASE + 6)
    got = npb(out)
    rows = np.arange(R * Ms) // Ms
    missing = (rows == 5) | (rows == 6)
    assert np.all(got[missing] == SENTINEL)
    sh = npb(xc["shards"])
    ref = load_oracle().ag_gemm(sh[rank].copy(), npb(xc["B"]), sh, R, rank)
    assert_bits_equal(got[~missing], ref[~missing], "AG other shards")


def test_ag_skips_without_waiting_once_timed_out():
    """With a time-out already recorded in *status, a shard that is not
    ready is skipped at its first poll: the launch ends in far less than the
    one-second-plus that max_spins = 2^20 polls would take, and status keeps
    its first value."""
    import time
    Ms, N, K, R, rank = 128, 520, 256, 8, 0
    xc = wl.integer_inputs("ag", Ms, N, K, R, rank=rank, seed=23)
    x = to_dev(xc)
    flags = torch.ones(R, dtype=torch.int32, device=DEV)
    flags[4] = 0
    status = torch.full((1,), gc.GC_TIMEOUT_BASE + 2, dtype=torch.int32, device=DEV)
    out = filled((R * Ms, N))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gc.ag_gemm(x["A"], x["B"], x["shards"], flags, status, out, R=R, rank=rank, epoch=1,
               max_spins=1 << 20)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"  launch with a stalled shard after a recorded time-out: {dt * 1e3:.1f} ms")
    assert int(status.item()) == gc.GC_TIMEOUT_BASE + 2
    assert dt < 0.3, f"the launch waited {dt:.3f} s for a shard after a recorded time-out"
    got = npb(out)
    rows = np.arange(R * Ms) // Ms
    assert np.all(got[rows == 4] == SENTINEL)
    sh = npb(xc["shards"])
    ref = load_oracle().ag_gemm(sh[rank].copy(), npb(xc["B"]), sh, R, rank)
    assert_bits_equal(got[rows != 4], ref[rows != 4], "AG other shards")


def test_default_workspace_per_stream():
    """Calls on two streams get two default workspaces; calls on one stream
    reuse one.  Split launches on both streams at once stay exact."""
    M, N, K, R = 256, 1040, 2048, 4
    xc = wl.integer_inputs("ar", M, N, K, R, seed=24)
    x = to_dev(xc)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    w1 = gc.default_workspace(stream=s1)
    w2 = gc.default_workspace(stream=s2)
    assert w1.data_ptr() != w2.data_ptr()
    assert gc.default_workspace(stream=s1).data_ptr() == w1.data_ptr()
    assert gc.plan("ar", M, N, K, R, cus=torch.cuda.get_device_properties(0).multi_processor_count)["units"] > 0
    ref = gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=0, workspace=False)
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        for s in (s1, s2):
            with torch.cuda.stream(s):
                outs.append(gc.gemm_ar(x["A"], x["B"], x["peers"], R=R, rank=0, stream=s))
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert_bits_equal(npb(o), npb(ref), f"split launch {i} on two streams")
