"""Pins of the CPU oracle: checks against facts fixed outside the oracle.

Each ``pin_*`` function takes a loaded oracle build and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix.  The
test suite runs them on the real oracle (all must pass) and on builds with one
planted mistake each (at least one pin must fail for every plant), which shows
that the pins would catch that mistake.

What pins what:
  pin_rounding        IEEE round-to-nearest-even values worked out by hand,
                      and torch's float32 -> bf16 conversion (library routine)
  pin_brute_force     exact rational sums (fractions.Fraction) on tiny shapes:
                      with the fp64 accumulator every output is the nearest
                      bf16, ties to even; with the fp32 one it is the nearest
                      bf16 of a value within the binary32 summation bound
                      gamma_(n-1) * sum|terms| of the exact sum
  pin_fp32_order      hand-worked binary32 sums where one rounding of the
                      accumulator decides the bf16 result: the fp32 oracle
                      must add k ascending, then the peers, in binary32 (and
                      the fp64 one must give the exact answer)
  pin_integer_exact   small-integer inputs: the oracle equals exact integer
                      arithmetic (numpy int64 matmul) bit for bit
  pin_closed_forms    B = I gives A back; A = 0 gives the lone peer back;
                      zero peers match numpy's float64 matmul within 1 ulp
  pin_rs_golden       slice bounds against tests/golden/rs_slices.txt
  pin_pages_reference a literal re-enactment of the pages' test reference
                      (zero-pad to ceil(M/R)*R rows, sum every rank's bf16
                      partial, all_reduce / reduce_scatter chunking)
  pin_invariants      RS equals the matching rows of AR; ws holds bf16(A.B) on
                      the non-owned rows and is untouched on the owned rows;
                      AG equals AR on the concatenated shards with no peers;
                      appending zero rows changes no valid row
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction

import numpy as np
import torch

from workloads import bits, from_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def decode(h: int) -> float:
    """Value of one raw bf16 bit pattern (bf16 = upper half of a binary32)."""
    return struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))[0]


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_bf16(rng, shape, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))
    return bits(x.to(torch.bfloat16))


def _int_bf16(rng, shape, lim):
    return bits(torch.from_numpy(rng.integers(-lim, lim + 1, shape).astype(np.float32)).to(torch.bfloat16))


# ---------------------------------------------------------------------------
def pin_rounding(orc):
    # Hand-derived from the binary format: 8 significant bits, spacing 2^-7 in
    # [1, 2); ties go to the even last bit.
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),               # tie between 1 and 1+2^-7 -> even (1)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),           # tie between 1+2^-7 and 1+2^-6 -> even
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                   # smallest subnormal
        (2.0 ** -134, 0x0000),                   # tie between 0 and 2^-133 -> even (0)
        (3 * 2.0 ** -134, 0x0002),               # tie between 1 and 2 ulps -> even (2)
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie above the largest -> even (inf)
        (1e39, 0x7F80),
        (255.0, 0x437F),
        (257.0, 0x4380),                         # tie 256/258 -> 256
        (259.0, 0x4382),                         # tie 258/260 -> 260 (0x4382)
    ]
    for x, want in cases:
        got = orc.round_bf16(x)
        assert got == want, f"round_bf16({x!r}) = {got:#06x}, want {want:#06x}"
    # Library routine: torch rounds float32 -> bf16 to nearest even; every
    # float32 value is exactly a double, so the two must agree bit for bit.
    rng = _rng(1)
    xs = np.concatenate([rng.standard_normal(2000).astype(np.float32) * np.float32(s)
                         for s in (1e-3, 1.0, 7.0, 1e4)])
    # include exact ties: bf16 value + half a bf16 ulp
    ties = (np.arange(1, 400, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    xs = np.concatenate([xs, ties, -ties])
    ref = bits(torch.from_numpy(xs).to(torch.bfloat16))
    got = np.array([orc.round_bf16(float(v)) for v in xs], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs torch, first x={xs[bad[0]]!r}"


def _nearest_check(exact: Fraction, h: int):
    """h must be a nearest bf16 to `exact`, ties to even."""
    v = Fraction(decode(h))
    d = abs(exact - v)
    for nb in ((h + 1) & 0xFFFF, (h - 1) & 0xFFFF, h ^ 0x8000 if (h & 0x7FFF) == 0 else h):
        if (nb & 0x7F80) == 0x7F80:
            continue
        dn = abs(exact - Fraction(decode(nb)))
        assert d <= dn, f"{h:#06x} is not nearest to {float(exact)!r} (neighbour {nb:#06x})"
        if d == dn and nb != h:
            assert (h & 1) == 0, f"tie at {float(exact)!r} not resolved to even"


def _within_check(terms: list, h: int):
    """h must be the nearest bf16 of some y with |y - S| <= gamma_(n-1) *
    sum|terms|, S the exact sum of the n terms: the binary32 bound of a
    recursive sum (each addition rounded to nearest, unit roundoff 2^-24),
    whatever its order."""
    exact = sum(terms, Fraction(0))
    n = len(terms)
    u = Fraction(1, 2 ** 24)
    gamma = (n - 1) * u / (1 - (n - 1) * u) if n > 1 else Fraction(0)
    err = gamma * sum(abs(t) for t in terms)
    v = Fraction(decode(h))
    # rounding interval of h: half-way to each finite neighbour
    up = Fraction(decode((h + 1) & 0xFFFF)) if (h & 0x7FFF) < 0x7F7F else v
    dn = Fraction(decode((h - 1) & 0xFFFF)) if (h & 0x7FFF) != 0 else -Fraction(decode(0x0001))
    if h & 0x8000:
        up, dn = dn, up
    lo_r, hi_r = (v + min(up, dn)) / 2, (v + max(up, dn)) / 2
    assert max(lo_r, exact - err) <= min(hi_r, exact + err), (
        f"{h:#06x} is not the bf16 of any value within {float(err)!r} of {float(exact)!r}")


def pin_brute_force(orc):
    check = ((lambda terms, h: _nearest_check(sum(terms, Fraction(0)), h)) if orc.acc == "fp64"
             else _within_check)
    rng = _rng(2)
    for (M, N, K, R) in [(3, 5, 7, 2), (4, 6, 16, 4), (2, 3, 33, 3), (5, 4, 1, 2), (2, 3, 200, 8)]:
        A = _rand_bf16(rng, (M, K), 1.0)
        B = _rand_bf16(rng, (K, N), 1.0 / np.sqrt(K))
        peers = _rand_bf16(rng, (R - 1, M, N), 1.0)
        out = orc.gemm_ar(A, B, peers, R)
        for i in range(M):
            for j in range(N):
                terms = [Fraction(decode(A[i, k])) * Fraction(decode(B[k, j])) for k in range(K)]
                terms += [Fraction(decode(peers[p, i, j])) for p in range(R - 1)]
                check(terms, int(out[i, j]))
    # K = N square case with structure that a transposed read would break
    A = _rand_bf16(rng, (3, 8), 1.0)
    B = _rand_bf16(rng, (8, 8), 1.0)
    out = orc.gemm_ar(A, B, np.zeros((1, 3, 8), np.uint16), 2)
    for i in range(3):
        for j in range(8):
            check([Fraction(decode(A[i, k])) * Fraction(decode(B[k, j])) for k in range(8)] +
                  [Fraction(0)], int(out[i, j]))


def pin_fp32_order(orc):
    """Sums whose bf16 result depends on one binary32 rounding, worked out
    by hand (IEEE 754 binary32: 24-bit significand, ties to even).

    (a) 1.0625 * 1.0625 + 2^-15 * 2^-15 = (1 + 2^-3 + 2^-8) + 2^-30.  In
        binary32 the second term is below half an ulp of the first (2^-24)
        and is lost, leaving the exact bf16 tie 1.125 + 2^-8, which goes to
        the even 1.125 (0x3F90).  The exact sum lies above the tie: 1.1328125
        (0x3F91).
    (b) k ascending over 2^12*2^12, 1*1, -2^12*2^12: 2^24 + 1 is a binary32
        tie that goes to the even 2^24, then - 2^24 leaves 0 (0x0000).  The
        exact sum, or k descending, gives 1 (0x3F80).
    (c) the GEMM part 2^12*2^12 = 2^24, then peers 1 and -2^24: the same tie
        leaves 0.  Peers first give -(2^24 - 1) + 2^24 = 1, the exact sum.
    """
    f32 = orc.acc == "fp32"
    to = lambda xs: bits(torch.tensor(xs, dtype=torch.float64).to(torch.bfloat16))
    A = to([[1.0625, 2.0 ** -15]])
    B = to([[1.0625], [2.0 ** -15]])
    got = int(orc.gemm_ar(A, B, np.zeros((1, 1, 1), np.uint16), 2)[0, 0])
    want = 0x3F90 if f32 else 0x3F91
    assert got == want, f"(a) lost low-order term: got {got:#06x}, want {want:#06x} ({orc.acc})"
    A = to([[2.0 ** 12, 1.0, -2.0 ** 12]])
    B = to([[2.0 ** 12], [1.0], [2.0 ** 12]])
    got = int(orc.gemm_ar(A, B, np.zeros((1, 1, 1), np.uint16), 2)[0, 0])
    want = 0x0000 if f32 else 0x3F80
    assert got == want, f"(b) k order: got {got:#06x}, want {want:#06x} ({orc.acc})"
    A = to([[2.0 ** 12]])
    B = to([[2.0 ** 12]])
    peers = to([[[1.0]], [[-2.0 ** 24]]])
    got = int(orc.gemm_ar(A, B, peers, 3)[0, 0])
    want = 0x0000 if f32 else 0x3F80
    assert got == want, f"(c) peers after the GEMM part: got {got:#06x}, want {want:#06x} ({orc.acc})"
    # the same through RS (rank 0 owns the single row) and AG (no peers: (a), (b))
    o, _ = orc.gemm_rs(A, B, peers, 3, 0)
    assert o.shape == (1, 1) and int(o[0, 0]) == want, f"(c) through RS ({orc.acc})"


def pin_integer_exact(orc):
    rng = _rng(3)
    for (M, N, K, R) in [(7, 9, 16, 8), (16, 24, 12, 4), (33, 8, 16, 2), (1, 1, 1, 2)]:
        A = rng.integers(-2, 3, (M, K))
        B = rng.integers(-2, 3, (K, N))
        P = rng.integers(-16, 17, (R - 1, M, N))
        exact = A @ B + P.sum(0)              # |exact| <= 64 + 112 < 256: exact in bf16
        assert np.abs(exact).max() < 256
        to = lambda x: bits(torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16))
        out = orc.gemm_ar(to(A), to(B), to(P), R)
        want = to(exact)
        assert np.array_equal(out, want), "integer GEMM-AR is not exact"
        for r in range(R):
            o, _ = orc.gemm_rs(to(A), to(B), to(P), R, r)
            Pm = -(-M // R)
            padded = np.zeros((Pm * R, N), np.int64)
            padded[:M] = exact
            assert np.array_equal(o, to(padded[r * Pm:(r + 1) * Pm])), f"integer RS rank {r}"
        # AG: shards of M rows, concatenated
        shards = rng.integers(-2, 3, (R, M, K))
        for r in (0, R - 1):
            o = orc.ag_gemm(to(shards[r]), to(B), to(shards), R, r)
            assert np.array_equal(o, to(shards.reshape(R * M, K) @ B)), f"integer AG rank {r}"


def pin_closed_forms(orc):
    rng = _rng(4)
    # B = I (K = N), no peer contribution: out == A bit for bit
    M, N = 6, 16
    A = _rand_bf16(rng, (M, N), 3.0)
    I = bits(torch.eye(N, dtype=torch.bfloat16))
    zero_peers = np.zeros((3, M, N), np.uint16)
    assert np.array_equal(orc.gemm_ar(A, I, zero_peers, 4), A), "A.I + 0 != A"
    # A = 0, one peer: out == the peer bit for bit
    K = 12
    Z = np.zeros((M, K), np.uint16)
    B = _rand_bf16(rng, (K, N))
    peer = _rand_bf16(rng, (1, M, N), 5.0)
    assert np.array_equal(orc.gemm_ar(Z, B, peer, 2), peer[0]), "0.B + peer != peer"
    # zero peers: numpy float64 matmul (a library routine), rounded by torch
    M, N, K = 9, 20, 300
    A = _rand_bf16(rng, (M, K))
    B = _rand_bf16(rng, (K, N), 1 / np.sqrt(K))
    f = lambda h: from_bits(h).to(torch.float64).numpy()
    ref = f(A) @ f(B)
    out = orc.gemm_ar(A, B, np.zeros((1, M, N), np.uint16), 2)
    got = f(out)
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got - ref) <= ulp), "zero-peer GEMM-AR differs from numpy matmul by > 1 ulp"


def pin_rs_golden(orc):
    with open(os.path.join(GOLDEN, "rs_slices.txt")) as fh:
        rows = [l.split() for l in fh if l.strip() and not l.startswith("#")]
    assert rows
    for M, R, r, P, lo, hi in (map(int, x) for x in rows):
        got = orc.rs_slice(M, R, r)
        assert got == (P, lo, hi), f"rs_slice({M},{R},{r}) = {got}, want {(P, lo, hi)}"


def pin_pages_reference(orc):
    """Re-enact the pages' test reference: torch.mm into a zero-padded
    [ceil(M/R)*R, N] bf16 partial per rank, then all_reduce (AR, rows [:M])
    or reduce_scatter_single (RS, chunk r).  Each rank's partial is bf16;
    here the other ranks' partials are the peer buffers.  The pages round the
    local partial to bf16 before the sum and the oracle does not, so values
    agree within the stated tolerance, and padding rows exactly."""
    rng = _rng(5)
    for (M, N, K, R) in [(13, 24, 40, 4), (8, 16, 64, 8), (5, 8, 16, 8), (130, 32, 96, 2)]:
        A = _rand_bf16(rng, (M, K))
        B = _rand_bf16(rng, (K, N), 1 / np.sqrt(K))
        peers = _rand_bf16(rng, (R - 1, M, N))
        tA, tB = from_bits(A), from_bits(B)
        padded_M = (M + R - 1) // R * R
        for r in range(R):
            partials = []
            others = iter(range(R - 1))
            for rank in range(R):
                part = torch.zeros((padded_M, N), dtype=torch.bfloat16)
                if rank == r:
                    torch.mm(tA, tB, out=part[:M])   # bf16 partial, as the pages' reference
                else:
                    part[:M] = from_bits(peers[next(others)])
                partials.append(part.double())
            total = sum(partials)
            ar_ref = total[:M]
            rs_ref = total.reshape(R, padded_M // R, N)[r]
            f = lambda h: from_bits(h).to(torch.float64)
            ar = f(orc.gemm_ar(A, B, peers, R))
            assert torch.all((ar - ar_ref).abs() <= 1e-2 * ar_ref.abs() + 1e-2), "AR vs pages' reference"
            rs, _ = orc.gemm_rs(A, B, peers, R, r)
            rs = f(rs)
            assert rs.shape == rs_ref.shape, "RS slice height"
            assert torch.all((rs - rs_ref).abs() <= 1e-2 * rs_ref.abs() + 1e-2), f"RS vs pages' reference r={r}"
            valid = max(0, min(M - r * (padded_M // R), padded_M // R))
            assert torch.all(rs[valid:] == 0), "padding rows must be zero"


def pin_invariants(orc):
    rng = _rng(6)
    M, N, K, R = 37, 24, 48, 4
    A = _rand_bf16(rng, (M, K))
    B = _rand_bf16(rng, (K, N), 1 / np.sqrt(K))
    peers = _rand_bf16(rng, (R - 1, M, N))
    ar = orc.gemm_ar(A, B, peers, R)
    gemm_only = orc.gemm_ar(A, B, np.zeros((R - 1, M, N), np.uint16), R)
    sentinel = np.uint16(0x7FC1)
    for r in range(R):
        P, lo, hi = orc.rs_slice(M, R, r)
        ws = np.full((M, N), sentinel, np.uint16)
        out, ws = orc.gemm_rs(A, B, peers, R, r, ws)
        assert out.shape == (P, N)
        assert np.array_equal(out[:hi - lo], ar[lo:hi]), "RS rows != AR rows"
        assert np.all(out[hi - lo:] == 0)
        assert np.all(ws[lo:hi] == sentinel), "owned ws rows must stay untouched"
        own = np.zeros(M, bool)
        own[lo:hi] = True
        assert np.array_equal(ws[~own], gemm_only[~own]), "ws != bf16(A.B) on non-owned rows"
    # padding independence: zero rows appended to A and to every peer
    extra = 11
    A2 = np.concatenate([A, np.zeros((extra, K), np.uint16)])
    P2 = np.concatenate([peers, np.zeros((R - 1, extra, N), np.uint16)], axis=1)
    ar2 = orc.gemm_ar(A2, B, P2, R)
    assert np.array_equal(ar2[:M], ar) and np.all(ar2[M:] == 0), "padding changed valid rows"
    # AG == AR on the concatenated shards with zero peers
    Ms = 9
    shards = _rand_bf16(rng, (R, Ms, K))
    cat = shards.reshape(R * Ms, K)
    ref = orc.gemm_ar(cat, B, np.zeros((R - 1, R * Ms, N), np.uint16), R)
    for r in range(R):
        assert np.array_equal(orc.ag_gemm(shards[r].copy(), B, shards, R, r), ref), f"AG rank {r}"
    # AG source rows
    for g in (0, Ms - 1, Ms, R * Ms - 1):
        q, t = orc.ag_source(Ms, R, g)
        assert q * Ms + t == g and 0 <= t < Ms


ALL_PINS = [pin_rounding, pin_brute_force, pin_fp32_order, pin_integer_exact, pin_closed_forms,
            pin_rs_golden, pin_pages_reference, pin_invariants]
