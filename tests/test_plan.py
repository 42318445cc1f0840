"""The launch planner (gemm_coll_plan: tile height, tile count, split along
K), checked on the CPU: the choices for the named workloads, and, over many
shapes, compute-unit counts and options, the invariants the kernel relies on
-- every tile exactly once, at most one workgroup per split unit and no more
units than compute units (each unit owns one workspace slot), at most 16
chunks per tile (16 claim words), chunks a multiple of 8 K-steps, and every
chunk long enough for the 8 K-steps of each peer partial it adds."""
import itertools
import random

import pytest

import tensor_bf16_gemm_amd as gc
import workloads as wl


def cdiv(a, b):
    return -(-a // b)


def m_rows_of(mode, M, R, rank):
    if mode == "rs":
        P = cdiv(M, R)
        return max((rank + 1) * P, M)
    return M


def check_plan(mode, M, N, K, R, rank, cus, ws, rows):
    p = gc.plan(mode, M, N, K, R, rank, cus=cus, workspace=ws, tile_rows=rows)
    if M == 0 or N == 0:
        assert p["tiles"] == 0
        return p
    bm = p["tile_rows"]
    assert bm in (64, 128, 224, 256)
    if rows:
        assert bm == rows
    shards = R if mode == "ag" else 1
    tiles = cdiv(m_rows_of(mode, M, R, rank), bm) * cdiv(N, 256) * shards
    assert p["tiles"] == tiles
    assert p["whole_tiles"] + p["split_tiles"] == tiles
    assert p["peer_nt"] in (0, 1) and (not p["peer_nt"] or bm >= 224)
    kt = cdiv(K, 32)
    if p["units"] == 0:
        assert p["split_tiles"] == 0 and p["chunks"] == 0 and p["chunk_steps"] == 0
        assert p["grid"] == min(tiles, cus)
        return p
    # split: the last partial round only, after full rounds of whole tiles
    assert ws, "no split without a workspace"
    assert bm != 224
    assert p["whole_tiles"] % cus == 0 and 0 < p["split_tiles"] < cus
    q, ch = p["chunks"], p["chunk_steps"]
    assert 2 <= q <= 16
    assert ch % 8 == 0 and ch < kt
    assert q == cdiv(kt, ch)
    assert p["units"] == q * p["split_tiles"] <= cus
    assert p["grid"] == p["units"]
    npeers = 0 if mode == "ag" else R - 1
    for c in range(q):
        length = min(kt, (c + 1) * ch) - c * ch
        assert length > 0
        peers_c = cdiv((c + 1) * npeers, q) - cdiv(c * npeers, q)
        assert 8 * peers_c <= length, (c, peers_c, length)
    return p


@pytest.mark.parametrize("name,rows,chunks,steps", [
    ("kda4096_ar", 224, 0, 0),      # 475 tiles of 224 rows: two rounds, no split
    ("kda64_ar", 64, 10, 24),       # 25 tiles in 10 chunks of 24 K-steps
    ("kda16_ar", 64, 10, 24),
    ("mla_ar", 128, 7, 32),         # 30 tiles of 128 rows in 7 chunks of 32
    ("mla_rs", 128, 7, 32),
    ("kda512_ar", 256, 4, 56),
    ("kda1024_ar", 256, 2, 112),
    ("tiny_ar", 64, 2, 8),
])
def test_named_workloads(name, rows, chunks, steps):
    w = wl.WORKLOADS[name]
    p = check_plan(w.mode, w.M, w.N, w.K, w.R, w.rank, 256, True, 0)
    assert (p["tile_rows"], p["chunks"], p["chunk_steps"]) == (rows, chunks, steps), p


def test_full_round_then_split_tail():
    """M=8448, N=2048, K=7168: a round of 256 whole tiles, then 8 tiles in 14 chunks."""
    p = check_plan("ar", 8448, 2048, 7168, 8, 0, 256, True, 0)
    assert (p["tile_rows"], p["whole_tiles"], p["split_tiles"], p["chunks"], p["chunk_steps"]) == \
        (256, 256, 8, 14, 16)


def test_no_workspace_no_split():
    for M in (16, 256, 512, 8448):
        p = check_plan("ar", M, 6288, 7168, 8, 0, 256, False, 0)
        assert p["units"] == 0


def test_decode_heights_without_split():
    """Short tiles also win when nothing can be split: less MFMA work per step."""
    assert gc.plan("ar", 16, 6288, 7168, 8, workspace=False)["tile_rows"] == 64
    assert gc.plan("ar", 100, 6288, 7168, 8, workspace=False)["tile_rows"] in (64, 128)


def test_invariants_grid():
    shapes = itertools.product(
        ("ar", "rs", "ag"),
        (1, 16, 64, 65, 100, 128, 129, 256, 300, 513, 1024, 4096, 8448),
        (8, 264, 1040, 3648, 6288),
        (0, 8, 72, 256, 1024, 4096, 7168),
        (2, 4, 8, 16),
    )
    n = 0
    for mode, M, N, K, R in shapes:
        for cus in (256, 80):
            check_plan(mode, M, N, K, R, R - 1, cus, True, 0)
            n += 1
    assert n > 1000


def test_invariants_random():
    rng = random.Random(1234)
    for _ in range(3000):
        mode = rng.choice(("ar", "rs", "ag"))
        R = rng.choice((2, 4, 8, 16))
        M = rng.randint(0, 9000)
        N = 8 * rng.randint(1, 2000)
        K = 8 * rng.randint(0, 2000)
        rank = rng.randrange(R)
        cus = rng.choice((256, 304, 228, 80, 32))
        ws = rng.random() < 0.8
        rows = rng.choice((0, 0, 0, 64, 128, 224, 256))
        out_rows = M * R if mode == "ag" else M
        if max(M * K, K * N, out_rows * N) * 2 >= 1 << 31:
            with pytest.raises(RuntimeError, match="not supported"):
                gc.plan(mode, M, N, K, R, rank, cus=cus, workspace=ws, tile_rows=rows)
            continue
        check_plan(mode, M, N, K, R, rank, cus, ws, rows)


@pytest.mark.parametrize("kw", [
    dict(cus=0), dict(cus=5000), dict(tile_rows=96), dict(R=3), dict(R=1), dict(rank=8),
    dict(N=12), dict(K=20), dict(M=-1),
])
def test_plan_rejects(kw):
    args = dict(mode="ar", M=256, N=256, K=256, R=8, rank=0)
    opts = {k: kw.pop(k) for k in ("cus", "tile_rows") if k in kw}
    args.update(kw)
    with pytest.raises(RuntimeError, match="invalid argument"):
        gc.plan(args.pop("mode"), **args, **opts)


def test_plan_rejects_mode():
    L = gc.lib()
    out = gc.GcPlan()
    import ctypes
    assert L.gemm_coll_plan(3, 256, 256, 256, 8, 0, 256, 1, 0, ctypes.byref(out)) == gc.GC_EINVAL
    assert L.gemm_coll_plan(0, 256, 256, 256, 8, 0, 256, 1, 0, None) == gc.GC_EINVAL


def test_plan_oversized():
    with pytest.raises(RuntimeError, match="not supported"):
        gc.plan("ar", 1 << 20, 256, 1 << 10, 8)
