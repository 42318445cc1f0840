// gemm_coll.hip -- host side of the C ABI declared in include/gemm_coll.h:
// argument validation, tile-configuration choice and the launch on the
// caller's stream.  Device code lives in gc_kernel.hpp.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "gc_kernel.hpp"
#include "gemm_coll.h"
#include "peer_sum.hpp"

static_assert(GC_MODE_AR == gc::MODE_AR && GC_MODE_RS == gc::MODE_RS && GC_MODE_AG == gc::MODE_AG,
              "mode numbers of the C ABI and the kernel");

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];      // 0 = not queried yet
std::atomic<uint32_t> g_epoch[kMaxDevices];    // split-launch counter

int cu_count(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Every buffer is addressed through 32-bit byte offsets with an out-of-range
// sentinel at 2^31, so each one must stay below 2 GiB.
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;

bool fits(int64_t rows, int64_t cols) { return rows * cols * 2 < kMaxBufferBytes; }

int check_common(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R,
                 int rank, const gc_peers *peers, const gc_bf16 *out)
{
    if (M < 0 || N < 0 || K < 0)
        return GC_EINVAL;
    if (!(R > 1 && R <= 16 && 128 % R == 0))
        return GC_EINVAL;
    if (rank < 0 || rank >= R)
        return GC_EINVAL;
    if (N % 8 != 0 || K % 8 != 0)
        return GC_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return GC_ENOTSUP;
    if (M == 0 || N == 0)
        return GC_OK;  // nothing to do; pointers may be NULL
    if (!peers || !out || !aligned16(out))
        return GC_EINVAL;
    switch (peers->tile_rows) {
    case 0: case 64: case 128: case 224: case 256:
        break;
    default:
        return GC_EINVAL;
    }
    // A and B are not read when K == 0 (the output is then the peer sum).
    if (K > 0 && (!A || !B || !aligned16(A) || !aligned16(B)))
        return GC_EINVAL;
    return GC_OK;
}

// Workspace layout for G workgroups (at most G split units, one per
// workgroup, and fewer than G split tiles): an 8-byte arrival counter and 16
// claim words per tile, two flag words per unit, then one fp32 partial tile
// per unit.  Each part starts on a 256-byte boundary.
constexpr int64_t a256(int64_t x) { return (x + 255) / 256 * 256; }
constexpr int64_t count_bytes(int groups) { return a256((int64_t)groups * 8); }
constexpr int64_t claim_bytes(int groups) { return a256((int64_t)groups * 16 * 4); }
constexpr int64_t flag_bytes(int groups) { return a256((int64_t)groups * 8); }
constexpr int64_t workspace_bytes_for(int groups)
{
    return count_bytes(groups) + claim_bytes(groups) + flag_bytes(groups) +
           (int64_t)groups * gc::PART_FLOATS * 4;
}

// The split state of gemm_ar_noalloc: the workspace layout above for up to
// kScratchSlots compute units (256, MI355X's count: 64 MiB + 20 KiB), in
// device memory of the code object itself, one copy per device, zero at
// load and held until the process ends.  Host code never passes `scratch`
// itself to a kernel (in host code the name stands for a host-side shadow,
// not a device address): scratch_address() looks up each device's copy
// once, with that device current, and calls use that address.
constexpr int kScratchSlots = 256;
constexpr int64_t kScratchBytes = workspace_bytes_for(kScratchSlots);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];   // device address, per device

int scratch_address(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return GC_ENOTSUP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return GC_EIO;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return GC_OK;
}

// Chunk size (K-steps, a multiple of 8) for a problem of `tiles` < groups
// tiles, cut into q <= min(16, groups / tiles) chunks so that every unit has
// a workgroup of its own.  Cost model in K-step units, fitted to
// measurements at M=256 and 512, N=3648 and 6288, K=7168 (256-row tiles): a
// unit's K loop takes its chunk, and every unit adds the traffic of handing
// its partial over (about 0.5 MB through memory), worth 1/6 of a step each:
// cost = chunk + units / 6.  Whole tiles cost kt + tiles / 6 on this scale.
// (Measured at M=256, 15 tiles: 10 chunks of 24 steps 46.7 us, 7 of 32
// 50.3 us, 14 of 16 50.5 us, 4 of 56 62.5 us.)  Shorter tiles of `bm` rows
// scale both terms by what they move: a step loads (bm + 256) x 32 bf16, a
// partial is bm x 256 fp32, so the weights become 6 (bm + 256) / 512 per
// step and bm / 256 per unit (15 : 1 at 64 rows, 9 : 1 at 128).  Returns
// `kt` for whole tiles.
int pick_chunk(int kt, int tiles, int groups, int bm)
{
    const int qmax = std::min(16, groups / tiles);
    const int64_t ws = 6 * (int64_t)(bm + 256), wu = 2 * (int64_t)bm;   // both x 512
    int best = kt;
    int64_t best_cost = ws * kt + wu * tiles;
    for (int q = 2; q <= qmax; ++q) {
        const int chunk = ((kt + q - 1) / q + 7) / 8 * 8;
        if (chunk >= kt)
            continue;
        const int64_t units = (int64_t)((kt + chunk - 1) / chunk) * tiles;   // <= q * tiles
        const int64_t cost = ws * chunk + wu * units;
        if (cost < best_cost) {
            best_cost = cost;
            best = chunk;
        }
    }
    return best;
}

// Chunk size for splitting `rest` (< groups) tiles along K, or kt when they
// are better run whole or cannot be split: every unit needs a workgroup of
// its own, and chunk c, which adds the items of peers [ceil(c*np/q),
// ceil((c+1)*np/q)) at its first steps, must have 8 steps per peer.
int split_chunk(int kt, int64_t rest, int groups, int npeers, int bm)
{
    if (kt <= 8 || rest <= 0 || rest >= groups || 8 * npeers > kt)
        return kt;
    const int chunk = pick_chunk(kt, (int)rest, groups, bm);
    if (chunk >= kt)
        return kt;
    const int q = (kt + chunk - 1) / chunk;
    if ((int64_t)q * rest > groups)
        return kt;
    for (int c = 0; c < q; ++c) {
        const int len = std::min(kt, (c + 1) * chunk) - c * chunk;
        const int np = ((c + 1) * npeers + q - 1) / q - (c * npeers + q - 1) / q;
        if (8 * np > len)
            return kt;
    }
    return chunk;
}

// Cost, on pick_chunk's scale (x 512), of running `tiles` tiles of `bm`
// rows: full rounds of whole tiles, then the last partial round split along
// K when split_chunk allows it (chunk < kt), else whole.
int64_t plan_cost(int kt, int64_t tiles, int groups, int npeers, int bm, bool can_split)
{
    const int64_t ws = 6 * (int64_t)(bm + 256), wu = 2 * (int64_t)bm;
    const int64_t rest = tiles % groups;
    int64_t c = tiles / groups * ws * kt;
    if (rest > 0) {
        const int chunk = can_split ? split_chunk(kt, rest, groups, npeers, bm) : kt;
        c += chunk < kt ? ws * chunk + wu * ((kt + chunk - 1) / chunk) * rest : ws * kt + wu * rest;
    }
    return c;
}

// Slice of rank r in GEMM-RS: P = ceil(M/R) rows, global rows [r*P,
// (r+1)*P); the valid ones, [lo, hi), are those below M.  `end` is the last
// slice row + 1, which may pass M (padding rows covered by tiles).
void rs_slice(int64_t M, int R, int rank, int64_t &P, int64_t &lo, int64_t &hi, int64_t &end)
{
    P = (M + R - 1) / R;
    lo = (int64_t)rank * P;
    hi = lo + P;
    end = hi;
    if (lo > M)
        lo = M;
    if (hi > M)
        hi = M;
}

// Launch plan of a call: tile height and count, and the split of the last
// partial round along K.  Host arithmetic only (no device call), so that
// gemm_coll_plan can report it without a GPU.
struct Plan {
    int bm = 256;              // tile rows: 64, 128, 224 or 256
    int tiles_m = 0, tiles_n = 0, num_tiles = 0;
    int dp_tiles = 0;          // whole tiles (all of them when nothing is split)
    int sk_tiles = 0, sk_q = 0, sk_chunk = 0, sk_units = 0;
    int grid = 0;              // workgroups of the last launch
    bool peer_nt = false;
};

// m_rows: rows covered by tiles (per shard for AG); item_peers: peer
// partials the kernel adds (0 for AG); peer_bytes: bytes of peer partials
// the launch reads.
int make_plan(int64_t m_rows, int64_t N, int64_t K, int64_t shards, int item_peers,
              int64_t peer_bytes, int cus, bool ws_ok, uint32_t tile_rows, Plan &pl)
{
    pl = Plan();
    pl.tiles_n = (int)((N + gc::BN - 1) / gc::BN);
    auto tiles_for = [&](int64_t bm) { return (m_rows + bm - 1) / bm * pl.tiles_n * shards; };
    const int kt = (int)((K + gc::BK - 1) / gc::BK);
    // Tile height.  With fewer 256-row tiles than CUs, the cheapest by
    // plan_cost of 256 rows and of the shorter heights, 128 and 64 rows (4 or
    // 2 row blocks per wave), whose tiles still fit in one round: shorter
    // tiles waste less MFMA work and hand-over traffic on rows past M and
    // give more tiles to split, but a second round costs about as much as
    // the first (the cost model would price a round of 64-row tiles at 5/8
    // of a round of 256-row tiles; at M=512, N=1040, K=896, AG over 8
    // shards, 64-row tiles in a round and a split tail took 35.8 us, 128-row
    // tiles in one round 19.4).  Measured at N=6288, K=7168, R=8: M=16 and
    // 64 take 64 rows (32 us against 49 and 51 with 256); MLA M=256, N=3648
    // takes 128 rows (40 us against 45; 64 rows 41); M=512 keeps 256 (128
    // rows 78 us against 68).
    // With a full round of 256-row tiles or more: 64 or 128 rows for at most
    // 64 or 128 rows per shard, else 256 rows, or 224 where that is cheaper
    // by 3 % or more, counted in rounds of 256-row tiles.  224-row tiles
    // cost 7/8 of a round per round.  With 256-row tiles, a last partial
    // round can be split along K (see below): about (chunk + 20 steps of
    // hand-over) / kt of a round, else one more round.  At M=4096, N=6288 on
    // 256 CUs, 475 tiles of 224 rows fill two rounds where 400 of 256 rows
    // (144 left over, too many to split) also took two: 224.  At M=8448,
    // N=2048, K=7168, 264 tiles of 256 rows are a round plus 8 tiles split
    // 14 ways: 256 rows, measured 248 us against 333 us with 224.
    const int64_t t256 = tiles_for(256), t224 = tiles_for(224);
    int bm = 256;
    if (tile_rows != 0) {
        bm = (int)tile_rows;
    } else if (t256 < cus) {
        int64_t best = plan_cost(kt, t256, cus, item_peers, 256, ws_ok);
        for (int h : {128, 64}) {
            if (tiles_for(h) > cus)
                continue;
            const int64_t c = plan_cost(kt, tiles_for(h), cus, item_peers, h, ws_ok);
            if (c < best) {
                best = c;
                bm = h;
            }
        }
    } else if (m_rows <= 128) {
        bm = m_rows <= 64 ? 64 : 128;
    } else {
        const int64_t r256 = t256 % cus;
        const int ch = ws_ok ? split_chunk(kt, r256, cus, item_peers, 256) : kt;
        const double c256 = (double)(t256 / cus) +
                            (r256 == 0 ? 0.0 : ch < kt ? (ch + 20.0) / kt : 1.0);
        const double c224 = (double)((t224 + cus - 1) / cus) * (224.0 / 256.0);
        if (c224 < 0.97 * c256)
            bm = 224;
    }
    const int64_t total = tiles_for(bm);
    if (total > INT32_MAX)
        return GC_ENOTSUP;
    pl.bm = bm;
    pl.tiles_m = (int)((m_rows + bm - 1) / bm);
    pl.num_tiles = (int)total;
    pl.dp_tiles = pl.num_tiles;
    pl.grid = pl.num_tiles < cus ? pl.num_tiles : cus;
    // Peer partials are read once.  When they are far larger than the
    // last-level cache, their loads are marked non-temporal so that they do
    // not evict the A and B tiles (measured at M=4096, 360 MB of peers: 3 %
    // faster; on peer sets that the cache can hold, as in repeated calls on
    // the same buffers, the plain loads are faster).  Tiles of 128 rows or
    // fewer always load them plainly (no instance of their own).
    pl.peer_nt = bm >= 224 && peer_bytes > ((int64_t)128 << 20);
    // The tiles of the last partial round (all of them when there are fewer
    // tiles than workgroups) may be split along K, when the cost model says
    // that pays: then the full rounds run first as whole tiles, in a launch
    // of their own, and the split launch takes the rest.  (At M=4096, 400
    // tiles on 256 CUs, the 144 left over cannot take two chunks each, and
    // splitting them into more units than CUs was measured slower.)
    const int rest = pl.num_tiles % cus;
    if (bm != 224 && ws_ok && rest > 0) {
        const int chunk = split_chunk(kt, rest, cus, item_peers, bm);
        if (chunk < kt) {
            pl.dp_tiles = pl.num_tiles - rest;
            pl.sk_tiles = rest;
            pl.sk_chunk = chunk;
            pl.sk_q = (kt + chunk - 1) / chunk;
            pl.sk_units = pl.sk_q * rest;
            pl.grid = pl.sk_units;
        }
    }
    return GC_OK;
}

template <int MODE>
int dispatch(gc::Args &a, const gc_peers *peers, hipStream_t stream)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return GC_EIO;
    // One 512-thread workgroup per CU (the kernel holds up to 160 KiB of
    // LDS); a persistent workgroup walks its list of tiles and segments.
    const int cus = cu_count(dev);
    // (A workspace of `cus` slots is addressed with 32-bit offsets: at most
    // 4096 slots of 256 KiB.)
    const bool ws_ok = peers->workspace != nullptr && cus <= 4096 &&
                       peers->workspace_bytes >= (uint64_t)workspace_bytes_for(cus);
    // Peer items (AR, RS) take 8 * peers consecutive K-steps of a whole
    // tile, from its first step on (measured at M=4096: shifting them per
    // tile was 10 % slower).  In a split tile each chunk takes its own peers
    // at its first steps.
    const int64_t peer_rows = MODE == gc::MODE_RS ? a.hi - a.lo : a.M;
    Plan pl;
    const int err = make_plan(a.m_rows, a.N, a.K, MODE == gc::MODE_AG ? a.R : 1,
                              MODE == gc::MODE_AG ? 0 : a.npeers,
                              MODE == gc::MODE_AG ? 0 : (int64_t)a.npeers * peer_rows * a.N * 2, cus,
                              ws_ok, peers->tile_rows, pl);
    if (err)
        return err;
    if (pl.num_tiles == 0)
        return GC_OK;
    const int bm = pl.bm;
    const bool peer_nt = pl.peer_nt;
    const int grid = pl.grid;
    a.tiles_n = pl.tiles_n;
    a.tiles_m = pl.tiles_m;
    a.num_tiles = pl.num_tiles;
    a.group_m = 4;
    a.dp_tiles = pl.dp_tiles;
    a.sk_tiles = pl.sk_tiles;
    a.sk_q = pl.sk_q;
    a.sk_chunk = pl.sk_chunk;
    a.sk_units = pl.sk_units;
    if (pl.sk_units > 0) {
        char *ws = (char *)peers->workspace;
        a.sk_count = (unsigned long long *)ws;
        a.sk_claim = (uint32_t *)(ws + count_bytes(cus));
        a.sk_flags = (uint32_t *)(ws + count_bytes(cus) + claim_bytes(cus));
        a.sk_part = (float *)(ws + count_bytes(cus) + claim_bytes(cus) + flag_bytes(cus));
        a.sk_slots = cus;
        a.sk_epoch = g_epoch[dev < kMaxDevices ? dev : 0].fetch_add(1) + 1;
        a.sk_max_spins = 1u << 22;
        // About 0.3 ms of polling: far more than the spread of the units'
        // arrival times when they run at once (measured: up to 25 us), short
        // when they do not.
        a.sk_wait_spins = 256;
        // For tests: peers->split_wait_spins overrides that limit (a limit of
        // 1 makes nearly every unit give up at once, so that the last unit to
        // arrive finishes their shares).
        if (peers->split_wait_spins != 0)
            a.sk_wait_spins = peers->split_wait_spins;
        // The last unit to arrive leaves the others about 30 us to claim
        // their shares (they see its flag and claim within a few us) before
        // it claims what is left.
        a.sk_grace_spins = 32;
    }
    constexpr bool NT_OK = MODE != gc::MODE_AG;
    // Instances: row blocks per wave (tile rows / 32), non-temporal peer
    // loads (256- and 224-row tiles only), split units or whole tiles.
    auto launch = [&](int fmt, bool nt, bool split, int g, const gc::Args &x) {
        const dim3 gd(g), bd(gc::NT);
        nt = NT_OK && nt;
        if (split) {
            switch (fmt) {
            case 2: hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 2, true>), gd, bd, 0, stream, x); break;
            case 4: hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 4, true>), gd, bd, 0, stream, x); break;
            default: hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 8, true>), gd, bd, 0, stream, x); break;
            }
            return;
        }
        switch (fmt) {
        case 2: hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 2, false>), gd, bd, 0, stream, x); break;
        case 4: hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 4, false>), gd, bd, 0, stream, x); break;
        case 7:
            if (nt)
                hipLaunchKernelGGL((gc::gc_kernel<MODE, NT_OK, 7, false>), gd, bd, 0, stream, x);
            else
                hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 7, false>), gd, bd, 0, stream, x);
            break;
        default:
            if (nt)
                hipLaunchKernelGGL((gc::gc_kernel<MODE, NT_OK, 8, false>), gd, bd, 0, stream, x);
            else
                hipLaunchKernelGGL((gc::gc_kernel<MODE, false, 8, false>), gd, bd, 0, stream, x);
            break;
        }
    };
    const int fmt = bm / 32;
    if (a.sk_units > 0) {
        // The full rounds as whole tiles, then the split launch: tiles
        // dp_tiles .. num_tiles-1, one unit per workgroup.  (Stream order
        // makes the second wait for the first.)
        if (a.dp_tiles > 0) {
            gc::Args d = a;
            d.sk_units = 0;
            launch(fmt, peer_nt, false, cus, d);
        }
        // (the split tail reads few peers: plain loads)
        launch(fmt, false, true, grid, a);
    } else {
        launch(fmt, peer_nt, false, grid, a);
    }
    return hipGetLastError() == hipSuccess ? GC_OK : GC_EIO;
}

template <int NP>
void launch_peer_sum(const uint16_t *local, const uint16_t *partials, int64_t stride, int64_t n,
                     uint16_t *out, int blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((gc::peer_sum_kernel<NP>), dim3(blocks), dim3(gc::PS_THREADS), 0, stream,
                       local, partials, stride, n, out);
}

}  // namespace

extern "C" {

int gemm_coll_should_run(int64_t M) { return M >= 128 ? 1 : 0; }

int gemm_coll_plan(int mode, int64_t M, int64_t N, int64_t K, int R, int rank, int cus,
                   int with_workspace, uint32_t tile_rows, gc_plan *plan)
{
    if (!plan || mode < GC_MODE_AR || mode > GC_MODE_AG || cus < 1 || cus > 4096)
        return GC_EINVAL;
    if (M < 0 || N < 0 || K < 0 || !(R > 1 && R <= 16 && 128 % R == 0) || rank < 0 || rank >= R)
        return GC_EINVAL;
    if (N % 8 != 0 || K % 8 != 0)
        return GC_EINVAL;
    switch (tile_rows) {
    case 0: case 64: case 128: case 224: case 256:
        break;
    default:
        return GC_EINVAL;
    }
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return GC_ENOTSUP;
    const bool ag = mode == GC_MODE_AG;
    if (!fits(M, K) || !fits(K, N) || !fits(ag ? M * R : M, N))
        return GC_ENOTSUP;
    int64_t m_rows = M, peer_rows = M;
    if (mode == GC_MODE_RS) {
        int64_t P, lo, hi, end;
        rs_slice(M, R, rank, P, lo, hi, end);
        m_rows = end > M ? end : M;
        peer_rows = hi - lo;
    }
    Plan pl;
    int err = GC_OK;
    if (M > 0 && N > 0)
        err = make_plan(m_rows, N, K, ag ? R : 1, ag ? 0 : R - 1,
                        ag ? 0 : (int64_t)(R - 1) * peer_rows * N * 2, cus, with_workspace != 0,
                        tile_rows, pl);
    if (err)
        return err;
    plan->tile_rows = (uint32_t)pl.bm;
    plan->tiles = pl.num_tiles;
    plan->whole_tiles = pl.dp_tiles;
    plan->split_tiles = pl.sk_tiles;
    plan->chunks = pl.sk_q;
    plan->chunk_steps = pl.sk_chunk;
    plan->units = pl.sk_units;
    plan->grid = pl.grid;
    plan->peer_nt = pl.peer_nt ? 1 : 0;
    return GC_OK;
}

int64_t gemm_coll_workspace_bytes(void)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return GC_EIO;
    return workspace_bytes_for(cu_count(dev));
}

const char *gemm_coll_strerror(int code)
{
    switch (code) {
    case GC_OK:
        return "success";
    case GC_EINVAL:
        return "invalid argument (NULL or misaligned pointer, R or rank out of range, negative "
               "size, N/K not a multiple of 8, or tile_rows other than 0, 64, 128, 224 and 256)";
    case GC_ENOTSUP:
        return "shape not supported by this kernel set (a buffer of 2 GiB or more)";
    case GC_EIO:
        return "HIP kernel launch failed";
    case GC_ENOSPC:
        return "gemm_ar_noalloc: the library's static scratch (split state for up to 256 "
               "compute units) is smaller than this device needs";
    default:
        if (code >= GC_TIMEOUT_BASE && code < GC_TIMEOUT_BASE + 16)
            return "AG-GEMM: a shard's ready flag did not arrive in time";
        return "unknown error code";
    }
}

int gemm_ar(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R, int rank,
            const gc_peers *peers, gc_bf16 *out, void *stream)
{
    int err = check_common(A, B, M, N, K, R, rank, peers, out);
    if (err || M == 0 || N == 0)
        return err;
    if (!peers->partials || !aligned16(peers->partials))
        return GC_EINVAL;
    if (!fits(M, K) || !fits(K, N) || !fits(M, N))
        return GC_ENOTSUP;
    gc::Args a = {};
    a.A = A;
    a.B = B;
    a.partials = peers->partials;
    a.out = out;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.R = R;
    a.rank = rank;
    a.npeers = R - 1;
    a.m_rows = (int)M;
    a.status = peers->status;
    return dispatch<gc::MODE_AR>(a, peers, (hipStream_t)stream);
}

int gemm_ar_noalloc(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R,
                    int rank, const gc_peers *peers, gc_bf16 *out, void *stream)
{
    // The checks of gemm_ar first, so that invalid calls fail before any
    // device call.
    int err = check_common(A, B, M, N, K, R, rank, peers, out);
    if (err || M == 0 || N == 0)
        return err;
    if (!peers->partials || !aligned16(peers->partials))
        return GC_EINVAL;
    if (!fits(M, K) || !fits(K, N) || !fits(M, N))
        return GC_ENOTSUP;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return GC_EIO;
    // The split state of a call needs workspace_bytes_for(compute units):
    // no problem size needs more, and the scratch holds it for up to
    // kScratchSlots units.
    if (workspace_bytes_for(cu_count(dev)) > kScratchBytes)
        return GC_ENOSPC;
    void *ws = nullptr;
    err = scratch_address(dev, &ws);
    if (err)
        return err;
    gc_peers p = *peers;
    p.workspace = ws;
    p.workspace_bytes = (uint64_t)kScratchBytes;
    return gemm_ar(A, B, M, N, K, R, rank, &p, out, stream);
}

// GEMM-RS, or (two_shot) the two-shot GEMM-AR that extends it.
static int rs_common(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R, int rank,
              const gc_peers *peers, gc_bf16 *out, void *stream, bool two_shot)
{
    int err = check_common(A, B, M, N, K, R, rank, peers, out);
    if (err || M == 0 || N == 0)
        return err;
    if (!peers->partials || !aligned16(peers->partials) || !peers->ws || !aligned16(peers->ws))
        return GC_EINVAL;
    if (two_shot && (!peers->peer_out || !aligned16(peers->peer_out)))
        return GC_EINVAL;
    if (!fits(M, K) || !fits(K, N) || !fits(M, N))
        return GC_ENOTSUP;
    if (M == 0 || N == 0)
        return GC_OK;
    int64_t P, lo, hi, end;
    rs_slice(M, R, rank, P, lo, hi, end);
    gc::Args a = {};
    a.A = A;
    a.B = B;
    a.partials = peers->partials;
    a.out = out;
    a.ws = peers->ws;
    a.peer_out = two_shot ? peers->peer_out : nullptr;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.R = R;
    a.rank = rank;
    a.npeers = R - 1;
    a.P = (int)P;
    a.lo = (int)lo;
    a.hi = (int)hi;
    a.m_rows = (int)(end > M ? end : M);
    a.status = peers->status;
    return dispatch<gc::MODE_RS>(a, peers, (hipStream_t)stream);
}

int gemm_rs(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R, int rank,
            const gc_peers *peers, gc_bf16 *out, void *stream)
{
    return rs_common(A, B, M, N, K, R, rank, peers, out, stream, false);
}

int gemm_ar_two_shot(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R,
                     int rank, const gc_peers *peers, gc_bf16 *out, void *stream)
{
    return rs_common(A, B, M, N, K, R, rank, peers, out, stream, true);
}

int ag_gemm(const gc_bf16 *A, const gc_bf16 *B, int64_t Ms, int64_t N, int64_t K, int R, int rank,
            const gc_peers *peers, gc_bf16 *out, void *stream)
{
    int err = check_common(A, B, Ms, N, K, R, rank, peers, out);
    if (err || Ms == 0 || N == 0)
        return err;
    // (with K = 0 the shards hold no element and are never read)
    if ((K > 0 && (!peers->shards || !aligned16(peers->shards))) || !peers->flags ||
        ((uintptr_t)peers->flags & 3u) || !peers->status || ((uintptr_t)peers->status & 3u))
        return GC_EINVAL;
    if (!fits(Ms, K) || !fits(K, N) || !fits(Ms * R, N))
        return GC_ENOTSUP;
    gc::Args a = {};
    a.A = A;
    a.B = B;
    a.shards = peers->shards;
    a.flags = peers->flags;
    a.status = peers->status;
    a.epoch = peers->epoch;
    // A poll is one system-scope load (about a microsecond) plus a short
    // s_sleep; the default bound gives up after one to two seconds.
    a.max_spins = peers->max_spins ? peers->max_spins : (1u << 20);
    a.out = out;
    a.M = (int)Ms;
    a.N = (int)N;
    a.K = (int)K;
    a.R = R;
    a.rank = rank;
    a.m_rows = (int)Ms;
    return dispatch<gc::MODE_AG>(a, peers, (hipStream_t)stream);
}

int ag_push_shards(const gc_bf16 *src, gc_bf16 *dst, int64_t Ms, int64_t K, int R, int rank,
                   uint32_t *flags, const uint32_t *epoch_word, void *stream)
{
    if (R < 2 || R > 16 || 128 % R != 0 || rank < 0 || rank >= R || Ms < 0 || K < 0)
        return GC_EINVAL;
    if (!src || !dst || !flags || !epoch_word || !aligned16(src) || !aligned16(dst) ||
        ((uintptr_t)flags & 3u) || ((uintptr_t)epoch_word & 3u))
        return GC_EINVAL;
    const size_t shard = (size_t)Ms * (size_t)K;   // elements
    hipStream_t st = (hipStream_t)stream;
    // Round s brings shard q = (rank - s) mod R, the order ag_gemm consumes
    // them in; the flag of a shard is written after its copy, in the same
    // stream, so it is raised only once the shard has landed.  Both go
    // through the DMA engines (no compute units), so they make progress
    // while ag_gemm holds every compute unit.
    for (int s = 1; s < R; ++s) {
        const int q = (rank - s + R) % R;
        if (shard > 0 && hipMemcpyAsync(dst + q * shard, src + q * shard, shard * 2,
                                        hipMemcpyDeviceToDeviceNoCU, st) != hipSuccess)
            return GC_EIO;
        if (hipMemcpyAsync(flags + q, epoch_word, 4, hipMemcpyDeviceToDeviceNoCU, st) != hipSuccess)
            return GC_EIO;
    }
    return GC_OK;
}


int gemm_coll_peer_sum(const gc_bf16 *local, const gc_bf16 *partials, int64_t rows, int64_t N,
                       int npeers, int64_t peer_stride, gc_bf16 *out, void *stream)
{
    if (rows < 0 || N < 0 || npeers < 0 || npeers > 15)
        return GC_EINVAL;
    const int64_t n = rows * N;
    if (n == 0)
        return GC_OK;
    if (!local || !out || !aligned16(local) || !aligned16(out))
        return GC_EINVAL;
    if (npeers > 0 && (!partials || !aligned16(partials) || peer_stride % 8 != 0 ||
                       (npeers > 1 && peer_stride < n)))
        return GC_EINVAL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return GC_EIO;
    // enough workgroups for every CU several times over, each lane a few
    // 16-byte vectors
    const int64_t want = (n / 8 + gc::PS_THREADS - 1) / gc::PS_THREADS;
    const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)cu_count(dev) * 16));
    const uint16_t *l = (const uint16_t *)local, *pp = (const uint16_t *)partials;
    uint16_t *o = (uint16_t *)out;
    hipStream_t st = (hipStream_t)stream;
    switch (npeers) {
    case 0: launch_peer_sum<0>(l, pp, peer_stride, n, o, blocks, st); break;
    case 1: launch_peer_sum<1>(l, pp, peer_stride, n, o, blocks, st); break;
    case 2: launch_peer_sum<2>(l, pp, peer_stride, n, o, blocks, st); break;
    case 3: launch_peer_sum<3>(l, pp, peer_stride, n, o, blocks, st); break;
    case 4: launch_peer_sum<4>(l, pp, peer_stride, n, o, blocks, st); break;
    case 5: launch_peer_sum<5>(l, pp, peer_stride, n, o, blocks, st); break;
    case 6: launch_peer_sum<6>(l, pp, peer_stride, n, o, blocks, st); break;
    case 7: launch_peer_sum<7>(l, pp, peer_stride, n, o, blocks, st); break;
    case 8: launch_peer_sum<8>(l, pp, peer_stride, n, o, blocks, st); break;
    case 9: launch_peer_sum<9>(l, pp, peer_stride, n, o, blocks, st); break;
    case 10: launch_peer_sum<10>(l, pp, peer_stride, n, o, blocks, st); break;
    case 11: launch_peer_sum<11>(l, pp, peer_stride, n, o, blocks, st); break;
    case 12: launch_peer_sum<12>(l, pp, peer_stride, n, o, blocks, st); break;
    case 13: launch_peer_sum<13>(l, pp, peer_stride, n, o, blocks, st); break;
    case 14: launch_peer_sum<14>(l, pp, peer_stride, n, o, blocks, st); break;
    default: launch_peer_sum<15>(l, pp, peer_stride, n, o, blocks, st); break;
    }
    return hipGetLastError() == hipSuccess ? GC_OK : GC_EIO;
}

}  // extern "C"
