// gc_kernel.hpp -- gfx950 device code of the fused TP GEMM + reduction.
//
// One persistent kernel template serves the three modes:
//   AR  out = bf16(acc + sum of the R-1 peer partials)          (all rows)
//   RS  slice rows as AR into out; other valid rows bf16(acc) into ws
//       (two-shot AR: the same, with the reduced slice rows stored into a
//       full-height out and into each of the R-1 peer outputs)
//   AG  out rows of shard q = bf16(acc); shards taken in ring order, each
//       behind a ready flag polled in the kernel
// (GEMM-AR / GEMM-RS: "[Kimi-K3] Extend GEMM-RS to GEMM-AR", 实现拆解 step 1
//  and the test reference in 关键源码片段; AG-GEMM: "[Kimi-K3] AG-GEMM for
//  Sequence Parallelism", Purpose, Implementation details, and the remark
//  under its component breakdown table about one GEMM kernel that waits
//  inside the kernel.)
//
// Tile: 256 x 256 outputs per workgroup of eight waves (two per SIMD) in a
// 2 (m) x 4 (n) grid; each wave owns 128 x 64 outputs as 8 x 4 blocks of
// v_mfma_f32_16x16x32_bf16.  A second instance has 224-row tiles (7 x 4
// blocks per wave), which the host picks where it fills the last round of
// tiles better (at M=4096, N=6288: 475 tiles in two rounds of 256 instead of
// 400 of the taller tiles, 12 % less work per workgroup).  K advances 32 per step through a ring of four
// LDS stages (16 KiB of A + 16 KiB of B each), so the loads of a stage are
// issued three steps before it is consumed.
//
// Operand staging:
//   A stage  [256 m][32 k]  64 B per row; 16-byte chunk c of row m is stored
//            at chunk c ^ ((m/2) % 4).  A fragment read (lane: row m =
//            lane%16, chunk lane/16) is then free of bank conflicts on
//            gfx950; the key (m/4) % 4, conflict-free if a ds_read_b128
//            served 16 consecutive lanes per pass, measured two-way
//            conflicts (8 LDS cycles per read instead of 4).
//   B stage  [32 k][256 n]  512 B per row (B is N-contiguous and stays so);
//            32-byte chunk q of row k is stored at q ^ f(k) with
//            f(k) = (k % 4) + 4 * ((k / 8) % 2), so the 32 lanes of a
//            ds_read_b64_tr_b16 pass cover all 64 banks.
// Both move global -> LDS with 16-byte buffer loads that write LDS directly
// (no VGPR staging); each wave instruction fills 1 KiB of LDS in lane order,
// so the swizzle is applied by choosing which global chunk each lane
// fetches.  Loads past M, N or K return zeros (buffer range check).
//
// Fragments: the MFMA's first operand is B^T (n rows, 8 consecutive k per
// lane), read with two ds_read_b64_tr_b16 per block: within each 16-lane
// group, lane j receives element j%4 of the 8-byte chunks addressed by
// lanes 4e + j/4 (e = 0..3), so lanes that address rows k..k+3 at column
// offsets 0,4,8,12 deliver to lane j the four k-values of column j.  The
// second operand is A (m rows) read with ds_read_b128.  The 16 x 16 result
// block is then C^T in MFMA layout: lane l holds row m = l%16, columns
// n = 4*(l/16) .. +3 -- four consecutive outputs, 8 bytes in memory.
//
// Peer partials (AR, RS): the R-1 peer tiles are added into the fp32
// accumulators while the K loop runs.  Item w = (peer w/8 - phase, row
// block w%8) is the wave's 16 x 64 block of that peer; it is loaded into one
// of two LDS slots of the wave at step w-2 and added at step w, so the peer
// traffic streams behind the MFMA work.  The items of a whole tile take its
// first 8 * peers steps (items the K loop does not reach are added after
// it); in a tile split along K, each chunk takes its own share of the peers
// at its first steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

enum Mode { MODE_AR = 0, MODE_RS = 1, MODE_AG = 2 };

// Kernel arguments (passed by value).
struct Args {
    const uint16_t *A;         // AR/RS: [M][K]; AG: this rank's shard [Ms][K]
    const uint16_t *B;         // [K][N]
    const uint16_t *partials;  // AR/RS: [R-1][M][N]
    uint16_t *out;             // AR: [M][N]; RS: [P][N]; AG: [R*Ms][N]
    uint16_t *ws;              // RS: [M][N]
    uint16_t *peer_out;        // RS as two-shot AR: [R-1][M][N], or null
    const uint16_t *shards;    // AG: [R][Ms][K]
    const uint32_t *flags;     // AG: [R]
    int32_t *status;           // AG
    uint32_t epoch;
    uint32_t max_spins;
    int M;                     // valid rows (AG: Ms, rows per shard)
    int N, K;
    int R, rank;
    int npeers;                // AR/RS: R-1
    // Peer items: a whole tile adds peer p's items at steps 8p .. 8p+7; a
    // split unit of chunk c adds those of peers [ceil(c*npeers/sk_q),
    // ceil((c+1)*npeers/sk_q)) at its first steps (the host keeps every
    // chunk long enough for them), so the item loads are spread over the
    // tile's units.
    int P, lo, hi;             // RS: slice height and owned valid rows [lo, hi)
    int m_rows;                // rows covered by tiles (per shard for AG)
    int tiles_m, tiles_n;      // per shard for AG
    int num_tiles;             // total (AG: R * tiles_m * tiles_n)
    int group_m;               // row tiles per L2 group
    // Work split.  A whole-tile launch takes tiles 0 .. dp_tiles-1, round by
    // round.  A split launch cuts each of the sk_tiles tiles after them
    // (tiles dp_tiles .. dp_tiles+sk_tiles-1) along K into sk_q <= 16 chunks
    // of sk_chunk steps (a multiple of 8; the last may be shorter), giving
    // sk_units = sk_q * sk_tiles units numbered chunk-major (unit u is
    // chunk u / sk_tiles of tile dp_tiles + u % sk_tiles), one per workgroup:
    // the workgroups of one XCD run the same K range of neighbouring tiles.
    // The units of a tile exchange fp32 partials through sk_part[u] and
    // finish the tile in shares (see the kernel).  Counters, flags and
    // claims hold the launch epoch, so none of them is ever reset.
    int dp_tiles;
    int sk_tiles, sk_q, sk_chunk, sk_units;
    // Slots of the workspace: sk_slots tile slots (counter, claims) and as
    // many unit slots (flags, partial).  A split launch with more units or
    // tiles than slots, or more than 16 chunks, does no work (see the kernel).
    int sk_slots;
    unsigned long long *sk_count;  // [sk_slots]: (epoch << 32) | arrivals
    uint32_t *sk_claim;        // [sk_slots][16]: epoch of the launch that claimed the share
    uint32_t *sk_flags;        // [2 * sk_slots]: epoch, partial valid
    float *sk_part;            // [sk_slots][BM*BN]
    uint32_t sk_epoch;
    uint32_t sk_max_spins;     // guard on waits that always end
    uint32_t sk_wait_spins;    // how long a unit waits for its tile's other units
    uint32_t sk_grace_spins;   // how long the last unit leaves the others to claim
};

constexpr int BM = 256, BN = 256, BK = 32, NT = 512;  // BM: the taller of the two tiles
constexpr int WAVES = NT / 64;             // 8: 2 (m) x 4 (n)
constexpr int WM = 128, WN = 64, FM = 8, FN = 4;
// Peer items are numbered in groups of 8 K-steps, one per row block slot;
// with 7 row blocks per wave the eighth slot of each group is empty.
constexpr int ITEMS_PER_GROUP = 8;
constexpr int STAGES = 4;
constexpr int A_BYTES = BM * BK * 2;       // 16 KiB per stage
constexpr int B_BYTES = BK * BN * 2;       // 16 KiB per stage
constexpr int PSLOT = 16 * WN * 2;         // one peer block of a wave: 2 KiB
// Loads a wave issues per step: stage DMA (2 of A + 2 of B) and peer item (2).
constexpr int DMA_PER_STEP = 4, PEER_PER_ITEM = 2;
constexpr int PART_FLOATS = BM * BN;       // one fp32 partial tile
constexpr uint32_t PART_BYTES = PART_FLOATS * 4u;

// Out-of-range offset for buffer accesses: every buffer addressed here is
// < 2 GiB, so this offset is past num_records; loads return 0, stores drop.
constexpr uint32_t OOB = 0x80000000u;
constexpr int BUFFER_FLAGS = 0x00020000;  // raw buffer, 32-bit data format
// Cache policy of a buffer access: sc0 | sc1 (system coherent: a store writes
// through to memory, a load misses every cache).
constexpr int CPOL_SYS = 1 | 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                             BUFFER_FLAGS);
}

// Buffer resource for the loads below: base, num_records, raw 32-bit format.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t make_rsrc4(const void *p, uint32_t bytes)
{
    const uint64_t a = (uint64_t)p;
    return (u32x4_t){(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, (uint32_t)BUFFER_FLAGS};
}

// A wave-uniform value the compiler may not fold or hoist (an empty asm that
// claims to change it).  LDS addresses built from it are formed where they
// are used instead of being kept in registers for every unrolled step.
__device__ __forceinline__ uint32_t opaque(uint32_t x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// The same for a per-lane value: code after the K loop recomputes its lane
// offsets from this instead of keeping the loop's copies alive through it.
__device__ __forceinline__ int opaque_v(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

template <typename T>
__device__ __forceinline__ const __attribute__((address_space(3))) T *lds_ptr(uint32_t a)
{
    return (const __attribute__((address_space(3))) T *)(uintptr_t)a;
}

// LDS byte address of a __shared__ object, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes global -> LDS at lds + 16 * lane.  Issued as inline assembly so
// that the compiler does not track it: the loop below knows exactly how many
// of these are in flight and waits for them itself (wait_vmcnt), where the
// compiler's own tracking of LDS-DMA loads would wait for nearly all of them.
// M0 is written here only; on gfx950 no other code relies on its value.
__device__ __forceinline__ void dma16(u32x4_t r, uint32_t lds, uint32_t off)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(off), "s"(r)
                 : "memory");
}

// As dma16, marked non-temporal (nt): streaming data read once, which the
// caches should not keep at the expense of the A and B tiles.
__device__ __forceinline__ void dma16_nt(u32x4_t r, uint32_t lds, uint32_t off)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(lds), "v"(off), "s"(r)
                 : "memory");
}

// As dma16, with the system-coherent cache policy (sc0 sc1): the load misses
// every cache, so it sees data another XCD wrote through to memory.  The
// offset is a lane part plus a scalar part (soffset), so that a run of loads
// at different block offsets needs one lane register, not one per block.
__device__ __forceinline__ void dma16_sys(u32x4_t r, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen sc0 sc1 lds"
                 :
                 : "s"(lds), "v"(voff), "s"(r), "s"(soff)
                 : "memory");
}

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ u32x2_t pack_bf16x4(f32x4_t v)
{
    bf16x4_t h = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    return __builtin_bit_cast(u32x2_t, h);
}

// Four bf16 (raw bits in two dwords) -> fp32, exactly.
// Two neighbouring accumulator blocks of a row block (columns 16j .. 16j+31,
// j even), packed to bf16 and regrouped so that every lane holds 8
// consecutive columns of its row: lane (fi, fg) holds columns
// 4fg .. 4fg+3 of each block, and the lanes of 16-lane rows 2k and 2k+1
// (fg = 2k, 2k+1) trade halves with v_permlane16_swap (odd rows of its first
// operand with even rows of its second), after which lane (fi, fg) holds
// columns 8 (fg / 2) + 16 (fg % 2) .. +7 of the pair: block j's for even fg,
// block j+1's for odd fg.  One 16-byte store per lane then writes 16 rows x
// 64 bytes.  All 64 lanes must be active.
__device__ __forceinline__ u32x4_t pack_pair(f32x4_t x, f32x4_t y)
{
    const u32x2_t px = pack_bf16x4(x), py = pack_bf16x4(y);
    const auto s0 = __builtin_amdgcn_permlane16_swap(px[0], py[0], false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(px[1], py[1], false, false);
    return (u32x4_t){s0[0], s1[0], s0[1], s1[1]};
}

__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ f32x4_t unpack_bf16x4(u32x2_t w)
{
    f32x4_t r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xFFFF0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xFFFF0000u);
    return r;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// (Inline assembly with a memory clobber, so that no LDS access moves
// across it.)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0()
{
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}

// Workgroup barrier without the compiler's implicit "vmcnt(0)" that a
// __syncthreads() gets while LDS-DMA loads are pending: every caller waits
// explicitly for exactly the loads the barrier must cover.
// The scheduling barriers keep every instruction on its side of it, so the
// phases of the ping-pong schedule below stay where the code puts them.
__device__ __forceinline__ void barrier_only()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// f(0), f(1), ..., f(7), each index a compile-time constant.
template <class F>
__device__ __forceinline__ void unroll8(F &&f)
{
    f(std::integral_constant<int, 0>{});
    f(std::integral_constant<int, 1>{});
    f(std::integral_constant<int, 2>{});
    f(std::integral_constant<int, 3>{});
    f(std::integral_constant<int, 4>{});
    f(std::integral_constant<int, 5>{});
    f(std::integral_constant<int, 6>{});
    f(std::integral_constant<int, 7>{});
}

// Logical tile of workgroup `b` in one round of `G` workgroups.  Workgroups
// are dispatched round-robin over the 8 XCDs (b % 8); each XCD is handed a
// contiguous run of logical tiles so that the tiles resident on one XCD share
// rows of A and columns of B in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int G)
{
    const int base = G >> 3, rem = G & 7;
    const int x = b & 7, j = b >> 3;
    return x * base + (x < rem ? x : rem) + j;
}

// PEER_NT: peer partials are loaded non-temporal (AR / RS).
// FMT: row blocks of 16 per wave, 8 (256-row tiles) or 7 (224-row tiles).
// SPLIT: the launch runs split units only (after the dp_tiles whole tiles
// that a launch before it took); otherwise whole tiles only, and the
// hand-over code is not compiled in.  (Each instance then
// gets a register allocation of its own: the hand-over's registers do not
// weigh on the whole-tile K loop, nor the reverse.)
template <int MODE, bool PEER_NT, int FMT, bool SPLIT>
__global__ __launch_bounds__(NT, 2) void gc_kernel(Args p)
{
    static_assert(FMT == 8 || FMT == 7 || FMT == 4 || FMT == 2, "row blocks per wave");
    static_assert(!SPLIT || FMT != 7, "224-row tiles are never split");
    if constexpr (SPLIT) {
        // Every workspace index below stays inside the sk_slots slots when
        // sk_units and sk_tiles fit and a tile has at most 16 chunks (one
        // claim word each).  The host plans no other launch; a launch that
        // breaks this anyway leaves at once in every workgroup (a uniform
        // test, before any wait), writes no output and reports a failed
        // hand-over, instead of touching memory past the workspace.
        if (p.sk_units > p.sk_slots || p.sk_tiles > p.sk_slots || p.sk_q > 16) {
            if (threadIdx.x == 0 && blockIdx.x == 0 && p.status)
                atomicCAS(p.status, 0, 1000 + 16);
            return;
        }
    }
    constexpr int FMt = FMT, WMt = 16 * FMT, BMt = 2 * WMt;
    constexpr int NSEG = 2 * FMt;          // hand-over segments per wave
    // One array per operand and stage: distinct LDS objects carry distinct
    // alias scopes, so the compiler knows that the loads filling one stage
    // cannot alias the fragment reads of another and does not wait for them.
    // (Few enough objects that the compiler's per-object tracking of LDS-DMA
    // loads stays exact.)  Each stage holds A then B.
    __shared__ __attribute__((aligned(16))) uint8_t sS0[A_BYTES + B_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sS1[A_BYTES + B_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sS2[A_BYTES + B_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sS3[A_BYTES + B_BYTES];
    // Peer staging (AR / RS): two slots of one 16 x 64 bf16 block per wave.
    __shared__ __attribute__((aligned(16))) uint8_t sP0[WAVES * PSLOT];
    __shared__ __attribute__((aligned(16))) uint8_t sP1[WAVES * PSLOT];
    __shared__ int s_ready;
    constexpr bool PEERS = MODE != MODE_AG;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int G = gridDim.x;
    const int KT = (p.K + BK - 1) / BK;
    const uint32_t N2 = (uint32_t)p.N * 2u;

    const u32x4_t rB = make_rsrc4(p.B, (uint32_t)p.K * N2);

    // ---- per-lane constants -------------------------------------------------
    // A loader: wave instruction j (0..1) fills LDS rows 16*(2*wave+j) +
    // lane/4 (64 B each); the lane's stored chunk lane%4 holds logical chunk
    // (lane%4) ^ ((row/2)%4) = (lane%4) ^ ((lane/8)%4).
    const int a_c = (lane & 3) ^ ((lane >> 3) & 3);
    // B loader: wave instruction j (0..1) fills LDS rows k = 4*wave + 2*j +
    // lane/32 (512 B each); the lane's stored 16-byte slot lane%32 is half
    // lane%2 of stored 32-byte chunk (lane%32)/2 = logical chunk ^ f(k).
    const int b_slot = lane & 31;
    // fragment reads
    const int fi = lane & 15, fg = lane >> 4;
    const uint32_t a_frag = (uint32_t)(wm * WMt * 64 + fi * 64 + ((fg ^ ((fi >> 1) & 3)) << 4));
    const int fB = (fi >> 2) | ((fg & 1) << 2);
    // B^T block j of this wave is logical 32-byte chunk q = 4*wn + j.
    uint32_t b_frag_j[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
        b_frag_j[j] = (uint32_t)((8 * fg + (fi >> 2)) * 512 + (wn >> 1) * 256 + 8 * (fi & 3) +
                                 (((4 * (wn & 1) + j) ^ fB) * 32));

    // Work list of this workgroup: whole tiles round by round, then its
    // split units u = v, v + G, ..., each the K-steps [g0, g1) of one tile.
    const int v = xcd_remap(blockIdx.x, G);    // position within a round
    int dp_lin = 0;                            // first tile of the next whole-tile round
    int unit = v;                              // next split unit of this workgroup
    for (;;) {
        int L, g0, g1, phase, peer_end = p.npeers;
        bool bad = false;
        if (!SPLIT && dp_lin < p.dp_tiles) {
            const int lin = dp_lin;
            const int live = min(G, p.dp_tiles - lin);
            dp_lin = live < G ? p.dp_tiles : lin + G;   // no overflow past dp_tiles
            if ((int)blockIdx.x >= live)
                continue;                      // idle in this last, partial round
            L = lin + xcd_remap(blockIdx.x, live);
            g0 = 0;
            g1 = KT;
            phase = 0;
        } else if (SPLIT && unit < p.sk_units) {
            const int c = unit / p.sk_tiles;
            g0 = c * p.sk_chunk;
            g1 = min(KT, g0 + p.sk_chunk);
            L = p.dp_tiles + (unit - c * p.sk_tiles);
            // Peers [pa, pb) at steps g0 .. g0 + 8 (pb - pa) - 1: item w reads
            // peer w/8 - phase.
            const int pa = (c * p.npeers + p.sk_q - 1) / p.sk_q;
            peer_end = __builtin_amdgcn_readfirstlane(((c + 1) * p.npeers + p.sk_q - 1) / p.sk_q);
            phase = __builtin_amdgcn_readfirstlane(g0 / 8 - pa);
            unit += G;
        } else {
            break;
        }

        // Tile: shard step s (AG), row tile mt, column tile nt, grouped
        // column-major over `group_m` row tiles for L2 reuse.
        int s = 0, t = L;
        const int per_shard = p.tiles_m * p.tiles_n;
        if (MODE == MODE_AG) {
            s = t / per_shard;
            t -= s * per_shard;
        }
        const int gsize = p.group_m * p.tiles_n;
        const int grp = t / gsize;
        const int in_g = t - grp * gsize;
        const int gm0 = grp * p.group_m;
        const int gh = min(p.group_m, p.tiles_m - gm0);
        const int mt = gm0 + in_g % gh;
        const int nt = in_g / gh;
        const int m0 = mt * BMt, n0 = nt * BN;

        // Every load of the previous segment has landed and every wave is
        // done reading its LDS stages before this segment's loads reuse them.
        wait_vmcnt<0>();
        barrier_only();
        // Fragment offsets, redefined here: if the compiler parked them in
        // scratch, their reload completes now and not through a wait for
        // every outstanding load at the top of each pass of the K loop.
        uint32_t bfj[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            bfj[j] = (uint32_t)opaque_v((int)b_frag_j[j]);
        const uint32_t afr = (uint32_t)opaque_v((int)a_frag);

        // In a split launch every segment is a split unit, unit - G (derived
        // from the loop state instead of being kept live across the K loop).
        const bool split = SPLIT && p.sk_q > 1;
        auto cur_unit = [&]() { return unit - G; };
        // Raise the partial-ready flag of unit u (after its partial, if
        // any, is stored and written back).
        // Flags are two words per unit: [2u] the epoch of its last hand-over,
        // [2u+1] whether that partial is valid.  Partials and flags move with
        // system-coherent accesses (sc0 sc1: stores write through, loads
        // miss the L2), so handing one over needs no L2 write-back or
        // invalidation, which would evict the A and B tiles every other
        // workgroup of the XCD is using.  Order: every store of the partial
        // completed (vmcnt 0 in every wave), then the valid word, then the
        // epoch word.
        auto signal_partial = [&](uint32_t ok) {
            wait_vmcnt<0>();
            barrier_only();
            if (tid == 0) {
                __hip_atomic_store(p.sk_flags + 2 * cur_unit() + 1, ok, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
                wait_vmcnt<0>();
                __hip_atomic_store(p.sk_flags + 2 * cur_unit(), p.sk_epoch, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_SYSTEM);
                wait_vmcnt<0>();       // raised before the unit counts itself in
            }
        };

        const uint16_t *Asrc = p.A;
        int q = 0;
        if (MODE == MODE_AG) {
            q = p.rank - s;
            if (q < 0)
                q += p.R;
            if (q != p.rank) {
                Asrc = p.shards + (size_t)q * p.M * p.K;
                if (tid == 0) {
                    uint32_t spins = 0;
                    int ok = 0;
                    for (;;) {
                        uint32_t f = __hip_atomic_load(p.flags + q, __ATOMIC_ACQUIRE,
                                                       __HIP_MEMORY_SCOPE_SYSTEM);
                        if ((int32_t)(f - p.epoch) >= 0) {
                            ok = 1;
                            break;
                        }
                        // Once a time-out is recorded (by any workgroup),
                        // a shard that is not ready is skipped at once: a
                        // launch whose producer has stalled then takes about
                        // one waiting period, not one per tile or per shard.
                        if (++spins >= p.max_spins ||
                            __hip_atomic_load(p.status, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT) != 0)
                            break;
                        __builtin_amdgcn_s_sleep(8);
                    }
                    if (!ok)
                        atomicCAS(p.status, 0, 1000 + q);
                    s_ready = ok;
                }
                __syncthreads();
                const int ok = s_ready;
                __syncthreads();
                if (!ok) {
                    // The tile cannot be finished.  A split unit still goes
                    // through the hand-over (with no K-steps and an invalid
                    // partial) so that the tile's other units do not wait
                    // for it until their time-out.
                    if (!split)
                        continue;
                    bad = true;
                    g1 = g0;
                }
            }
        }
        const u32x4_t rA = make_rsrc4(Asrc, (uint32_t)p.M * (uint32_t)p.K * 2u);

        // ---- loader offsets for this tile at k0 = 0 (rows past M and
        // columns past N already folded into OOB); a step adds its k0 ----
        uint32_t a_off[2], b_off[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // (rows of the stage past a 224-row tile load nothing)
            const int row = m0 + 16 * (2 * wave + j) + (lane >> 2);
            a_off[j] = 16 * (2 * wave + j) < BMt && row < p.M
                           ? ((uint32_t)row * (uint32_t)p.K + (uint32_t)(8 * a_c)) * 2u
                           : OOB;
            const int k = 4 * wave + 2 * j + (lane >> 5);
            const int fk = (k & 3) | (((k >> 3) & 1) << 2);
            const int n = n0 + 16 * ((b_slot >> 1) ^ fk) + 8 * (b_slot & 1);
            b_off[j] = n < p.N ? ((uint32_t)k * (uint32_t)p.N + (uint32_t)n) * 2u : OOB;
        }
        // Loads of stage kt into (sa, sb).  Steps past the K loop issue the
        // same number of loads, all out of range, so that the wait counts of
        // the loop stay constant.
        // Steps at or past g1 (the end of this segment) issue the same number
        // of loads, all out of range.
        auto dma_stage = [&](int kt, const uint8_t *sa, const uint8_t *sb) {
            const int k0 = kt * BK;
            const uint32_t ka = (uint32_t)k0 * 2u, kb = (uint32_t)k0 * N2;
            const uint32_t la = lds_addr(sa) + (uint32_t)(16 * (2 * wave) * 64);
            const uint32_t lb = lds_addr(sb) + (uint32_t)((4 * wave) * 512);
            if (kt >= g1) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(rA, la + j * 1024, OOB);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(rB, lb + j * 1024, OOB);
            } else if (k0 + BK <= p.K) {   // whole step inside K: no per-lane K test
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(rA, la + j * 1024, a_off[j] + ka);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(rB, lb + j * 1024, b_off[j] + kb);
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(rA, la + j * 1024, k0 + 8 * a_c < p.K ? a_off[j] + ka : OOB);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    dma16(rB, lb + j * 1024,
                          k0 + 4 * wave + 2 * j + (lane >> 5) < p.K ? b_off[j] + kb : OOB);
            }
        };

        // ---- peer items (AR / RS) ----
        // Item (peer pp, row block i) is the wave's 16 x 64 block of that
        // peer partial: rows blk .. blk+15 (blk = m0 + 128*wm + 16*i), columns
        // n0 + 64*wn .. +63.  It moves global -> LDS with two 16-byte DMA
        // instructions per wave, instruction t reading whole 128-byte rows
        // 8t .. 8t+7 of the block (rows cut into 64-byte pieces read about a
        // third slower from HBM).  In LDS block row r takes 128 bytes at
        // r * 128, its 16-byte chunk c (columns 8c .. 8c+7) at position
        // c ^ ((r/2) % 8), so that a read-back pass over 16 rows hits 16
        // distinct banks; the DMA writes in lane order, so lane l of
        // instruction t fetches row r = 8t + l/8, chunk (l%8) ^ ((r/2) % 8)
        // (for t = 1 that is instruction 0's chunk ^ 4).  The buffer starts
        // at the first row that may be read (>= row_lo) and ends at row_hi,
        // so rows outside [row_lo, row_hi) read as zero (rows below wrap past
        // 2^31); chunks past N are masked per lane on edge tiles.  Items
        // outside [wlo, whi) load nothing (an empty buffer).
        const int row_lo = MODE == MODE_RS ? p.lo : 0;
        const int row_hi = MODE == MODE_RS ? p.hi : p.M;
        int W = 0;
        if (PEERS && m0 < row_hi && m0 + BMt > row_lo)
            W = peer_end * ITEMS_PER_GROUP;
        // row lane/8 and chunk (lane%8) ^ ((lane/16)%4) for instruction 0
        const int pd_n = n0 + wn * WN + 8 * ((lane & 7) ^ ((lane >> 4) & 3));
        const uint32_t pd_off = (uint32_t)(lane >> 3) * N2 + (uint32_t)pd_n * 2u;
        // Items this segment adds: those whose step lies in it (the drain
        // after the K loop moves the window to the items past KT).  The
        // phase shifts the tile's item steps; item w reads peer w/8 - phase
        // (pbase is the peer array moved back by `phase` peers).
        int wlo = max(g0, 8 * phase), whi = min(g1, 8 * phase + W);
        const uint16_t *pbase = p.partials - (size_t)phase * p.M * p.N;
        // Item w into the 2 KiB of LDS at ls.
        auto peer_dma_at = [&](uint32_t ls, int w, int i, uint32_t pd_off, int pd_n) {
            const bool live_item = w >= wlo && w < whi && i < FMt;
            const int pp = live_item ? (w >> 3) : phase;
            const int blk = m0 + wm * WMt + 16 * i;
            const int start = max(blk, row_lo);
            const int rows = live_item ? max(row_hi - start, 0) : 0;
            const u32x4_t rp = make_rsrc4(
                pbase + (size_t)pp * p.M * p.N + (size_t)start * p.N, (uint32_t)rows * N2);
            const uint32_t off = pd_off - (uint32_t)(start - blk) * N2;
            // instruction 1: rows 8 further on, chunk ^ 4 (32 columns back
            // when the lane's chunk has bit 2 set, forward otherwise)
            const bool back = (lane & 4) != 0;
            const int pd_n1 = back ? pd_n - 32 : pd_n + 32;
            const uint32_t off1 = off + 8u * N2 + (back ? (uint32_t)-64 : 64u);
            if constexpr (PEER_NT) {
                dma16_nt(rp, ls, pd_n < p.N ? off : OOB);
                dma16_nt(rp, ls + 1024, pd_n1 < p.N ? off1 : OOB);
            } else {
                dma16(rp, ls, pd_n < p.N ? off : OOB);
                dma16(rp, ls + 1024, pd_n1 < p.N ? off1 : OOB);
            }
        };
        auto peer_dma = [&](const uint8_t *slotbuf, int w, int i, uint32_t pd_off, int pd_n) {
            peer_dma_at(lds_addr(slotbuf) + (uint32_t)(wave * PSLOT), w, i, pd_off, pd_n);
        };
        // Reading back: lane (fi, fg) needs row fi, columns 16*j + 4*fg .. +3,
        // i.e. half fg%2 of chunk c = 2*j + fg/2, at position c ^ s of the
        // row (s = (fi/2) % 8).  With s = 2*sh + sl that is byte
        // pc_off ^ (32*j), pc_off = 128*fi + 8*(fg%2) + 16*((fg/2) ^ sl) + 32*sh.
        const uint32_t pc_off = (uint32_t)(fi * 128 + 8 * (fg & 1) + 16 * ((fg >> 1) ^ ((fi >> 1) & 1)) +
                                           32 * ((fi >> 2) & 3));

        f32x4_t acc[FMt][FN];
#pragma unroll
        for (int i = 0; i < FMt; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

        auto read_frags = [&](const uint8_t *cA, bf16x8_t (&fa)[FN], bf16x8_t (&fb)[FMt]) {
            const uint32_t sa = opaque(lds_addr(cA)), sb = sa + A_BYTES;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const uint32_t base = sb + bfj[j];
                bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4_t *)lds_ptr<bf16x4_t>(base));
                bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4_t *)lds_ptr<bf16x4_t>(base + 4 * 512));
                fa[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            const uint32_t ab = sa + afr;
#pragma unroll
            for (int i = 0; i < FMt; ++i)
                fb[i] = *lds_ptr<bf16x8_t>(ab + i * 16 * 64);
        };
        auto mfmas = [&](const bf16x8_t (&fa)[FN], const bf16x8_t (&fb)[FMt]) {
#pragma unroll
            for (int i = 0; i < FMt; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[j], fb[i], acc[i][j], 0, 0, 0);
        };

        // Prologue: virtual steps g0-3, g0-2, g0-1 issue stages g0 .. g0+2 and
        // peer items g0-1 (nothing), g0, g0+1, exactly as a loop step would.
        // (g0 is a multiple of 8: the stage ring restarts at the segment, the
        // slot of item w is w % 2 and its row block w % 8.)
        dma_stage(g0, sS0, sS0 + A_BYTES);
        if (PEERS)
            peer_dma(sP1, g0 - 1, 7, pd_off, pd_n);
        dma_stage(g0 + 1, sS1, sS1 + A_BYTES);
        if (PEERS)
            peer_dma(sP0, g0, 0, pd_off, pd_n);
        dma_stage(g0 + 2, sS2, sS2 + A_BYTES);
        if (PEERS)
            peer_dma(sP1, g0 + 1, 1, pd_off, pd_n);

        // ---- main loop: ping-pong between the two waves of each SIMD ----
        // Waves 0-3 (group 0) and 4-7 (group 1) sit one per SIMD each.  Step
        // kt is a memory phase M(kt) -- fragment reads of stage kt, loads of
        // stage kt+3, peer item kt added and item kt+2 loaded -- then a
        // compute phase C(kt) of 32 MFMAs.  Group 1 runs one phase behind
        // group 0, so on every SIMD one wave computes while the other does
        // its memory phase; a barrier separates phases:
        //   group 0:  M0 C0 M1 C1 ...      group 1:  -- M0 C0 M1 C1 ...
        // At the end of M(kt) a wave has its own loads of stage kt+1 done
        // (the loads after them -- stages kt+2, kt+3, items kt..kt+2 -- may
        // fly) and its fragment reads of stage kt complete, so after the
        // next barrier of the other group's M(kt+1)... every stage read is
        // complete and every stage about to be read has landed.
        // The loop is unrolled by 8 so that the stage, the peer slot and the
        // peer row block are compile-time constants.
        //
        // The peer items of a segment take its first steps: the window
        // [wlo, whi) starts at g0.  Steps [g0, E), E the end of the window
        // rounded up to whole groups of 8, run as above; the steps after E
        // issue no peer loads at all (no empty ones either).  Their waits
        // for stage kt+1 then count only the stage loads after it, except in
        // steps E and E+1, when the empty loads of items E and E+1 (issued
        // in steps E-2 and E-1) are still younger than it.
        constexpr int AFTER = 2 * DMA_PER_STEP + (PEERS ? 3 * PEER_PER_ITEM : 0);
        const bool lag = wave >= 4;
        wait_vmcnt<AFTER>();          // own loads of stage 0 done
        if (lag)
            barrier_only();
        // ITEMS: the step adds item kt and loads item kt+2; otherwise tr is
        // the step's distance from E (0, 1, or 2 for any later step).
        auto step = [&](auto uc, auto items_c, int kt, int tr) {
            constexpr int u = decltype(uc)::value;
            constexpr bool ITEMS = PEERS && decltype(items_c)::value;
            uint8_t *cS = (u & 3) == 0 ? sS0 : (u & 3) == 1 ? sS1 : (u & 3) == 2 ? sS2 : sS3;
            uint8_t *nS = (u & 3) == 0 ? sS3 : (u & 3) == 1 ? sS0 : (u & 3) == 2 ? sS1 : sS2;
            uint8_t *cA = cS, *nA = nS, *nB = nS + A_BYTES;
            uint8_t *sl = (u & 1) ? sP1 : sP0;
            // ---- M(kt) ----
            barrier_only();
            bf16x8_t fa[FN], fb[FMt];
            read_frags(cA, fa, fb);
            dma_stage(kt + 3, nA, nB);
            if constexpr (ITEMS) {
                // Item kt was issued in M(kt-2); after it came stage
                // kt+2, item kt+1 and stage kt+3.
                wait_vmcnt<2 * DMA_PER_STEP + PEER_PER_ITEM>();
                if (u < FMt && kt >= wlo && kt < whi) {
                    u32x2_t pv[FN];
                    const uint32_t pb = opaque(lds_addr(sl)) + wave * PSLOT;
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        pv[j] = *lds_ptr<u32x2_t>(pb + (pc_off ^ (uint32_t)(32 * j)));
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[u % FMt][j] += unpack_bf16x4(pv[j]);
                }
                wait_lgkmcnt0();  // slot read back before it is refilled
                peer_dma(sl, kt + 2, (u + 2) & 7, pd_off, pd_n);
                wait_vmcnt<AFTER>();  // own loads of stage kt+1 done
            } else if constexpr (PEERS) {
                if (tr == 0)
                    wait_vmcnt<2 * DMA_PER_STEP + 2 * PEER_PER_ITEM>();
                else if (tr == 1)
                    wait_vmcnt<2 * DMA_PER_STEP + PEER_PER_ITEM>();
                else
                    wait_vmcnt<2 * DMA_PER_STEP>();
            } else {
                wait_vmcnt<AFTER>();
            }
            wait_lgkmcnt0();      // stage kt fully read into registers
            // ---- C(kt) ----
            barrier_only();
            mfmas(fa, fb);
        };
        const int E = PEERS ? min(g1, g0 + ((max(whi - g0, 0) + 7) & ~7)) : g0;
        for (int kt0 = g0; kt0 < E; kt0 += 8)
            unroll8([&](auto uc) {
                const int kt = kt0 + decltype(uc)::value;
                if (kt < E)
                    step(uc, std::true_type{}, kt, 0);
            });
        for (int kt0 = E; kt0 < g1; kt0 += 8) {
            const bool first = kt0 == E;
            unroll8([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                const int kt = kt0 + u;
                if (kt < g1)
                    step(uc, std::false_type{}, kt, first ? (u < 2 ? u : 2) : 2);
            });
        }
        if (!lag)
            barrier_only();           // same barrier count in both groups

        // Lane offsets for the rest of the segment, recomputed (see opaque_v).
        const int ln = opaque_v(lane);
        const int fi2 = ln & 15, fg2 = ln >> 4;
        const int pm_base2 = m0 + wm * WMt + fi2;

        // ---- split tile: exchange partials, finish the tile in shares ----
        // Each wave's 4*FMt accumulator blocks form NSEG = 2*FMt segments,
        // row block i and column half h (blocks (i, 2h) and (i, 2h+1)); share
        // k of a tile's q units is segments [NSEG*k/q, NSEG*(k+1)/q) (empty
        // for some k when q > NSEG).  Every unit stores its whole
        // fp32 partial, raises its flag and counts itself in on the tile's
        // arrival counter.  A unit that is not the last to arrive waits a
        // short, bounded time for the other units' flags; if they all come,
        // it claims its own share.  The last to arrive (every partial is then
        // stored) claims its own share, gives the other units a short time
        // to claim theirs, and claims those still unclaimed.  A unit then
        // finishes the shares it holds: it adds the other units' copies of
        // their segments and stores them.  A share is claimed by a
        // compare-and-swap of its word to the launch epoch, so exactly one
        // unit finishes it.  Nobody waits without bound for a unit that has
        // not arrived, so the scheme completes whatever the order in which
        // workgroups get a CU; when they run at once, a tile's reduction is
        // spread over all of its units, none of which reads more than about
        // 1/q of each of the other partials.
        // A partial is kept in accumulator order (wave, block, lane), 16
        // bytes per lane per block, so every access is a full 1 KiB per wave.
        uint32_t smask = (1u << (2 * FMt)) - 1u;   // segments to finish: all, for a whole tile
        if constexpr (SPLIT) {
            const int u = __builtin_amdgcn_readfirstlane(cur_unit());
            const int sc = __builtin_amdgcn_readfirstlane(u / p.sk_tiles);
            const int stt = u - sc * p.sk_tiles;
            const int nq = p.sk_q;
            const uint32_t lane16 = (uint32_t)ln * 16u;
            const uint32_t wave_off = (uint32_t)(wave * FMt * FN * 1024);
            // The partial slots, as one buffer over the whole region: an
            // offset past the last slot stores nothing and loads zeros.
            const uint32_t part_region = (uint32_t)p.sk_slots * PART_BYTES;
            if (!bad) {
                const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.sk_part, part_region);
                const uint32_t vo = lane16 + (uint32_t)u * PART_BYTES;
#pragma unroll
                for (int i = 0; i < FMt; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(u32x4_t, acc[i][j]), rp, (int)vo,
                            (int)(wave_off + (uint32_t)((i * FN + j) * 1024)), CPOL_SYS);
            }
            signal_partial(bad ? 0u : 1u);
            // Wave 0 counts the unit in, watches the other units' flags and
            // claim words (one lane per unit) and claims; the verdict goes to
            // every wave through the first word of stage 0 (every wave's
            // stage loads have landed and its stage reads are done:
            // signal_partial waited for them).
            int *cell = (int *)sS0;
            if (wave == 0) {
                int n = 0;
                if (lane == 0) {
                    unsigned long long *ctr = p.sk_count + stt;
                    unsigned long long cur =
                        __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    unsigned long long nxt;
                    for (;;) {
                        nxt = (uint32_t)(cur >> 32) == p.sk_epoch
                                  ? cur + 1
                                  : ((unsigned long long)p.sk_epoch << 32) | 1ull;
                        if (__hip_atomic_compare_exchange_strong(ctr, &cur, nxt, __ATOMIC_RELAXED,
                                                                 __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_SYSTEM))
                            break;
                    }
                    n = (int)(uint32_t)nxt;
                }
                const bool lst = __builtin_amdgcn_readlane(n, 0) >= nq;
                const bool act = lane < nq - 1;
                const int cp = lane < sc ? lane : lane + 1;
                const uint32_t *fl = p.sk_flags + 2 * (act ? cp * p.sk_tiles + stt : 0);
                // The last unit finds every flag raised; the limit there is
                // only a guard.
                const uint32_t limit = lst ? p.sk_max_spins : p.sk_wait_spins;
                bool done = !act, valid = true;
                uint32_t spins = 0;
                for (;;) {
                    if (!done) {
                        const uint32_t f = __hip_atomic_load(fl, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_SYSTEM);
                        if ((int32_t)(f - p.sk_epoch) >= 0) {
                            done = true;
                            valid = __hip_atomic_load(fl + 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_SYSTEM) != 0;
                        }
                    }
                    if (__builtin_amdgcn_ballot_w64(!done) == 0)
                        break;
                    if (++spins >= limit) {
                        if (lst && lane == 0 && p.status)
                            atomicCAS(p.status, 0, 1000 + 16);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                const bool all = __builtin_amdgcn_ballot_w64(!(done && valid)) == 0 && !bad;
                // Claims: lane k acts for share k.
                uint32_t *cw = p.sk_claim + stt * 16 + (lane < nq ? lane : 0);
                auto claim = [&](bool want) {
                    bool got = false;
                    if (want) {
                        uint32_t cur = __hip_atomic_load(cw, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_SYSTEM);
                        got = cur != p.sk_epoch &&
                              __hip_atomic_compare_exchange_strong(cw, &cur, p.sk_epoch,
                                                                   __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                                   __HIP_MEMORY_SCOPE_SYSTEM);
                    }
                    return __builtin_amdgcn_ballot_w64(got);
                };
                uint64_t won = all ? claim(lane == sc) : 0;
                if (all && lst) {
                    // Give the other units a short time to claim their shares.
                    bool settled = !(lane < nq && lane != sc);
                    uint32_t gspins = 0;
                    for (;;) {
                        if (!settled)
                            settled = __hip_atomic_load(cw, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_SYSTEM) == p.sk_epoch;
                        if (__builtin_amdgcn_ballot_w64(!settled) == 0 || ++gspins >= p.sk_grace_spins)
                            break;
                        __builtin_amdgcn_s_sleep(2);
                    }
                    won |= claim(!settled);
                }
                uint32_t m = 0;
                for (int k = 0; k < nq; ++k)
                    if ((won >> k) & 1u)
                        m |= (1u << (NSEG * (k + 1) / nq)) - (1u << (NSEG * k / nq));
                if (lane == 0)
                    *cell = (int)m;
            }
            __syncthreads();
            smask = (uint32_t)__builtin_amdgcn_readfirstlane(*cell);
            __syncthreads();
            if (smask == 0)
                continue;              // nothing to finish here
            // Add the other units' copies of the segments in smask: items t =
            // (unit t / ns, t % ns-th segment of smask) of 2 KiB per wave,
            // through a ring of eight 2 KiB slots in the wave's 16 KiB of the
            // idle stages, DEPTH items in flight.  Items past the end are
            // loads out of range (they fill their slot with zeros).
            const int ns = __builtin_popcount(smask);
            const int T = (nq - 1) * ns;
            const uint8_t *wst = (wave >> 1) == 0 ? sS0 : (wave >> 1) == 1 ? sS1
                               : (wave >> 1) == 2 ? sS2 : sS3;
            const uint32_t ring = lds_addr(wst) + (uint32_t)((wave & 1) * 16384);
            auto seg_of = [&](int k) {     // k-th segment (from 0) of smask
                uint32_t mm = smask;
                for (int r = 0; r < k; ++r)
                    mm &= mm - 1u;
                return __builtin_ctz(mm);
            };
            constexpr int DEPTH = 6;
            const u32x4_t rpart = make_rsrc4(p.sk_part, part_region);
            auto issue = [&](int t) {
                const int pc = t / ns;
                const int cp = pc < sc ? pc : pc + 1;
                const int sg = seg_of(t - pc * ns);
                const uint32_t vo =
                    t < T ? lane16 + (uint32_t)(cp * p.sk_tiles + stt) * PART_BYTES : OOB;
                const uint32_t slot = ring + (uint32_t)((t & 7) * 2048);
                const uint32_t so = wave_off + (uint32_t)(sg * 2048);
                dma16_sys(rpart, slot, vo, so);
                dma16_sys(rpart, slot + 1024u, vo, so + 1024u);
            };
#pragma unroll
            for (int t = 0; t < DEPTH; ++t)
                issue(t);
            for (int t = 0; t < T; ++t) {
                wait_vmcnt<2 * (DEPTH - 1)>();   // item t landed
                const uint32_t slot = ring + (uint32_t)((t & 7) * 2048);
                const u32x4_t x0 = *lds_ptr<u32x4_t>(slot + lane16);
                const u32x4_t x1 = *lds_ptr<u32x4_t>(slot + 1024u + lane16);
                wait_lgkmcnt0();
                const int sg = seg_of(t % ns);
#pragma unroll
                for (int s2 = 0; s2 < NSEG; ++s2)
                    if (sg == s2) {
                        acc[s2 >> 1][2 * (s2 & 1)] += __builtin_bit_cast(f32x4_t, x0);
                        acc[s2 >> 1][2 * (s2 & 1) + 1] += __builtin_bit_cast(f32x4_t, x1);
                    }
                issue(t + DEPTH);
            }
            wait_vmcnt<0>();
        }

        // ---- peer items the K loop did not reach ----
        // (K shorter than the 8 * npeers item steps.)  The K loop is over, so
        // each wave streams them through its 16 KiB of the idle LDS stages,
        // once every wave's stage loads have landed and its stage reads are
        // done: half-groups of 4 items (row blocks 0-3 or 4-7 of a group of
        // 8), the next half-group loading while one is added.  Every
        // half-group issues the same 8 loads; items outside the window read
        // an empty range, so they add zeros.
        // (A split launch has every item inside the K loop: the host splits
        // only when 8 * npeers <= KT.)
        if (!SPLIT && PEERS && W > KT) {
            wait_vmcnt<0>();
            barrier_only();
            wlo = KT;
            whi = W;
            const int pd_n2 = n0 + wn * WN + 8 * ((ln & 7) ^ ((ln >> 4) & 3));
            const uint32_t pd_off2 = (uint32_t)(ln >> 3) * N2 + (uint32_t)pd_n2 * 2u;
            const uint32_t pc_off2 = (uint32_t)(fi2 * 128 + 8 * (fg2 & 1) +
                                                16 * ((fg2 >> 1) ^ ((fi2 >> 1) & 1)) + 32 * ((fi2 >> 2) & 3));
            const uint8_t *wst = (wave >> 1) == 0 ? sS0 : (wave >> 1) == 1 ? sS1
                               : (wave >> 1) == 2 ? sS2 : sS3;
            const uint32_t reg = lds_addr(wst) + (uint32_t)((wave & 1) * 16384);
            const int g_first = KT & ~7;
            const int nh = 2 * ((W - g_first + 7) / 8);   // half-groups, an even count
            // half-group k: items g_first + 8 (k/2) + 4 (k%2) + r, row block
            // 4 (k%2) + r, into slot 4 (k%2) + r
            auto issue_half = [&](int k, int h) {
                const int wb = g_first + 8 * (k >> 1) + 4 * h;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    peer_dma_at(reg + (uint32_t)((4 * h + r) * PSLOT), wb + r, 4 * h + r, pd_off2,
                                pd_n2);
            };
            auto add_half = [&](int h) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * h + r;
                    if (i < FMt) {
                        u32x2_t pv[FN];
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            pv[j] = *lds_ptr<u32x2_t>(reg + (uint32_t)(i * PSLOT) +
                                                      (pc_off2 ^ (uint32_t)(32 * j)));
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[i][j] += unpack_bf16x4(pv[j]);
                    }
                }
                wait_lgkmcnt0();      // read back before the slots refill
            };
            issue_half(0, 0);
            issue_half(1, 1);
            for (int k = 0; k < nh; k += 2) {
                wait_vmcnt<8>();      // half-group k landed (k+1 may be in flight)
                add_half(0);
                issue_half(k + 2, 0);
                wait_vmcnt<8>();      // half-group k+1 landed
                add_half(1);
                issue_half(k + 3, 1);
            }
            wait_vmcnt<0>();          // the two half-groups past the end
        }

        // ---- epilogue: bf16 stores, 16 bytes per lane per pair of blocks ----
        // (of the owned segments only: in a split tile, the other units
        // store the rest; a segment is a pair of blocks, so a pair is owned
        // or not as a whole)
        auto own = [&](int i, int j) { return ((smask >> (2 * i + (j >> 1))) & 1u) != 0; };
        // first column of the lane's 8 in a pair of blocks (see pack_pair)
        const int pn16 = n0 + wn * WN + 8 * (fg2 >> 1) + 16 * (fg2 & 1);
        if (MODE == MODE_RS) {
            // Two-shot AR: out is [M][N] (slice rows at their own index, rows
            // past M not stored) and the slice rows also go to every peer
            // output; plain RS: out is the [P][N] slice.
            const bool two = p.peer_out != nullptr;
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out, (uint32_t)(two ? p.M : p.P) * N2);
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.ws, (uint32_t)p.M * N2);
            const int s0 = p.rank * p.P;   // first global row of the slice
#pragma unroll
            for (int i = 0; i < FMt; ++i) {
                const int m = pm_base2 + 16 * i;
                const bool in_slice = m >= s0 && m < s0 + p.P;
                const bool to_ws = !in_slice && m < p.M;
                const uint32_t rbase = (uint32_t)(in_slice ? m - s0 : m) * N2 + (uint32_t)pn16 * 2u;
                // The 16 rows of the block (uniform): all in the slice, all
                // outside it, or straddling its edge (both stores, masked).
                const int blk = m0 + wm * WMt + 16 * i;
                const bool any_out = blk < s0 || blk + 16 > s0 + p.P;
                const bool any_in = blk + 16 > s0 && blk < s0 + p.P;
                const bool slice_st = in_slice && (!two || m < p.M);
                const uint32_t obase = two ? (uint32_t)m * N2 + (uint32_t)pn16 * 2u : rbase;
                u32x4_t pk[FN / 2];
#pragma unroll
                for (int h = 0; h < FN / 2; ++h)
                    pk[h] = pack_pair(acc[i][2 * h], acc[i][2 * h + 1]);
#pragma unroll
                for (int h = 0; h < FN / 2; ++h) {
                    const bool ok = pn16 + 32 * h < p.N && own(i, 2 * h);
                    if (any_in)
                        store16(ro, (ok && slice_st) ? obase + 64u * h : OOB, pk[h]);
                    if (any_out)
                        store16(rw, (ok && to_ws) ? rbase + 64u * h : OOB, pk[h]);
                }
                if (two && any_in) {
                    for (int q = 0; q < p.npeers; ++q) {
                        const __amdgpu_buffer_rsrc_t rq =
                            make_rsrc(p.peer_out + (size_t)q * p.M * p.N, (uint32_t)p.M * N2);
#pragma unroll
                        for (int h = 0; h < FN / 2; ++h) {
                            const bool ok = pn16 + 32 * h < p.N && own(i, 2 * h);
                            store16(rq, (ok && slice_st) ? obase + 64u * h : OOB, pk[h]);
                        }
                    }
                }
            }
        } else {
            uint16_t *ob = p.out + (MODE == MODE_AG ? (size_t)q * p.M * p.N : 0);
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(ob, (uint32_t)p.M * N2);
#pragma unroll
            for (int i = 0; i < FMt; ++i) {
                const int m = pm_base2 + 16 * i;
                const uint32_t rbase = (uint32_t)m * N2 + (uint32_t)pn16 * 2u;
#pragma unroll
                for (int h = 0; h < FN / 2; ++h) {
                    const bool ok = m < p.M && pn16 + 32 * h < p.N && own(i, 2 * h);
                    store16(ro, ok ? rbase + 64u * h : OOB, pack_pair(acc[i][2 * h], acc[i][2 * h + 1]));
                }
            }
        }
    }
}

}  // namespace gc
