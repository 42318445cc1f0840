/*
 * gemm_coll.h -- fused tensor-parallel BF16 GEMM + cross-rank reduction for
 * AMD MI355X (gfx950).
 *
 * One rank's share of a tensor-parallel projection: the BF16 GEMM and the
 * reduction or gather that tensor parallelism wraps around it, in one kernel.
 *
 *   gemm_ar   GEMM-AR: the local fp32 accumulator plus every other rank's
 *             partial; every rank gets the full sum ("[Kimi-K3] Extend GEMM-RS
 *             to GEMM-AR", 功能与动机 and 实现拆解 step 1; test reference,
 *             all_reduce branch, in 关键源码片段).
 *   gemm_rs   GEMM-RS: the same sum, but this rank keeps only its own row
 *             slice (same page, 实现拆解 step 1 and the reduce_scatter branch
 *             of the test reference).
 *   gemm_ar_two_shot
 *             GEMM-AR by the pages' own data flow: each rank reduces its row
 *             slice over the peers' partials and stores the reduced slice
 *             into every rank's output (same page, 实现拆解 step 1: the
 *             owner's local_M slice, then the multicast store); here one
 *             rank's share, with the other ranks' outputs as local buffers.
 *   ag_gemm   AG-GEMM: the token shards of all ranks, concatenated along M,
 *             times B, with the shards consumed in ring order ("[Kimi-K3]
 *             AG-GEMM for Sequence Parallelism", Purpose and Implementation
 *             details).
 *   ag_push_shards
 *             the other ranks' side of AG-GEMM, emulated: DMA-engine copies
 *             of their shards into ag_gemm's receive buffer, each followed
 *             by its ready flag, in ring order (same page).
 *
 * The other ranks are represented by buffers in this GPU's memory (their
 * partial products, or their shards); nothing here moves data between GPUs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Element type: gc_bf16 holds the raw bits of an IEEE bfloat16 (the upper
 *   16 bits of a binary32).  Products accumulate in fp32; the single rounding
 *   to bf16 is round-to-nearest-even.
 * - Layouts are dense row-major: A [M][K] (row stride K), B [K][N] (row stride
 *   N; the pages store the weight as [N][K] and use its transpose, so B is
 *   that transpose), outputs [rows][N].
 * - All data pointers are device pointers on the current HIP device, 16-byte
 *   aligned; N and K must be multiples of 8 (rows are whole 16-byte vectors).
 *   With K = 0 the operands that hold no element (A, B, AG's shards) may be
 *   NULL.
 * - R, the tensor-parallel size, must satisfy 1 < R <= 16 and 128 % R == 0,
 *   i.e. R in {2, 4, 8, 16} (the validation chain of maybe_init_gemm_rs_ar,
 *   "[Kimi-K3] Extend GEMM-RS to GEMM-AR", 关键源码片段); 0 <= rank < R.
 * - Ownership: the caller owns every buffer, including the optional
 *   workspace.  The library allocates no device memory and never
 *   synchronizes.  Its only mutable state is a per-device cache of the
 *   compute-unit count and a per-device launch counter (an atomic that
 *   stamps each split launch with a new epoch, so that the workspace's
 *   counters, flags and claim words are never reset); calls are thread-safe,
 *   but a workspace serves one call at a time: two calls in flight at once
 *   (on different streams) need two workspaces.  Work is enqueued on
 *   `stream` (a hipStream_t; NULL = the null stream) and is complete only
 *   when that stream is.  Outputs must not alias any input.
 * - Errors: a negative return means nothing was launched.
 *     GC_EINVAL   a NULL or misaligned pointer, R or rank out of range,
 *                 a negative size, N or K not a multiple of 8
 *     GC_ENOTSUP  a shape this kernel set cannot address (a buffer of 2 GiB
 *                 or more, or a size above INT32_MAX)
 *     GC_EIO      the HIP launch failed
 *     GC_ENOSPC   gemm_ar_noalloc only: its static scratch is too small for
 *                 the device
 *   M == 0 (or N == 0) is valid and launches nothing.
 * - K-split hand-over: the workgroups sharing a split tile wait for one
 *   another only a bounded time, and the last of them to finish its part of
 *   the K loop completes whatever share of the tile the others did not
 *   claim, so no call can deadlock whatever the order in which workgroups
 *   get a compute unit.  If that last workgroup's own (guard) wait gives up,
 *   the tile is left unwritten and, when peers->status is not NULL, *status
 *   is set to GC_TIMEOUT_BASE + 16.  (For tests, gc_peers.split_wait_spins
 *   sets how long the other workgroups wait before leaving their share to
 *   the last one.)  The split state lives in the workspace (one slot per
 *   compute unit); a launch never indexes past it: the host plans at most
 *   one split unit per slot, and the kernel checks this again and does no
 *   work (status GC_TIMEOUT_BASE + 16) if it ever did not hold.
 *
 * gemm_coll_peer_sum is not a fused path: it is the reduction step of the
 * unfused baseline (a library GEMM, then this kernel) that the fused entry
 * points are measured against.
 */
#ifndef GEMM_COLL_H
#define GEMM_COLL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t gc_bf16;

#define GC_OK 0
#define GC_EINVAL (-22)
#define GC_ENOTSUP (-95)
#define GC_EIO (-5)
#define GC_ENOSPC (-28)
/* AG-GEMM reports a shard whose ready flag never came as *status = GC_TIMEOUT_BASE + q. */
#define GC_TIMEOUT_BASE 1000

/*
 * Where the other ranks' data lives.  Fields a call does not use are ignored.
 */
typedef struct gc_peers {
    /* gemm_ar / gemm_rs: [R-1][M][N] partial products of the other ranks.
       Slot p holds rank (p < rank ? p : p + 1): ascending rank order, this
       rank skipped. */
    const gc_bf16 *partials;
    /* gemm_rs: [M][N] this rank's published partial (see gemm_rs). */
    gc_bf16 *ws;
    /* ag_gemm: [R][Ms][K] every rank's shard; slot `rank` is not read. */
    const gc_bf16 *shards;
    /* ag_gemm: [R] ready flags (4-byte aligned device memory); shard q is
       ready when (int32_t)(flags[q] - epoch) >= 0.  Flags are never reset:
       each call passes a larger epoch.  flags[rank] is not read. */
    const uint32_t *flags;
    uint32_t epoch;
    /* Device int32, written only on a time-out: required by ag_gemm (see
       there), optional (may be NULL) for gemm_ar / gemm_rs. */
    int32_t *status;
    /* ag_gemm: polls of one flag before giving up; 0 = the default
       (about one second). */
    uint32_t max_spins;
    /* All calls, optional: device workspace of at least
       gemm_coll_workspace_bytes() bytes (about 64 MiB on MI355X),
       zero-filled before its first use and not used by two calls at the
       same time.  With it, a problem with fewer 256 x 256 output tiles than
       compute units has its tiles split along K into chunks run by
       different workgroups (fp32 partial sums exchanged through it); with
       NULL, or with a full round of tiles or more, every tile is computed
       whole.  Results agree to rounding of the fp32 partial sums. */
    void *workspace;
    uint64_t workspace_bytes;
    /* All calls, optional: output tile height in rows, 0 = chosen per
       problem (64 for at most 64 rows per shard, 128 for at most 128, else
       256, or 224 where that gives the workgroups less work); 64, 128, 224
       or 256 = forced; any other value is GC_EINVAL.  Results agree to
       rounding of the fp32 sums (the peer partials are added at different
       K-steps).  224-row tiles are never split along K. */
    uint32_t tile_rows;
    /* gemm_ar_two_shot: [R-1][M][N] stand-ins for the other ranks' outputs,
       slot p for rank (p < rank ? p : p + 1); receives this rank's reduced
       slice rows (see gemm_ar_two_shot).  Ignored by the other calls. */
    gc_bf16 *peer_out;
    /* For tests of the K-split hand-over, optional: 0 = the default; n > 0 =
       the workgroups sharing a split tile wait only n polls for one another
       before leaving their share to the last of them (see "K-split
       hand-over" above).  Results do not change. */
    uint32_t split_wait_spins;
} gc_peers;

/*
 * GEMM-AR.
 *   out[i][j] = bf16( sum_k A[i][k] * B[k][j] + sum_p partials[p][i][j] ),
 *   for all i < M, j < N; the GEMM accumulates in fp32 and the peer partials
 *   are added in fp32 before the one rounding.
 * A [M][K], B [K][N], peers->partials [R-1][M][N], out [M][N] (caller-owned:
 * unlike the pages' symmetric-memory workspace, nothing is reused between
 * calls, so an earlier result stays valid).
 */
int gemm_ar(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R, int rank,
            const gc_peers *peers, gc_bf16 *out, void *stream);

/*
 * GEMM-AR that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, result and
 * launches as gemm_ar; peers->workspace and peers->workspace_bytes are
 * ignored.  In their place the K-split state (arrival counters, claim words,
 * flags and fp32 partial tiles) lives in a static device array of the
 * library, 64 MiB + 20 KiB: the workspace for up to 256 compute units, one
 * copy per device, zero at load and held until the process ends.  No
 * problem size needs more; on a device with more than 256 compute units the
 * call returns GC_ENOSPC and launches nothing.  Nothing is cleared between
 * calls: every launch stamps its counters, flags and claims with a new
 * epoch, so the state a previous call left behind is never mistaken for
 * this call's.  All calls on one device share its array: two such calls in
 * flight at the same time (on different streams, or from different host
 * threads) race on it and may return wrong results; serialize them.  The
 * first call on a device looks up the array's device address (no
 * allocation); later calls only launch kernels.
 */
int gemm_ar_noalloc(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R,
                    int rank, const gc_peers *peers, gc_bf16 *out, void *stream);

/*
 * GEMM-RS.  P = ceil(M/R); rank r owns global rows [r*P, (r+1)*P) (the pages'
 * reference pads the partial to P*R rows and reduce-scatters it).
 *   out [P][N]: out[t] = bf16(A[r*P+t].B + sum_p partials[p][r*P+t]) when
 *               r*P + t < M, and 0 for the padding rows past M;
 *   peers->ws [M][N] (required): every row i < M that this rank does not own
 *               receives bf16(A[i].B), its own partial, which the owning rank
 *               would reduce; the owned rows of ws are left untouched.
 * peers->partials [R-1][M][N] is read only on the owned rows.
 */
int gemm_rs(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R, int rank,
            const gc_peers *peers, gc_bf16 *out, void *stream);

/*
 * GEMM-AR, two-shot: this rank's part of the pages' GEMM-AR data flow.
 * Everything gemm_rs does (same P, slice and peers->ws), except that the
 * reduced slice rows go to a full-height output and to every peer output:
 *   out [M][N]: rows i in [r*P, min((r+1)*P, M)) receive
 *               bf16(A[i].B + sum_p partials[p][i]); the other rows are left
 *               untouched (their owners store them);
 *   peers->peer_out [R-1][M][N] (required): the same rows receive the same
 *               values in every slot, standing in for the stores into the
 *               other ranks' outputs (the pages' multicast store; unicast
 *               stores over xGMI on MI355X); other rows untouched;
 *   peers->ws [M][N] (required): as gemm_rs.
 * peers->partials [R-1][M][N] is read only on the owned rows.
 */
int gemm_ar_two_shot(const gc_bf16 *A, const gc_bf16 *B, int64_t M, int64_t N, int64_t K, int R,
                     int rank, const gc_peers *peers, gc_bf16 *out, void *stream);

/*
 * AG-GEMM.  Shard q has Ms rows; the global activation is the concatenation
 * of the R shards, and
 *   out[q*Ms + t][j] = bf16( sum_k S_q[t][k] * B[k][j] ),
 * with S_rank = A (this rank's shard) and S_q = peers->shards[q] otherwise.
 * One persistent kernel takes the shards in ring order q = rank, rank-1, ...
 * (mod R): the local shard first, then each shard as it would arrive from
 * the previous rank.  Before the first K-step of a tile of shard q != rank it
 * polls flags[q] (system-scope acquire) until the shard is ready.  A shard
 * still not ready after max_spins polls is skipped: its output rows are left
 * unwritten and *status is set to GC_TIMEOUT_BASE + q (the first such shard
 * wins).  Once *status is non-zero, a tile whose shard is not ready is
 * skipped at its first poll, without waiting, so a launch whose producer has
 * stalled ends after about one waiting period.  *status is otherwise never
 * written: the caller clears it (a non-zero *status at the start of a call
 * makes that call skip, rather than wait for, any shard not yet ready).
 * A [Ms][K], peers->shards [R][Ms][K], flags [R], status, out [R*Ms][N].
 */
int ag_gemm(const gc_bf16 *A, const gc_bf16 *B, int64_t Ms, int64_t N, int64_t K, int R, int rank,
            const gc_peers *peers, gc_bf16 *out, void *stream);

/*
 * Dispatch gate: 1 if the fused path should be used for M tokens, else 0.
 * The fused kernels are slower than the unfused path for M < 128 ("[Kimi-K3]
 * Extend GEMM-RS to GEMM-AR", 实现拆解 step 3 and 风险与影响), so callers use
 * their unfused GEMM there.  The entry points themselves run any M >= 0.
 */
int gemm_coll_should_run(int64_t M);

/* Launch plan that a call with these arguments makes (host arithmetic only:
 * no device is touched, so it also runs without a GPU), for tests and for
 * callers that want to see the tiling.  `mode` is GC_MODE_AR, GC_MODE_RS
 * (also gemm_ar_two_shot) or GC_MODE_AG (M is then Ms, the shard rows);
 * `cus` the device's compute units (256 on MI355X); `with_workspace` whether
 * the call passes a large enough gc_peers.workspace; `tile_rows` as in
 * gc_peers.  Tiles are numbered shard-major (AG), then in groups of row
 * tiles; the first whole_tiles run whole, the split_tiles after them are cut
 * along K into `chunks` chunks of chunk_steps K-steps of 32 (the last chunk
 * may be shorter), one workgroup per (chunk, tile) unit.  GC_EINVAL for
 * arguments the entry points would refuse (and for `plan` NULL, `mode` out
 * of range or `cus` outside 1 .. 4096), GC_ENOTSUP likewise; M or N == 0
 * gives an empty plan (tiles 0). */
#define GC_MODE_AR 0
#define GC_MODE_RS 1
#define GC_MODE_AG 2
typedef struct gc_plan {
    uint32_t tile_rows;   /* 64, 128, 224 or 256 */
    int32_t tiles;        /* output tiles (over all shards for AG) */
    int32_t whole_tiles;  /* tiles computed whole, in rounds of `grid` */
    int32_t split_tiles;  /* tiles split along K after them (0: none) */
    int32_t chunks;       /* K chunks per split tile (0: none) */
    int32_t chunk_steps;  /* K-steps per chunk, a multiple of 8 (0: none) */
    int32_t units;        /* split_tiles * chunks, one workgroup each */
    int32_t grid;         /* workgroups of the last launch */
    int32_t peer_nt;      /* peer partials loaded non-temporal */
} gc_plan;
int gemm_coll_plan(int mode, int64_t M, int64_t N, int64_t K, int R, int rank, int cus,
                   int with_workspace, uint32_t tile_rows, gc_plan *plan);

/* Bytes of workspace that lets a call split tiles along K on the current
 * device (see gc_peers.workspace); negative on a HIP error. */
int64_t gemm_coll_workspace_bytes(void);

/* Static description of a return code (never NULL). */
const char *gemm_coll_strerror(int code);

/* AG-GEMM's producer side, emulated on one GPU: enqueues on `stream`, in
 * ring order (round s = 1 .. R-1 brings shard q = (rank - s) mod R, the
 * order in which ag_gemm consumes them), a copy of shard q from src into
 * dst followed by a 4-byte copy of *epoch_word into flags[q], all through
 * the DMA engines, so that they make progress while an ag_gemm launched on
 * another stream holds every compute unit and polls those flags ("[Kimi-K3]
 * AG-GEMM for Sequence Parallelism", Implementation details: the copy
 * engine pushes one shard per round and then signals its receiver).  On one
 * GPU the other ranks' shards are src; dst is ag_gemm's peers->shards.
 *   src, dst    [R][Ms][K] bf16, 16-byte aligned, not overlapping; slot
 *               `rank` of dst is neither read nor written.
 *   flags       [R] uint32, 4-byte aligned (ag_gemm's peers->flags).
 *   epoch_word  device pointer to the uint32 epoch to raise the flags to
 *               (ag_gemm's peers->epoch), read by each flag copy.
 * R and rank as for the other entry points.  GC_EINVAL for a NULL or
 * misaligned pointer or R, rank or a size out of range; GC_EIO if a copy
 * cannot be enqueued (earlier rounds may then already be enqueued). */
int ag_push_shards(const gc_bf16 *src, gc_bf16 *dst, int64_t Ms, int64_t K, int R, int rank,
                   uint32_t *flags, const uint32_t *epoch_word, void *stream);

/* Unfused baseline, reduction step: out = bf16(local + the sum of npeers
 * peer blocks), elementwise over rows x N, summed in fp32 in the order local,
 * peer 0, ..., peer npeers-1 and rounded to nearest-even once.  After a
 * library GEMM has written local = bf16(A.B), this is the unfused reference
 * of "[Kimi-K3] Extend GEMM-RS to GEMM-AR" (test reference in 关键源码片段:
 * the local matmul rounded to bf16, then the all-reduce) on one GPU.
 *   local, out  [rows][N] dense; out may equal local, and must not overlap
 *               the peer blocks otherwise.
 *   partials    npeers blocks of [rows][N], block p starting p * peer_stride
 *               elements after block 0 (a row slice [lo, hi) of [R-1][M][N]
 *               partials: partials + lo*N with peer_stride = M*N).
 * Pointers 16-byte aligned; peer_stride a multiple of 8, and >= rows*N when
 * npeers > 1; 0 <= npeers <= 15.  GC_EINVAL otherwise, GC_EIO if the launch
 * fails; rows*N == 0 launches nothing.  Enqueued on `stream`. */
int gemm_coll_peer_sum(const gc_bf16 *local, const gc_bf16 *partials, int64_t rows, int64_t N,
                       int npeers, int64_t peer_stride, gc_bf16 *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_COLL_H */
