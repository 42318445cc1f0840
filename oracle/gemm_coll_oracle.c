/*
 * gemm_coll_oracle.c -- CPU oracle for the fused tensor-parallel BF16 GEMM +
 * reduction (GEMM-AR, GEMM-RS, AG-GEMM).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only in the seeded input generators.
 *
 * What it computes (the plain definitions, written out):
 *
 *   GEMM part:  G[i,j] = sum_{k=0}^{K-1} A[i,k] * B[k,j]
 *       A is [M,K] row-major, B is [K,N] row-major.  The pages' weight is
 *       [N,K] and is applied transposed ("weight.T" in the test reference of
 *       "[Kimi-K3] Extend GEMM-RS to GEMM-AR", section 关键源码片段); B here
 *       is that transpose, stored [K,N].
 *
 *   GEMM-AR:    out[i,j] = bf16( G[i,j] + sum_{p} peer_p[i,j] )   for i < M
 *       Every rank ends with the full cross-rank sum (the all_reduce branch
 *       of the test reference in "[Kimi-K3] Extend GEMM-RS to GEMM-AR").
 *
 *   GEMM-RS:    the partial is padded with zero rows to P*R rows,
 *       P = ceil(M/R), summed over ranks, and chunked; rank r receives rows
 *       [r*P, (r+1)*P) of the sum (the reduce_scatter branch of the same test
 *       reference: padded_M, reduce_scatter_single into padded_M/world_size
 *       rows).  Rows at or past M are the zero padding.  The rows this rank
 *       does not own keep its own partial, published as bf16(G) into ws.
 *
 *   AG-GEMM:    out[q*Ms + t, j] = bf16( sum_k S_q[t,k] * B[k,j] )
 *       i.e. one GEMM on the row-concatenation of the R shards ("[Kimi-K3]
 *       AG-GEMM for Sequence Parallelism", Purpose).  The ring order in which
 *       a kernel consumes the shards does not change the result.
 *
 * Arithmetic: every bf16 input is decoded exactly; the product of two bf16
 * values (8 significant bits each) is exact in binary32 and in binary64; the
 * sum runs in a fixed order (k ascending, then peers ascending) in one of two
 * precisions, chosen per call by `acc`:
 *   ORACLE_ACC_FP32  binary32 accumulator, each addition rounded to nearest
 *                    even: the fp32 accumulation over bf16 inputs that the
 *                    fused kernel's contract states (the default of the
 *                    Python front end);
 *   ORACLE_ACC_FP64  binary64 accumulator, nearly exact (for K and peer
 *                    counts of these sizes the error is far below a bf16
 *                    ulp), used to pin the fp32 one from outside.
 * The single rounding to bf16 is round-to-nearest-even of the accumulator
 * (IEEE 754 roundTiesToEven with an 8-bit significand and the binary32
 * exponent range).  The pages fix bf16 operands and a bf16 result but print
 * no accumulation precision for their reference.
 *
 * Rows are independent; OpenMP splits whole rows over threads, so the result
 * does not depend on the thread count.
 *
 * Planted-mistake builds (tests only): compiling with one of
 * -DORACLE_PLANT_{DROP_PEER,SKIP_LAST_K,SLICE_FLOOR,ROUND_TRUNC,AG_LOCAL_ONLY,
 * B_TRANSPOSED,WS_ALL_ROWS,ACC32_IN_DOUBLE,K_DESCENDING,PEERS_FIRST}
 * introduces one plausible mistake, so that the test suite can show that its
 * pins catch it.  The default build has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-22)
#define ORACLE_ENOMEM (-12)

/* accumulation precision (argument `acc` of the entry points) */
#define ORACLE_ACC_FP32 32
#define ORACLE_ACC_FP64 64

/* bf16 is the upper half of an IEEE binary32: decoding is a 16-bit shift. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_double(uint16_t h) { return bf16_to_double(h); }

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Round a double to the nearest bf16, ties to even.
 * bf16: sign, 8-bit exponent (binary32 range), 7 stored significand bits.
 * Normal numbers in [2^e, 2^(e+1)) have spacing 2^(e-7); below 2^-126 the
 * spacing stays 2^-133 (subnormals).  Halfway cases go to the neighbour with
 * an even last significand bit, which rint() does under the default rounding
 * mode.  Results at or above 2^128 overflow to infinity.
 */
uint16_t oracle_round_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    if (isinf(ax))
        return (uint16_t)(sign | 0x7F80);
    int ex;
    frexp(ax, &ex);              /* ax in [2^(ex-1), 2^ex) */
    int lead = ex - 1;           /* exponent of the leading bit */
    if (lead < -126)
        lead = -126;             /* subnormal range keeps the smallest spacing */
    int ulp_exp = lead - 7;
#ifdef ORACLE_PLANT_ROUND_TRUNC
    double q = trunc(ldexp(ax, -ulp_exp));
#else
    double q = rint(ldexp(ax, -ulp_exp)); /* exact scaling, then RNE */
#endif
    double y = ldexp(q, ulp_exp);
    if (y >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);
    float f = (float)y;          /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/*
 * One output row:
 *   out[j] = bf16( sum_{k<K} a[k]*B[k,j]  +  sum_{p<npeers} peer_p[j] )
 * a:      K bf16 values (one row of A)
 * B:      [K,N] row-major
 * peer_p: the row of peer p, at peer_rows + p*peer_stride
 * acc:    N accumulators of scratch (double or float, per `prec`)
 * The terms are added one at a time in the order written: k = 0, 1, ...,
 * K-1, then p = 0, 1, ..., npeers-1.  Each product a[k]*B[k,j] is exact in
 * either precision, so the only roundings are those of the additions (and
 * the final one to bf16).
 */
#ifdef ORACLE_PLANT_K_DESCENDING
#define K_INDEX(t, kend) ((kend) - 1 - (t))
#else
#define K_INDEX(t, kend) (t)
#endif

static void gemm_terms_f64(const uint16_t *a, const uint16_t *B, int64_t N, int64_t K, double *acc)
{
    int64_t kend = K;
#ifdef ORACLE_PLANT_SKIP_LAST_K
    if (kend > 0)
        kend -= 1;
#endif
    for (int64_t t = 0; t < kend; ++t) {
        int64_t k = K_INDEX(t, kend);
        double av = bf16_to_double(a[k]);
#ifdef ORACLE_PLANT_B_TRANSPOSED
        /* reads B as if it were [N,K]: only meaningful when K == N */
        for (int64_t j = 0; j < N; ++j)
            acc[j] += av * bf16_to_double(B[j * K + k]);
#else
        const uint16_t *brow = B + k * N;
        for (int64_t j = 0; j < N; ++j)
            acc[j] += av * bf16_to_double(brow[j]);
#endif
    }
}

static void gemm_terms_f32(const uint16_t *a, const uint16_t *B, int64_t N, int64_t K, float *acc)
{
    int64_t kend = K;
#ifdef ORACLE_PLANT_SKIP_LAST_K
    if (kend > 0)
        kend -= 1;
#endif
    for (int64_t t = 0; t < kend; ++t) {
        int64_t k = K_INDEX(t, kend);
        float av = bf16_to_float(a[k]);
#ifdef ORACLE_PLANT_B_TRANSPOSED
        for (int64_t j = 0; j < N; ++j)
            acc[j] += av * bf16_to_float(B[j * K + k]);
#else
        const uint16_t *brow = B + k * N;
        for (int64_t j = 0; j < N; ++j)
            acc[j] += av * bf16_to_float(brow[j]);
#endif
    }
}

static void oracle_row(const uint16_t *a, const uint16_t *B, const uint16_t *peer_rows,
                       int64_t peer_stride, int npeers, int64_t N, int64_t K, int prec,
                       void *scratch, uint16_t *out)
{
    int np = npeers;
#ifdef ORACLE_PLANT_DROP_PEER
    if (np > 0)
        np -= 1;
#endif
#ifdef ORACLE_PLANT_ACC32_IN_DOUBLE
    prec = ORACLE_ACC_FP64;
#endif
    if (prec == ORACLE_ACC_FP64) {
        double *acc = (double *)scratch;
        for (int64_t j = 0; j < N; ++j)
            acc[j] = 0.0;
#ifndef ORACLE_PLANT_PEERS_FIRST
        gemm_terms_f64(a, B, N, K, acc);
#endif
        for (int p = 0; p < np; ++p) {
            const uint16_t *prow = peer_rows + (int64_t)p * peer_stride;
            for (int64_t j = 0; j < N; ++j)
                acc[j] += bf16_to_double(prow[j]);
        }
#ifdef ORACLE_PLANT_PEERS_FIRST
        gemm_terms_f64(a, B, N, K, acc);
#endif
        for (int64_t j = 0; j < N; ++j)
            out[j] = oracle_round_bf16(acc[j]);
    } else {
        float *acc = (float *)scratch;
        for (int64_t j = 0; j < N; ++j)
            acc[j] = 0.0f;
#ifndef ORACLE_PLANT_PEERS_FIRST
        gemm_terms_f32(a, B, N, K, acc);
#endif
        for (int p = 0; p < np; ++p) {
            const uint16_t *prow = peer_rows + (int64_t)p * peer_stride;
            for (int64_t j = 0; j < N; ++j)
                acc[j] += bf16_to_float(prow[j]);
        }
#ifdef ORACLE_PLANT_PEERS_FIRST
        gemm_terms_f32(a, B, N, K, acc);
#endif
        /* a binary32 value is exactly a double: one rounding, to bf16 */
        for (int64_t j = 0; j < N; ++j)
            out[j] = oracle_round_bf16((double)acc[j]);
    }
}

/*
 * Rows given explicitly (for sampled checks at full size):
 *   A_rows    [nrows][K]          the sampled rows of A
 *   peer_rows [npeers][nrows][N]  the same rows of every peer partial
 *   out       [nrows][N]
 *   acc       ORACLE_ACC_FP32 or ORACLE_ACC_FP64 (accumulation precision)
 * out[t,j] = bf16( sum_k A_rows[t,k]*B[k,j] + sum_p peer_rows[p,t,j] ).
 */
int oracle_ar_rows(const uint16_t *A_rows, const uint16_t *B, const uint16_t *peer_rows,
                   int64_t nrows, int64_t N, int64_t K, int npeers, int acc, uint16_t *out)
{
    if (nrows < 0 || N < 0 || K < 0 || npeers < 0)
        return ORACLE_EINVAL;
    if (acc != ORACLE_ACC_FP32 && acc != ORACLE_ACC_FP64)
        return ORACLE_EINVAL;
    if (npeers > 0 && !peer_rows)
        return ORACLE_EINVAL;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        void *scratch = malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        if (!scratch) {
#pragma omp atomic write
            err = ORACLE_ENOMEM;
        }
        /* every thread reaches the worksharing loop, with or without scratch */
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < nrows; ++t)
            if (scratch)
                oracle_row(A_rows + t * K, B, peer_rows ? peer_rows + t * N : NULL,
                           nrows * N, npeers, N, K, acc, scratch, out + t * N);
        free(scratch);
    }
    return err;
}

/*
 * Reduce-scatter slice of rank r (test reference of "[Kimi-K3] Extend
 * GEMM-RS to GEMM-AR": the partial is padded to padded_M = ceil(M/R)*R rows
 * and reduce_scatter_single hands rank r the r-th of R equal chunks).
 *   *P  = ceil(M/R)                       rows of every rank's output
 *   *lo = r*P, *hi = min((r+1)*P, M)      valid global rows this rank owns
 * Output row t < P holds global row r*P + t when that is < M, else zero.
 */
int oracle_rs_slice(int64_t M, int R, int r, int64_t *P, int64_t *lo, int64_t *hi)
{
    if (M < 0 || R <= 0 || r < 0 || r >= R || !P || !lo || !hi)
        return ORACLE_EINVAL;
#ifdef ORACLE_PLANT_SLICE_FLOOR
    int64_t p = M / R;
#else
    int64_t p = (M + R - 1) / R;
#endif
    int64_t l = (int64_t)r * p;
    int64_t h = l + p;
    if (l > M)
        l = M;
    if (h > M)
        h = M;
    *P = p;
    *lo = l;
    *hi = h;
    return ORACLE_OK;
}

/*
 * GEMM-AR, whole matrices.
 *   A [M][K], B [K][N], peers [R-1][M][N] (slot p = the p-th other rank in
 *   ascending rank order), out [M][N].
 */
int oracle_gemm_ar(const uint16_t *A, const uint16_t *B, const uint16_t *peers,
                   int64_t M, int64_t N, int64_t K, int R, int acc, uint16_t *out)
{
    if (R < 1 || M < 0)
        return ORACLE_EINVAL;
    return oracle_ar_rows(A, B, peers, M, N, K, R - 1, acc, out);
}

/*
 * GEMM-RS, whole matrices.
 *   out [P][N]  P = ceil(M/R): out[t] = AR row r*P+t if that row is < M, else 0
 *   ws  [M][N]  rows i < M outside [lo,hi): bf16(G[i,:]) (this rank's own
 *               partial, which the owning rank would read); rows in [lo,hi)
 *               are left untouched.  ws may be NULL to skip the publish.
 */
int oracle_gemm_rs(const uint16_t *A, const uint16_t *B, const uint16_t *peers,
                   int64_t M, int64_t N, int64_t K, int R, int r, int acc,
                   uint16_t *out, uint16_t *ws)
{
    int64_t P, lo, hi;
    int err = oracle_rs_slice(M, R, r, &P, &lo, &hi);
    if (err)
        return err;
    int64_t owned = hi - lo;
    /* owned rows: sum over every rank's partial */
    if (owned > 0) {
        uint16_t *peer_rows = NULL;
        if (R > 1) {
            peer_rows = (uint16_t *)malloc((size_t)(R - 1) * owned * N * sizeof(uint16_t));
            if (!peer_rows)
                return ORACLE_ENOMEM;
            for (int p = 0; p < R - 1; ++p)
                memcpy(peer_rows + (int64_t)p * owned * N, peers + ((int64_t)p * M + lo) * N,
                       (size_t)owned * N * sizeof(uint16_t));
        }
        err = oracle_ar_rows(A + lo * K, B, peer_rows, owned, N, K, R - 1, acc, out);
        free(peer_rows);
        if (err)
            return err;
    }
    /* slice rows past M are the zero padding */
    for (int64_t t = owned; t < P; ++t)
        memset(out + t * N, 0, (size_t)N * sizeof(uint16_t));
    /* publish the non-owned rows of this rank's partial */
    if (ws) {
#ifdef ORACLE_PLANT_WS_ALL_ROWS
        err = oracle_ar_rows(A, B, NULL, M, N, K, 0, acc, ws);
        if (err)
            return err;
#else
        if (lo > 0) {
            err = oracle_ar_rows(A, B, NULL, lo, N, K, 0, acc, ws);
            if (err)
                return err;
        }
        if (hi < M)
            err = oracle_ar_rows(A + hi * K, B, NULL, M - hi, N, K, 0, acc, ws + hi * N);
#endif
    }
    return err;
}

/*
 * Source of output row g of AG-GEMM: shard q = g / Ms, row t = g % Ms.
 */
int oracle_ag_source(int64_t Ms, int R, int64_t g, int *q, int64_t *t)
{
    if (Ms <= 0 || R <= 0 || g < 0 || g >= Ms * R || !q || !t)
        return ORACLE_EINVAL;
    *q = (int)(g / Ms);
    *t = g % Ms;
    return ORACLE_OK;
}

/*
 * AG-GEMM, whole matrices.
 *   A_local [Ms][K]    this rank's shard
 *   shards  [R][Ms][K] every rank's shard (slot r is not read: A_local is)
 *   out     [R*Ms][N]  out[q*Ms + t] = bf16(S_q[t,:] . B)
 */
int oracle_ag_gemm(const uint16_t *A_local, const uint16_t *B, const uint16_t *shards,
                   int64_t Ms, int64_t N, int64_t K, int R, int r, int acc, uint16_t *out)
{
    if (Ms < 0 || R < 1 || r < 0 || r >= R)
        return ORACLE_EINVAL;
    for (int q = 0; q < R; ++q) {
        const uint16_t *src = (q == r) ? A_local : shards + (int64_t)q * Ms * K;
#ifdef ORACLE_PLANT_AG_LOCAL_ONLY
        src = A_local;
#endif
        int err = oracle_ar_rows(src, B, NULL, Ms, N, K, 0, acc, out + (int64_t)q * Ms * N);
        if (err)
            return err;
    }
    return ORACLE_OK;
}
