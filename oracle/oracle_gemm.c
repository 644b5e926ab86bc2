/*
 * CPU oracle for C = A.B over bf16 inputs, accumulated in binary64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code or header with the HIP library.
 *
 * What it computes (MikPoly page, part 1 "definitions", item 2 loop tiling,
 * the untiled triple loop): every output element starts at zero and receives
 * A[i][k]*B[k][j] for k = 0, 1, ..., K-1 in ascending order.  The operands
 * are the exact bf16 bit patterns the GPU consumes; bf16 -> binary32 ->
 * binary64 widening is exact and so is each bf16 x bf16 product in binary64
 * (at most 16 significant bits), so the only rounding is in the running sum.
 *
 * Layout: row-major A (M x K, leading dimension lda), B (K x N, ldb),
 * C (M x N, ldc), all in elements; batch entries are strideA/B/C apart.
 * C is overwritten (C := A.B); K = 0 yields zeros.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Number of threads the next parallel region will use. */
int oracle_threads(int requested)
{
#ifdef _OPENMP
    if (requested > 0) return requested;
    return omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

/*
 * Full product, batched.  Loop order i, k, j: each C[i][j] still receives its
 * terms in ascending k starting from 0.0, so the result is bit-identical to
 * the i, j, k triple loop of the definition.  If Cabs is not NULL it receives
 * sum_k |A[i][k]*B[k][j]| (used for the forward error bound of recursive
 * summation).  Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_gemm(int64_t batch, int64_t M, int64_t N, int64_t K,
                const uint16_t *A, int64_t lda, int64_t strideA,
                const uint16_t *B, int64_t ldb, int64_t strideB,
                double *C, int64_t ldc, int64_t strideC,
                double *Cabs, int nthreads)
{
    if (batch < 0 || M < 0 || N < 0 || K < 0) return -1;
    if (lda < K || ldb < N || ldc < N) return -1;
    int nt = oracle_threads(nthreads);
    double *Bd = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)(N > 0 ? N : 1));
    if (!Bd) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        const uint16_t *Ab = A + b * strideA;
        const uint16_t *Bb = B + b * strideB;
        double *Cb = C + b * strideC;
        double *Eb = Cabs ? Cabs + b * strideC : NULL;
        for (int64_t k = 0; k < K; ++k)
            for (int64_t j = 0; j < N; ++j)
                Bd[k * N + j] = widen_bf16(Bb[k * ldb + j]);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
        for (int64_t i = 0; i < M; ++i) {
            double *c = Cb + i * ldc;
            double *e = Eb ? Eb + i * ldc : NULL;
            for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
            if (e) for (int64_t j = 0; j < N; ++j) e[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = widen_bf16(Ab[i * lda + k]);
                const double *bk = Bd + k * N;
                for (int64_t j = 0; j < N; ++j) c[j] += a * bk[j];
                if (e) {
                    const double aa = a < 0 ? -a : a;
                    for (int64_t j = 0; j < N; ++j) {
                        const double bb = bk[j] < 0 ? -bk[j] : bk[j];
                        e[j] += aa * bb;
                    }
                }
            }
        }
    }
    free(Bd);
    return 0;
}

/*
 * Selected entries only: out[t] = C[rows[t]][cols[t]] of batch entry
 * bidx[t] (bidx may be NULL for batch entry 0), each by the plain ascending-k
 * dot product.  outabs (nullable) receives sum_k |a*b|.
 */
int oracle_gemm_entries(int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda, int64_t strideA,
                        const uint16_t *B, int64_t ldb, int64_t strideB,
                        int64_t count, const int64_t *bidx, const int64_t *rows,
                        const int64_t *cols, double *out, double *outabs, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    int nt = oracle_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nt) reduction(| : bad)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        const int64_t b = bidx ? bidx[t] : 0;
        if (i < 0 || i >= M || j < 0 || j >= N || b < 0) { bad = 1; continue; }
        const uint16_t *Ab = A + b * strideA;
        const uint16_t *Bb = B + b * strideB;
        double acc = 0.0, accabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = widen_bf16(Ab[i * lda + k]) * widen_bf16(Bb[k * ldb + j]);
            acc += p;
            accabs += p < 0 ? -p : p;
        }
        out[t] = acc;
        if (outabs) outabs[t] = accabs;
    }
    return bad ? -1 : 0;
}

/*
 * The same product as a sum of K outer products (rank-1 updates): for
 * k = 0, 1, ..., K-1 in ascending order, C += (column k of A) x (row k of
 * B), every row and column of the update visited from the last to the
 * first.  Each element still receives its K terms in ascending k starting
 * from zero, so the result must equal oracle_gemm bit for bit whatever the
 * order inside one update; the self-test relies on that (summation order
 * per element, not the visiting order of elements, fixes the rounding).
 * Single batch entry, run serially.
 */
int oracle_gemm_outer(int64_t M, int64_t N, int64_t K,
                      const uint16_t *A, int64_t lda,
                      const uint16_t *B, int64_t ldb,
                      double *C, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < N || ldc < N) return -1;
    for (int64_t i = 0; i < M; ++i)
        memset(C + i * ldc, 0, sizeof(double) * (size_t)N);
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t i = M - 1; i >= 0; --i) {
            const double a = widen_bf16(A[i * lda + k]);
            double *c = C + i * ldc;
            for (int64_t j = N - 1; j >= 0; --j) c[j] += a * widen_bf16(B[k * ldb + j]);
        }
    }
    return 0;
}
