/*
 * oracle.c -- reference GEMM for tests.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this file's library.  It shares no code, header or build step with the
 * GPU library and must never be called on a product path.
 *
 * What it computes is the plain definition of the general matrix multiply in
 * BLAS naming ("Matrix Multiplication Background User's Guide", section 2:
 * A is M x K, B is K x N, C is M x N), written out as a triple loop:
 *
 *     C[i][j] = epi( sum_{k = 0}^{K-1} A(i,k) * B(k,j) )
 *
 * with the sum taken in increasing k, in double precision, one rounding per
 * multiply and per add (the build passes -ffp-contract=off so no fused
 * multiply-add is formed).  Tiling only re-associates this sum ("Learning
 * Triton One Kernel at a Time: Matrix Multiplication", section on tiled GEMM),
 * so every blocked GPU schedule must land within rounding of it.
 *
 * Storage follows the row-major BLAS convention:
 *     A(i,k) = ta ? A[k*lda + i] : A[i*lda + k]
 *     B(k,j) = tb ? B[j*ldb + k] : B[k*ldb + j]
 * The operands arrive already widened (exactly) to double.
 *
 * epi is the identity (kind 0) or a leaky rectifier (kind 1):
 *     x >= 0 ? x : slope * x
 * the fused output transform named in the Triton news article's matrix
 * multiplication section.
 *
 * Alongside each value the oracle returns sum_k |A(i,k)| * |B(k,j)|, the scale
 * a floating-point error bound is stated against, and it counts the
 * multiply-adds it performed.
 *
 * A "fault" switch exists only so tests can plant a known mistake and check
 * that the pins notice it; it is off unless a test turns it on.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* planted-mistake switch, tests only: 0 none, 1 drop the last k term,
 * 2 read B transposed, 3 flip the sign of the k = 0 term, 4 swap the
 * leaky-rectifier branches */
static int g_fault = 0;

void oracle_plant_fault(int kind) { g_fault = kind; }

static double elem_a(const double *A, int64_t lda, int ta, int64_t i, int64_t k)
{
    return ta ? A[k * lda + i] : A[i * lda + k];
}

static double elem_b(const double *B, int64_t ldb, int tb, int64_t k, int64_t j)
{
    return tb ? B[j * ldb + k] : B[k * ldb + j];
}

/* B(k,j), or B(j,k) under planted fault 2 (only planted on square K == N) */
static double elem_b_f(const double *B, int64_t ldb, int tb, int64_t K, int64_t N,
                       int64_t k, int64_t j)
{
    if (g_fault == 2 && K == N)
        return elem_b(B, ldb, tb, j, k);
    return elem_b(B, ldb, tb, k, j);
}

static double epilogue(double x, int kind, double slope)
{
    if (kind == 1) {
        if (g_fault == 4)
            return x >= 0.0 ? slope * x : x;
        return x >= 0.0 ? x : slope * x;
    }
    return x;
}

typedef struct {
    int64_t M, N, K;
    const double *A;
    int64_t lda;
    int ta;
    const double *B;
    int64_t ldb;
    int tb;
    int epi;
    double slope;
    /* full mode */
    const double *Bt; /* logical B^T, N x K, gathered once (a copy) */
    double *C;
    int64_t ldc;
    double *absC;
    /* point mode */
    int64_t npts;
    const int64_t *I, *J;
    double *out, *absout;
    /* work split */
    int nthreads;
    int tid;
    int64_t macs;
} job_t;

/* One output element, the definition in increasing k. */
static void dot(const job_t *jb, const double *arow, const double *bcol,
                int64_t i, int64_t j, double *val, double *absval, int64_t *macs)
{
    double acc = 0.0, aacc = 0.0;
    int64_t kend = jb->K;
    if (g_fault == 1 && kend > 0)
        kend -= 1;
    for (int64_t k = 0; k < kend; ++k) {
        double a = arow ? arow[k] : elem_a(jb->A, jb->lda, jb->ta, i, k);
        double b = bcol ? bcol[k] : elem_b_f(jb->B, jb->ldb, jb->tb, jb->K, jb->N, k, j);
        double p = a * b;
        if (g_fault == 3 && k == 0)
            p = -p;
        acc = acc + p;
        double pa = (a < 0 ? -a : a) * (b < 0 ? -b : b);
        aacc = aacc + pa;
        *macs += 1;
    }
    *val = epilogue(acc, jb->epi, jb->slope);
    *absval = aacc;
}

static void *full_worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(jb->K > 0 ? jb->K : 1));
    if (!arow)
        return NULL;
    for (int64_t i = jb->tid; i < jb->M; i += jb->nthreads) {
        /* gather row i of A into a contiguous copy (a copy, no arithmetic) */
        for (int64_t k = 0; k < jb->K; ++k)
            arow[k] = elem_a(jb->A, jb->lda, jb->ta, i, k);
        for (int64_t j = 0; j < jb->N; ++j) {
            const double *bcol = jb->Bt + j * jb->K;
            double v, av;
            dot(jb, arow, bcol, i, j, &v, &av, &jb->macs);
            jb->C[i * jb->ldc + j] = v;
            if (jb->absC)
                jb->absC[i * jb->ldc + j] = av;
        }
    }
    free(arow);
    return NULL;
}

static void *point_worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    for (int64_t p = jb->tid; p < jb->npts; p += jb->nthreads) {
        double v, av;
        dot(jb, NULL, NULL, jb->I[p], jb->J[p], &v, &av, &jb->macs);
        jb->out[p] = v;
        if (jb->absout)
            jb->absout[p] = av;
    }
    return NULL;
}

static int run(job_t *proto, void *(*fn)(void *), int64_t *macs_out)
{
    int nt = proto->nthreads < 1 ? 1 : proto->nthreads;
    if (nt > 256)
        nt = 256;
    job_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nt; ++t) {
        jobs[t] = *proto;
        jobs[t].nthreads = nt;
        jobs[t].tid = t;
        jobs[t].macs = 0;
    }
    int started = 0;
    for (int t = 1; t < nt; ++t) {
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0)
            break;
        started = t;
    }
    /* threads that failed to start are run on the calling thread */
    fn(&jobs[0]);
    for (int t = started + 1; t < nt; ++t)
        fn(&jobs[t]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    int64_t total = 0;
    for (int t = 0; t < nt; ++t)
        total += jobs[t].macs;
    if (macs_out)
        *macs_out = total;
    return 0;
}

static int check_args(int64_t M, int64_t N, int64_t K, int64_t lda, int ta,
                      int64_t ldb, int tb)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (lda < (ta ? (M > 1 ? M : 1) : (K > 1 ? K : 1)))
        return -1;
    if (ldb < (tb ? (K > 1 ? K : 1) : (N > 1 ? N : 1)))
        return -1;
    return 0;
}

/* Whole product.  C and absC (may be NULL) are M x N with row stride ldc. */
int oracle_gemm_full(int64_t M, int64_t N, int64_t K,
                     const double *A, int64_t lda, int ta,
                     const double *B, int64_t ldb, int tb,
                     int epi, double slope,
                     double *C, double *absC, int64_t ldc,
                     int nthreads, int64_t *macs)
{
    if (check_args(M, N, K, lda, ta, ldb, tb) || ldc < (N > 1 ? N : 1))
        return -1;
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.M = M; jb.N = N; jb.K = K;
    jb.A = A; jb.lda = lda; jb.ta = ta;
    jb.B = B; jb.ldb = ldb; jb.tb = tb;
    jb.epi = epi; jb.slope = slope;
    jb.C = C; jb.absC = absC; jb.ldc = ldc;
    jb.nthreads = nthreads;
    /* columns of B gathered once into rows of a contiguous B^T copy */
    size_t nbt = (size_t)(N > 0 ? N : 1) * (size_t)(K > 0 ? K : 1);
    double *Bt = (double *)malloc(sizeof(double) * nbt);
    if (!Bt)
        return -3;
    for (int64_t j = 0; j < N; ++j)
        for (int64_t k = 0; k < K; ++k)
            Bt[j * K + k] = elem_b_f(B, ldb, tb, K, N, k, j);
    jb.Bt = Bt;
    int rc = run(&jb, full_worker, macs);
    free(Bt);
    if (macs && *macs < 0)
        rc = -3;
    return rc;
}

/* Selected elements (I[p], J[p]), p < npts. */
int oracle_gemm_points(int64_t M, int64_t N, int64_t K,
                       const double *A, int64_t lda, int ta,
                       const double *B, int64_t ldb, int tb,
                       int epi, double slope,
                       int64_t npts, const int64_t *I, const int64_t *J,
                       double *out, double *absout,
                       int nthreads, int64_t *macs)
{
    if (check_args(M, N, K, lda, ta, ldb, tb) || npts < 0)
        return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (I[p] < 0 || I[p] >= M || J[p] < 0 || J[p] >= N)
            return -2;
    job_t jb;
    memset(&jb, 0, sizeof jb);
    jb.M = M; jb.N = N; jb.K = K;
    jb.A = A; jb.lda = lda; jb.ta = ta;
    jb.B = B; jb.ldb = ldb; jb.tb = tb;
    jb.epi = epi; jb.slope = slope;
    jb.npts = npts; jb.I = I; jb.J = J;
    jb.out = out; jb.absout = absout;
    jb.nthreads = nthreads;
    return run(&jb, point_worker, macs);
}
