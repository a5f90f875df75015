/*
 * tg_gemm.h -- C ABI of the MI355X (gfx950) GEMM library libtg_gemm.so.
 *
 * Operation ("Matrix Multiplication Background User's Guide", sections 1-2,
 * in BLAS naming: A is M x K, B is K x N, C is M x N):
 *
 *     C[i][j] = epi( alpha * sum_{k < K} A(i,k) * B(k,j) + beta * C[i][j] )
 *
 * alpha = 1 and beta = 0 unless the epilogue sets TG_EPI_SCALE (the guide's
 * full BLAS statement scales the product and adds a multiple of the old C);
 * with beta = 0 the old C is not read (it may hold anything, NaN included).
 *
 * All matrices are row-major.  An operand may be stored transposed, as the
 * row-major array of its transpose (what the Triton matmul tutorial's
 * Y.T.contiguous() produces, "Learning Triton One Kernel at a Time: Matrix
 * Multiplication", section on memory coalescing):
 *
 *     A(i,k) = (trans & TG_TRANS_A) ? A[k*lda + i] : A[i*lda + k]
 *     B(k,j) = (trans & TG_TRANS_B) ? B[j*ldb + k] : B[k*ldb + j]
 *     C(i,j) = C[i*ldc + j]
 *
 * Inputs and output share one storage type (dtype); products are accumulated
 * in float32, alpha * sum + beta * C (the old C widened to float32) is formed
 * in float32, and epi is applied to it before the single rounding
 * (nearest-even) to the output type.  epi is the identity or a leaky
 * rectifier x >= 0 ? x : slope*x, the fused output transform the Triton news
 * article gives as the reason to hand-write matmul kernels ("OpenAI
 * open-sources Triton", matrix multiplication section).
 *
 * Leading dimensions (element counts):
 *     lda >= max(1, trans_a ? M : K),  ldb >= max(1, trans_b ? K : N),
 *     ldc >= max(1, N).
 * Strided views (an operand that is a slice of a wider matrix) are passed as
 * ld > width.  Misaligned pointers or leading dimensions are not errors; they
 * select a slower element-wise load path.
 *
 * Ownership and ordering: every pointer is caller-owned device memory; the
 * library keeps none of them after returning.  Work is enqueued on `stream`
 * (a hipStream_t; NULL = the null stream) and the call returns without
 * waiting: results are valid once the stream has been synchronised.  C must
 * not overlap A or B.
 *
 * Quick returns: M == 0 or N == 0 does nothing; K == 0 or alpha == 0 writes
 * epi(beta * C) without reading A or B (epi(0) = 0 when beta == 0).
 *
 * Errors: every entry point returns a tg_status; on failure nothing is
 * enqueued and tg_last_error() describes the cause (thread-local).
 *
 * Capture and threads: a call that needs no workspace, or is given one
 * through tg_gemm_ex, only launches kernels on `stream`, so it can be
 * recorded into a HIP graph (make one eager call first: it fills the
 * library's per-device caches); its kernels sum in fixed orders, so replays
 * reproduce the eager result bit for bit.  Calls from several host threads
 * on their own streams are independent.
 */
#ifndef TG_GEMM_H
#define TG_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TG_VERSION 107

/* storage type of A, B and C */
enum tg_dtype { TG_F32 = 0, TG_F16 = 1, TG_BF16 = 2 };

/* trans bits; first letter of the name is A's: TG_NT = A plain, B transposed */
enum tg_trans { TG_NN = 0, TG_TN = 1, TG_NT = 2, TG_TT = 3 };
#define TG_TRANS_A 1
#define TG_TRANS_B 2

enum tg_epi_kind { TG_EPI_NONE = 0, TG_EPI_LEAKY_RELU = 1 };

enum tg_status {
    TG_OK = 0,
    TG_ERR_ARG = -1,         /* negative size, leading dimension too small, unknown enum */
    TG_ERR_NULL = -2,        /* NULL pointer for an operand that has elements */
    TG_ERR_UNSUPPORTED = -3, /* a forced option that no kernel implements */
    TG_ERR_DEVICE = -4,      /* no gfx950 device, or a HIP runtime error */
    TG_ERR_LAUNCH = -5       /* a kernel launch failed */
};

/* Execution paths.  The planner picks one per call ("Matrix Multiplication
 * Background User's Guide", section 2: the arithmetic-intensity test decides
 * between math-bound and memory-bound; section 2.3: a library heuristic picks
 * the tile, and splits K when M and N are small and K is large). */
enum tg_path {
    TG_PATH_AUTO = -1,
    TG_PATH_NONE = 0,   /* quick return (M == 0, N == 0), or K == 0: C = epi(beta * C) */
    TG_PATH_MFMA = 1,   /* macro-tile matrix-core kernel (all storage types) */
    TG_PATH_SKINNY = 2, /* memory-bound narrow product (small N or small M), matrix cores */
    TG_PATH_GEMV = 3    /* M == 1 or N == 1: vector ALUs, no matrix cores */
};

/* flags of tg_epilogue */
#define TG_EPI_SCALE 1u /* use alpha and beta (otherwise alpha = 1, beta = 0) */

/* Output transform.  A zero-initialised struct (or NULL) is the plain product
 * C = A.B; unknown kinds or flag bits are TG_ERR_ARG. */
typedef struct tg_epilogue {
    uint32_t kind;  /* tg_epi_kind */
    float slope;    /* negative-side slope of TG_EPI_LEAKY_RELU */
    uint32_t flags; /* TG_EPI_SCALE */
    float alpha;    /* product scale, with TG_EPI_SCALE */
    float beta;     /* scale of the old C, with TG_EPI_SCALE; 0 = C is not read */
} tg_epilogue;

/* tg_options.split_k / tg_plan.split_k value for stream-K: instead of whole
 * tiles (or whole K splits) per workgroup, one workgroup per compute unit
 * takes an equal run of all the tiles' K stages (32-deep), so a product with
 * fewer tiles than compute units keeps every unit busy; tiles split between
 * workgroups are summed, in K order, by a fix-up kernel into C.  256 x 256
 * tiles, 16-bit 16-byte-aligned operands, fewer tiles than compute units
 * ("Matrix Multiplication Background User's Guide", section 3.2: the tail
 * wave; section 2.3: splitting K is the remedy libraries use). */
#define TG_SPLIT_STREAM_K (-1)

/* Optional planner overrides (NULL = all automatic).  A forced tile reproduces
 * the forced-tile measurements of "Matrix Multiplication Background User's
 * Guide", sections 3.1-3.2. */
typedef struct tg_options {
    int32_t path;    /* TG_PATH_AUTO, or a forced path */
    int32_t tile_m;  /* 0 = planner's choice, else a macro-tile height the path offers */
    int32_t tile_n;  /* 0 = planner's choice, else a macro-tile width */
    int32_t split_k; /* 0 = planner's choice, 1 = no split, s > 1 = split K s ways,
                        TG_SPLIT_STREAM_K = stream-K */
    int32_t k_groups; /* macro-tile path: 0 = planner's choice (1 when the tile is
                         forced), 1 = one group of waves per workgroup, 2 or 4 = that many
                         groups of waves per workgroup, each taking a consecutive part of
                         the workgroup's K range, their sums added in LDS (16-bit: 128 x 128
                         with 2, 64 x 64 with 4; float32: 128 x 128 with 2, 64 x 64 and
                         32 x 32 with 4); other values are TG_ERR_ARG, a count no kernel
                         offers for the operands TG_ERR_UNSUPPORTED */
} tg_options;

/* What the planner decided, and the quantization figures behind it. */
typedef struct tg_plan {
    int32_t path;        /* tg_path */
    int32_t tile_m, tile_n, tile_k;
    int32_t split_k;     /* K-splits (1 = none), or TG_SPLIT_STREAM_K */
    int32_t occupancy;   /* workgroups resident per compute unit */
    int32_t num_cus;     /* compute units the wave model used */
    int32_t vector_io;   /* 1 = 128-bit operand loads, 0 = element-wise, 2 = A and B first
                            copied into zero-padded 16-byte-aligned buffers at the start of
                            the workspace (K rounded up to 16 bytes), then 128-bit loads;
                            3 (float32) = the same copies laid out K-contiguous (A as M x K,
                            B as N x K, transposing operands stored the other way; when the
                            operands are aligned only those are copied) and the product
                            run as TG_NT; 4 (16-bit, skinny) = B alone first copied into a
                            zero-padded 16-byte-aligned buffer at the start of the workspace
                            (its rows rounded up to 8 elements), A read in place */
    int64_t tiles;       /* ceil(M/tile_m) * ceil(N/tile_n) */
    int64_t workgroups;  /* tiles * split_k (MFMA/skinny), the stream-K workgroups, or the GEMV grid */
    int64_t waves;       /* ceil(workgroups / (num_cus * occupancy)) */
    double tile_eff;     /* M*N / (tiles * tile_m * tile_n) */
    double wave_eff;     /* workgroups / (waves * num_cus * occupancy) */
    double pred_eff;     /* product of the two with the per-tile efficiency */
    double pred_us;      /* modelled run time, microseconds */
    double arith_intensity; /* 2MNK / (bytes of A, B and C), FLOP per byte */
    uint64_t workspace_bytes; /* float32 split-K partials or stream-K pieces, and aligned
                                 copies, the plan needs */
    int32_t k_groups;    /* macro-tile path: groups of waves per workgroup splitting its K
                            range, their sums added in LDS (no workspace, no second
                            launch; "Matrix Multiplication Background User's Guide",
                            section 2.3: splitting K); 1 elsewhere */
} tg_plan;

/* C = epi(alpha A . B + beta C) on the current HIP device.  epilogue may be
 * NULL (C = A . B).  When the plan needs workspace (float32 split-K partials,
 * or aligned copies of A and B), it comes from the calling thread's default
 * workspace (tg_set_workspace) when one is set, else it is a stream-ordered
 * allocation on `stream` from a memory pool the library keeps per device:
 * memory a call frees stays reserved for later calls until the process ends,
 * and a call that allocates cannot be recorded into a HIP graph.  (The guide
 * says only that a K split adds a reduction over partial tiles, "Matrix
 * Multiplication Background User's Guide", section 2.3; this call keeps the
 * split and supplies the buffer itself.)  Callers that must not allocate use
 * tg_gemm_ex with their own workspace, or tg_gemm_noalloc. */
int tg_gemm(int64_t M, int64_t N, int64_t K,
            const void *A, int64_t lda,
            const void *B, int64_t ldb,
            void *C, int64_t ldc,
            int dtype, int trans,
            const tg_epilogue *epilogue,
            void *stream);

/* tg_gemm with planner overrides and a caller-provided workspace.
 * workspace == NULL: as tg_gemm (the thread's default workspace, if set).  Otherwise it must be device memory aligned
 * to 256 bytes; when smaller than the plan's workspace_bytes the planner
 * falls back to an unsplit plan (not an error unless split_k was forced, then
 * TG_ERR_ARG).  Concurrent calls must not share a workspace. */
int tg_gemm_ex(int64_t M, int64_t N, int64_t K,
               const void *A, int64_t lda,
               const void *B, int64_t ldb,
               void *C, int64_t ldc,
               int dtype, int trans,
               const tg_epilogue *epilogue,
               const tg_options *opts,
               void *workspace, size_t workspace_bytes,
               void *stream);

/* Size of the static scratch of tg_gemm_noalloc: 64 MiB per device. */
#define TG_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* tg_gemm_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the call allocates nothing, with any allocator, and never uses the thread's
 * default workspace.  Whatever workspace the plan needs (float32 K-split
 * partials, stream-K pieces, aligned operand copies) comes from a scratch
 * array of TG_NOALLOC_SCRATCH_BYTES that the library holds in device memory on
 * every device it runs on, from the first call on that device until the
 * process ends.  An unforced plan that would need more is replaced as for a
 * small tg_gemm_ex workspace (no K split, then no copies); a forced K split
 * or stream-K that needs more is refused with TG_ERR_ARG, naming the maximum.
 * Every call on a device shares that device's scratch, and each call rewrites
 * whatever of it it reads: calls that may overlap on one device (several
 * streams, several host threads) race, and must be ordered by the caller.
 * Arguments and results as tg_gemm_ex. */
int tg_gemm_noalloc(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    void *C, int64_t ldc,
                    int dtype, int trans,
                    const tg_epilogue *epilogue,
                    const tg_options *opts,
                    void *stream);

/* The plan tg_gemm_ex would run on the current device (no launch). */
int tg_gemm_plan(int64_t M, int64_t N, int64_t K, int dtype, int trans,
                 const tg_options *opts, tg_plan *out);

/* The same planner as a pure model of a chip with num_cus compute units
 * (no device needed).  occupancy <= 0 uses the kernels' own residency;
 * a positive value overrides it (1 reproduces the one-tile-per-SM waves of
 * "Matrix Multiplication Background User's Guide", section 3.2). */
int tg_plan_model(int64_t M, int64_t N, int64_t K, int dtype, int trans,
                  int num_cus, int occupancy, const tg_options *opts, tg_plan *out);

/* Bytes of workspace the current device's plan needs (0 = none). */
size_t tg_workspace_size(int64_t M, int64_t N, int64_t K, int dtype, int trans,
                         const tg_options *opts);

/* The same for the planner's own choice (no overrides): the size of the
 * buffer of K-split partials ("Matrix Multiplication Background User's
 * Guide", section 2.3: a split adds a reduction over float32 partial tiles)
 * and of any aligned operand copies. */
size_t tg_workspace_bytes(int64_t M, int64_t N, int64_t K, int dtype, int trans);

/* Set the calling thread's default workspace: device memory of `bytes`
 * bytes, aligned to 256 bytes, owned by the caller and used (not copied) by
 * every later tg_gemm, and by tg_gemm_ex / tg_autotune calls whose own
 * workspace is NULL, until replaced; (NULL, 0) clears it.  A plan that needs
 * more than `bytes` falls back as with a small tg_gemm_ex workspace.  The
 * buffer holds partials only for the duration of each call on its stream:
 * calls that may overlap (other streams) need workspaces of their own.
 * Returns TG_ERR_ARG for a misaligned buffer, or NULL with bytes > 0. */
int tg_set_workspace(void *workspace, size_t bytes);

/* Benchmark mode ("Matrix Multiplication Background User's Guide", section
 * 2.3: a library may time its candidate kernels instead of trusting its
 * heuristic).  Runs the call once per candidate plan -- the planner's own
 * choice, every macro tile the kernels offer for these operands with K split
 * 1, 2, 3, 4, 6 or 8 ways, and the skinny path split 1, 2 or 4 ways when it
 * applies -- each timed `reps` times (>= 1) after one warm-up with events on
 * `stream`, and writes the fastest to *best (ready for tg_gemm_ex) and its
 * mean time in microseconds to *best_us (may be NULL).
 *
 * C is overwritten by every run with the product under `epilogue`'s kind and
 * slope; its alpha and beta are not applied while timing (beta would feed
 * each run's C into the next).  Blocks until the timing is done.  workspace
 * as for tg_gemm_ex (NULL: allocations are made per run).  Plans that need
 * more workspace than given are skipped.  Returns a tg_status.
 *
 * The winner is also recorded in a cache the library keeps per device, keyed
 * by the problem as the planner sees it (M, N, K, dtype, trans, lda, ldb, ldc
 * and whether A and B are 16-byte aligned; not the epilogue).  Later calls of
 * tg_gemm, tg_gemm_ex with opts == NULL, and tg_gemm_plan with opts == NULL
 * (which assumes packed, aligned operands) on the same device and problem use
 * the recorded plan instead of the heuristic; when a recorded K split finds
 * no room for its workspace, the call falls back as an unforced plan does.
 * The cache lives until the process ends or tg_tune_cache_clear. */
int tg_autotune(int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda,
                const void *B, int64_t ldb,
                void *C, int64_t ldc,
                int dtype, int trans,
                const tg_epilogue *epilogue,
                void *workspace, size_t workspace_bytes,
                void *stream, int reps,
                tg_options *best, float *best_us);

/* Row softmax ("OpenAI open-sources Triton", programming-model section: the
 * fused softmax that normalises each row of X on its own, keeping the row on
 * chip).  For every row i < M of the row-major M x N matrix X:
 *
 *     Y[i][j] = exp(X[i][j] - m_i) / sum_k exp(X[i][k] - m_i),  m_i = max_k X[i][k]
 *
 * in float32 arithmetic whatever the storage type (dtype, shared by X and Y),
 * rounded once (nearest-even) to it.  Rows holding NaN or +inf, or made only
 * of -inf, give NaN rows; -inf entries of other rows give 0.
 *
 * X(i,j) = X[i*ldx + j], Y(i,j) = Y[i*ldy + j]; ldx, ldy >= max(1, N).
 * Y may be X itself (in place, ldy == ldx); any other overlap is TG_ERR_ARG.
 * M, N < 2^31; M == 0 or N == 0 does nothing.  Rows up to 32768 elements stay
 * in registers (one read and one write of X's bytes); longer rows take two
 * passes (X read twice).  Pointers are caller-owned device memory; work is
 * enqueued on `stream` and the call returns without waiting.  Returns a
 * tg_status. */
int tg_softmax(int64_t M, int64_t N, const void *X, int64_t ldx, void *Y, int64_t ldy, int dtype,
               void *stream);

/* The launch shape tg_softmax uses for rows of N elements: waves (64 lanes)
 * per row and 16-byte chunks per lane of the register-resident kernel, or
 * 0 and 0 for the two-pass long-row kernel.  No device needed. */
int tg_softmax_shape(int64_t N, int dtype, int32_t *waves_per_row, int32_t *chunks_per_lane);

/* Forget every plan tg_autotune recorded on the current device.  Returns a
 * tg_status. */
int tg_tune_cache_clear(void);

/* Number of plans tg_autotune has recorded on the current device, or a
 * negative tg_status. */
int64_t tg_tune_cache_size(void);

/* Compute units of the current device, or a negative tg_status. */
int tg_device_cus(void);

/* Description of the last failure on this thread ("" after success). */
const char *tg_last_error(void);

/* TG_VERSION of the built library. */
int tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TG_GEMM_H */
