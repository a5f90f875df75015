// api.cpp -- the C ABI: argument checks, quick returns, planning, workspace,
// launches and error reporting.  See include/tg_gemm.h for the contract.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <string>
#include <vector>

#include "../../include/tg_gemm.h"
#include "kernels/launch.hpp"
#include "plan.h"

namespace tg {

// ---------------------------------------------------------------- dispatch by type

hipError_t launch_mfma(int dtype, int trans, int bm, int bn, bool vec, int kg, const MfmaArgs &a,
                       hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_mfma_f16(trans, bm, bn, vec, kg, a, s);
    case TG_BF16: return launch_mfma_bf16(trans, bm, bn, vec, kg, a, s);
    case TG_F32: return launch_mfma_f32(trans, bm, bn, vec, kg, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mfma2_sk(int dtype, int trans, const MfmaArgs &a, hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_mfma2_sk_f16(trans, a, s);
    case TG_BF16: return launch_mfma2_sk_bf16(trans, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mfma2(int dtype, int trans, int bm, int bn, int kg, const MfmaArgs &a, hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_mfma2_f16(trans, bm, bn, kg, a, s);
    case TG_BF16: return launch_mfma2_bf16(trans, bm, bn, kg, a, s);
    case TG_F32: return launch_mfma2_f32(trans, bm, bn, kg, a, s);
    }
    return hipErrorInvalidValue;
}

int mfma2_occupancy(int dtype, int trans, int bm, int bn, int kg)
{
    switch (dtype) {
    case TG_F16: return mfma2_occupancy_f16(trans, bm, bn, kg);
    case TG_BF16: return mfma2_occupancy_bf16(trans, bm, bn, kg);
    case TG_F32: return mfma2_occupancy_f32(trans, bm, bn, kg);
    }
    return 0;
}

// Which macro-tile kernel family runs a vector-load plan.  16-bit operands
// always take the LDS-DMA kernels (the planner sends leading dimensions above
// kDmaMaxLd16 through aligned copies or element-wise loads instead).  float32
// takes them for the 256 x 256 tile with K-contiguous A and B only (its
// leading dimensions count 16-bit units there: at most 2^21 float32 elements);
// its other tiles are the register-staged kernel.
static bool use_mfma2(int dtype, int trans, bool vec, int bm, int bn, int64_t lda, int64_t ldb)
{
    if (!vec)
        return false;
    if (dtype == TG_F32)
        return bm == 256 && bn == 256 && trans == TG_NT && lda <= kDmaMaxLd16 / 2 &&
               ldb <= kDmaMaxLd16 / 2;
    (void)lda;
    (void)ldb;
    return true;
}

int mfma_occupancy(int dtype, int trans, int bm, int bn, bool vec, int kg)
{
    switch (dtype) {
    case TG_F16: return mfma_occupancy_f16(trans, bm, bn, vec, kg);
    case TG_BF16: return mfma_occupancy_bf16(trans, bm, bn, vec, kg);
    case TG_F32: return mfma_occupancy_f32(trans, bm, bn, vec, kg);
    }
    return 0;
}

hipError_t launch_splitk_reduce(int dtype, const float *ws, int splits, int64_t wsld, int64_t plane,
                                int M, int N, void *C, int64_t ldc, const OutEpi &oe, int c_vec,
                                hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_splitk_reduce_f16(ws, splits, wsld, plane, M, N, C, ldc, oe, c_vec, s);
    case TG_BF16: return launch_splitk_reduce_bf16(ws, splits, wsld, plane, M, N, C, ldc, oe, c_vec, s);
    case TG_F32: return launch_splitk_reduce_f32(ws, splits, wsld, plane, M, N, C, ldc, oe, c_vec, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_pack(int dtype, const void *src, int64_t lds, int64_t rows, int64_t cols, void *dst,
                       int64_t drows, int64_t dcols, hipStream_t s, bool transposed)
{
    if (transposed) {
        switch (dtype) {
        case TG_F16: return launch_pack_t_f16(src, lds, rows, cols, dst, drows, dcols, s);
        case TG_BF16: return launch_pack_t_bf16(src, lds, rows, cols, dst, drows, dcols, s);
        case TG_F32: return launch_pack_t_f32(src, lds, rows, cols, dst, drows, dcols, s);
        }
        return hipErrorInvalidValue;
    }
    switch (dtype) {
    case TG_F16: return launch_pack_f16(src, lds, rows, cols, dst, drows, dcols, s);
    case TG_BF16: return launch_pack_bf16(src, lds, rows, cols, dst, drows, dcols, s);
    case TG_F32: return launch_pack_f32(src, lds, rows, cols, dst, drows, dcols, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scale_c(int dtype, void *C, int M, int N, int64_t ldc, const OutEpi &oe,
                          hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_scale_c_f16(C, M, N, ldc, oe, s);
    case TG_BF16: return launch_scale_c_bf16(C, M, N, ldc, oe, s);
    case TG_F32: return launch_scale_c_f32(C, M, N, ldc, oe, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_skinny(int dtype, bool trans_b, const SkinnyArgs &a, hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_skinny_f16(trans_b, a, s);
    case TG_BF16: return launch_skinny_bf16(trans_b, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_softmax(int dtype, int q, int c, bool vec, const SoftmaxArgs &a, hipStream_t s)
{
    switch (dtype) {
    case TG_F32: return launch_softmax_f32(q, c, vec, a, s);
    case TG_F16: return launch_softmax_f16(q, c, vec, a, s);
    case TG_BF16: return launch_softmax_bf16(q, c, vec, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int dtype, bool rows_form, bool vec, int lpr, const GemvArgs &a, hipStream_t s)
{
    switch (dtype) {
    case TG_F16: return launch_gemv_f16(rows_form, vec, lpr, a, s);
    case TG_BF16: return launch_gemv_bf16(rows_form, vec, lpr, a, s);
    case TG_F32: return launch_gemv_f32(rows_form, vec, lpr, a, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- errors

static thread_local std::string g_err;

static int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

static int ok()
{
    g_err.clear();
    return TG_OK;
}

// ---------------------------------------------------------------- device facts

// A problem as the planner sees it: sizes, layout, leading dimensions and
// alignment (the epilogue does not change the plan).
struct TuneKey {
    int64_t M, N, K, lda, ldb, ldc;
    int dtype, trans;
    bool aligned;
    bool operator<(const TuneKey &o) const
    {
        return std::tie(M, N, K, lda, ldb, ldc, dtype, trans, aligned) <
               std::tie(o.M, o.N, o.K, o.lda, o.ldb, o.ldc, o.dtype, o.trans, o.aligned);
    }
};

static TuneKey tune_key(const Problem &p)
{
    return TuneKey{p.M, p.N, p.K, p.lda, p.ldb, p.ldc, p.dtype, p.trans, p.ptrs_aligned};
}

struct DeviceInfo {
    bool probed = false;
    bool gfx950 = false;
    int cus = 0;
    int id = -1;
    std::string arch;
    // workspace pool: memory freed by a call stays reserved for the next one
    // (the device's default pool returns it at every synchronisation, and
    // mapping tens of MiB again costs more than the split or copy it serves)
    hipMemPool_t pool = nullptr;
    bool pool_tried = false;
    // device address of this device's copy of `scratch` (tg_gemm_noalloc),
    // taken once with this device current; null until then
    void *scratch_ptr = nullptr;
    // measured residency per (dtype, trans, tile, vec, K groups 1 / 2 / 4), 0 = not yet asked
    int occ[3][4][9][2][3] = {};
    // benchmark-mode winners (tg_autotune) per problem, used by calls that
    // pass no options; guarded by g_tune_mu
    std::map<TuneKey, tg_options> tuned;
};

static std::mutex g_tune_mu;

// Scratch of tg_gemm_noalloc: K-split partials, stream-K pieces and aligned
// operand copies, for callers that cannot allocate.  Every device the library
// runs on holds its own copy for the life of the process.  Host code never
// uses the name itself (on the host it is only a stand-in for the symbol):
// kernels get the device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[TG_NOALLOC_SCRATCH_BYTES];

// The cached benchmark-mode winner for p, if there is one.
static bool tune_lookup(DeviceInfo *dev, const Problem &p, tg_options *out)
{
    std::lock_guard<std::mutex> lk(g_tune_mu);
    auto it = dev->tuned.find(tune_key(p));
    if (it == dev->tuned.end())
        return false;
    *out = it->second;
    return true;
}

static std::mutex g_dev_mu;
static DeviceInfo g_dev[64];

static int current_device(DeviceInfo **info)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        int n = 0;
        if (hipGetDeviceCount(&n) != hipSuccess || n <= 0)
            return fail(TG_ERR_DEVICE, "no HIP device available");
        return fail(TG_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.probed) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(TG_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
        d.arch = prop.gcnArchName;
        d.gfx950 = d.arch.compare(0, 6, "gfx950") == 0;
        d.cus = prop.multiProcessorCount;
        d.id = dev;
        d.probed = true;
    }
    if (!d.gfx950)
        return fail(TG_ERR_DEVICE, "device %d is %s; this library is built for gfx950 only", dev,
                    d.arch.c_str());
    *info = &d;
    return TG_OK;
}

// Stream-ordered workspace from the device's library pool (created on first
// use, release threshold unlimited: the pool keeps its peak size until the
// process ends), or from the default pool if no pool can be made.
static hipError_t ws_alloc(DeviceInfo *d, void **ptr, size_t bytes, hipStream_t s)
{
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (!d->pool_tried) {
            d->pool_tried = true;
            hipMemPoolProps props{};
            props.allocType = hipMemAllocationTypePinned;
            props.location.type = hipMemLocationTypeDevice;
            props.location.id = d->id;
            hipMemPool_t pool = nullptr;
            if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
                uint64_t keep = UINT64_MAX;
                if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) == hipSuccess)
                    d->pool = pool;
                else
                    (void)hipMemPoolDestroy(pool);
            }
        }
    }
    if (d->pool)
        return hipMallocFromPoolAsync(ptr, bytes, d->pool, s);
    return hipMallocAsync(ptr, bytes, s);
}

static int tile_slot(int bm, int bn)
{
    // index of the tile in a small fixed table used for the occupancy cache
    static const int tiles[9][2] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}, {64, 64},
                                    {128, 256}, {64, 128},  {192, 256}, {32, 32}};
    for (int i = 0; i < 9; ++i)
        if (tiles[i][0] == bm && tiles[i][1] == bn)
            return i;
    return -1;
}

static int device_occ(int dtype, int trans, int bm, int bn, bool vec, int kg, void *ctx)
{
    DeviceInfo *d = (DeviceInfo *)ctx;
    const int ts = tile_slot(bm, bn);
    const int ki = kg == 1 ? 0 : kg == 2 ? 1 : kg == 4 ? 2 : -1;
    if (ts < 0 || ki < 0)
        return model_occupancy(dtype, bm, bn, vec, kg);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    int &slot = d->occ[dtype][trans][ts][vec ? 1 : 0][ki];
    if (slot == 0) {
        int n = use_mfma2(dtype, trans, vec, bm, bn, 0, 0) ? mfma2_occupancy(dtype, trans, bm, bn, kg)
                                                           : mfma_occupancy(dtype, trans, bm, bn, vec, kg);
        slot = n > 0 ? n : -1;
    }
    return slot > 0 ? slot : model_occupancy(dtype, bm, bn, vec, kg);
}

// ---------------------------------------------------------------- validation

static int check_args(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                      int64_t ldb, void *C, int64_t ldc, int dtype, int trans,
                      const tg_epilogue *epi)
{
    if (dtype < TG_F32 || dtype > TG_BF16)
        return fail(TG_ERR_ARG, "unknown dtype %d", dtype);
    if (trans < 0 || trans > 3)
        return fail(TG_ERR_ARG, "unknown trans %d", trans);
    if (epi && epi->kind != TG_EPI_NONE && epi->kind != TG_EPI_LEAKY_RELU)
        return fail(TG_ERR_ARG, "unknown epilogue kind %u", epi->kind);
    if (epi && (epi->flags & ~TG_EPI_SCALE) != 0)
        return fail(TG_ERR_ARG, "unknown epilogue flags 0x%x", epi->flags);
    if (M < 0 || N < 0 || K < 0)
        return fail(TG_ERR_ARG, "negative dimension (M=%lld N=%lld K=%lld)", (long long)M,
                    (long long)N, (long long)K);
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return fail(TG_ERR_ARG, "dimension above 2^31-1");
    const bool ta = trans & TG_TRANS_A, tb = trans & TG_TRANS_B;
    const int64_t need_a = std::max<int64_t>(1, ta ? M : K);
    const int64_t need_b = std::max<int64_t>(1, tb ? K : N);
    const int64_t need_c = std::max<int64_t>(1, N);
    if (lda < need_a)
        return fail(TG_ERR_ARG, "lda=%lld < %lld", (long long)lda, (long long)need_a);
    if (ldb < need_b)
        return fail(TG_ERR_ARG, "ldb=%lld < %lld", (long long)ldb, (long long)need_b);
    if (ldc < need_c)
        return fail(TG_ERR_ARG, "ldc=%lld < %lld", (long long)ldc, (long long)need_c);
    if (M > 0 && N > 0) {
        if (!C)
            return fail(TG_ERR_NULL, "C is NULL");
        if (K > 0 && !A)
            return fail(TG_ERR_NULL, "A is NULL");
        if (K > 0 && !B)
            return fail(TG_ERR_NULL, "B is NULL");
    }
    return TG_OK;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static Problem make_problem(int64_t M, int64_t N, int64_t K, int dtype, int trans, int64_t lda,
                            int64_t ldb, int64_t ldc, bool aligned)
{
    Problem p;
    p.M = M;
    p.N = N;
    p.K = K;
    p.dtype = dtype;
    p.trans = trans;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.ptrs_aligned = aligned;
    return p;
}

static Chip device_chip(const DeviceInfo &d)
{
    Chip c;
    c.num_cus = d.cus;
    return c;
}

// ---------------------------------------------------------------- execution

// The public epilogue as the kernels' output transform (NULL or a zeroed
// struct: the plain product).
static OutEpi out_epi(const tg_epilogue *epi)
{
    OutEpi oe;
    oe.kind = epi ? (int)epi->kind : TG_EPI_NONE;
    oe.slope = epi ? epi->slope : 0.0f;
    const bool scaled = epi && (epi->flags & TG_EPI_SCALE);
    oe.alpha = scaled ? epi->alpha : 1.0f;
    oe.beta = scaled ? epi->beta : 0.0f;
    return oe;
}

// rows_a, cols_b: rows of A and columns of B the macro-tile kernel may read
// (0: M and N; zero-padded copies hold more, rounded up to whole 16-byte chunks).
static int run_plan(const tg_plan &pl, const Problem &p, const void *A, const void *B, void *C,
                    const tg_epilogue *epi, void *ws, hipStream_t s, int64_t rows_a = 0,
                    int64_t cols_b = 0)
{
    const OutEpi oe = out_epi(epi);
    const int E = chunk_elems(p.dtype);
    hipError_t e = hipSuccess;
    if (pl.path == TG_PATH_NONE || oe.alpha == 0.0f) {
        // K == 0 or alpha == 0: no product term; A and B are not read
        if (p.M > 0 && p.N > 0)
            e = launch_scale_c(p.dtype, C, (int)p.M, (int)p.N, p.ldc, oe, s);
    } else if (pl.path == TG_PATH_MFMA) {
        MfmaArgs a{};
        a.A = A;
        a.B = B;
        a.C = C;
        a.ws = (float *)ws;
        a.lda = p.lda;
        a.ldb = p.ldb;
        a.ldc = p.ldc;
        a.M = (int)p.M;
        a.N = (int)p.N;
        a.K = (int)p.K;
        a.tiles_m = (int)((p.M + pl.tile_m - 1) / pl.tile_m);
        a.tiles_n = (int)((p.N + pl.tile_n - 1) / pl.tile_n);
        a.oe = oe;
        const int cb = elem_bytes(p.dtype);
        a.c_vec = (p.ldc % 4 == 0) && (((uintptr_t)C) % (4 * cb) == 0);
        a.rows_a = (int)(rows_a ? rows_a : p.M);
        a.cols_b = (int)(cols_b ? cols_b : p.N);
        if (pl.split_k == TG_SPLIT_STREAM_K) {
            // one workgroup per CU over all tiles' 32-deep K stages, then the fix-up
            a.sk_ipt = (int)((p.K + kStreamKStage - 1) / kStreamKStage);
            a.sk_total = (int64_t)a.tiles_m * a.tiles_n * a.sk_ipt;
            // fix-up bands: about 1024 workgroups over the tiles (1 to 16 rows each)
            const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
            a.sk_rows = 16;
            while (a.sk_rows > 1 && tiles * (256 / a.sk_rows) < 1024)
                a.sk_rows /= 2;
            a.splits = (int)pl.workgroups;
            a.kps = (int)p.K;
            e = launch_mfma2_sk(p.dtype, p.trans, a, s);
            if (e != hipSuccess)
                return fail(TG_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
            return TG_OK;
        }
        const int BK = pl.tile_k;
        int64_t kps = (p.K + pl.split_k - 1) / pl.split_k;
        kps = (kps + BK - 1) / BK * BK;
        a.kps = (int)kps;
        a.splits = pl.split_k;
        if (pl.vector_io != 0 && p.dtype != TG_F32 && (p.lda > kDmaMaxLd16 || p.ldb > kDmaMaxLd16))
            return fail(TG_ERR_UNSUPPORTED, "16-bit vector-load plan with a leading dimension above 2^22");
        if (use_mfma2(p.dtype, p.trans, pl.vector_io != 0, pl.tile_m, pl.tile_n, p.lda, p.ldb))
            e = launch_mfma2(p.dtype, p.trans, pl.tile_m, pl.tile_n, pl.k_groups, a, s);
        else
            e = launch_mfma(p.dtype, p.trans, pl.tile_m, pl.tile_n, pl.vector_io != 0, pl.k_groups, a, s);
        if (e == hipSuccess && pl.split_k > 1)
            e = launch_splitk_reduce(p.dtype, (const float *)ws, pl.split_k, p.N, p.M * p.N, (int)p.M, (int)p.N, C,
                                     p.ldc, oe, a.c_vec, s);
    } else if (pl.path == TG_PATH_SKINNY) {
        SkinnyArgs a{};
        a.A = A;
        a.B = B;
        a.C = C;
        a.ws = (float *)ws;
        a.lda = p.lda;
        a.ldb = p.ldb;
        a.ldc = p.ldc;
        a.M = (int)p.M;
        a.N = (int)p.N;
        a.K = (int)p.K;
        const int BK = pl.tile_k;
        int64_t kps = (p.K + pl.split_k - 1) / pl.split_k;
        kps = (kps + BK - 1) / BK * BK;
        a.kps = (int)kps;
        a.splits = pl.split_k;
        a.rb = pl.tile_m;
        a.nrb = (int)((p.M + a.rb - 1) / a.rb);
        a.skew = kSkinnySkew;
        a.oe = oe;
        const int cb = elem_bytes(p.dtype);
        a.c_vec = (p.ldc % 4 == 0) && (((uintptr_t)C) % (4 * cb) == 0);
        e = launch_skinny(p.dtype, (p.trans & TG_TRANS_B) != 0, a, s);
        if (e == hipSuccess && pl.split_k > 1)
            e = launch_splitk_reduce(p.dtype, (const float *)ws, pl.split_k, p.N, p.M * p.N, (int)p.M, (int)p.N, C,
                                     p.ldc, oe, a.c_vec, s);
    } else if (pl.path == TG_PATH_GEMV) {
        const bool ta = p.trans & TG_TRANS_A, tb = p.trans & TG_TRANS_B;
        const bool rows_form = pl.tile_m == 4;
        GemvArgs g{};
        g.ws = (float *)ws;
        g.K = (int)p.K;
        g.oe = oe;
        g.ksplit = pl.split_k;
        g.O = C;
        if (p.M == 1) {
            // out(j) = C[j]; vector a(k) = A(0,k); matrix B
            g.n = (int)p.N;
            g.os = 1;
            g.V = A;
            g.vs = ta ? p.lda : 1;
            g.X = B;
            g.ldx = p.ldb;
            (void)tb;
        } else {
            // N == 1: out(i) = C[i*ldc]; vector b(k) = B(k,0); matrix A
            g.n = (int)p.M;
            g.os = p.ldc;
            g.V = B;
            g.vs = tb ? 1 : p.ldb;
            g.X = A;
            g.ldx = p.lda;
        }
        if (!rows_form) {
            int64_t rps = (p.K + pl.split_k - 1) / pl.split_k;
            rps = (rps + 3) / 4 * 4;
            g.rows_per_split = (int)rps;
        } else {
            g.rows_per_split = (int)p.K;
        }
        const int lpr = rows_form ? 0 : pl.tile_n / E;
        e = launch_gemv(p.dtype, rows_form, pl.vector_io != 0, lpr, g, s);
    } else {
        return fail(TG_ERR_UNSUPPORTED, "path %d has no kernel", pl.path);
    }
    if (e != hipSuccess)
        return fail(TG_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    return TG_OK;
}

// The calling thread's default workspace (tg_set_workspace).
static thread_local void *t_ws = nullptr;
static thread_local size_t t_ws_bytes = 0;

// The device address of the current device's `scratch` array, taken on the
// first request with that device current and kept per device.
static int scratch_address(DeviceInfo *dev, void **out)
{
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (!dev->scratch_ptr) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(TG_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        dev->scratch_ptr = ptr;
    }
    *out = dev->scratch_ptr;
    return TG_OK;
}

// static_scratch: workspace is this device's `scratch` array (tg_gemm_noalloc);
// nothing is allocated, and a forced plan that needs more is refused.
static int gemm_impl(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                     int64_t ldb, void *C, int64_t ldc, int dtype, int trans,
                     const tg_epilogue *epi, const tg_options *opts, void *user_ws,
                     size_t user_ws_bytes, void *stream, bool static_scratch = false)
{
    if (!user_ws && !static_scratch) {
        user_ws = t_ws;
        user_ws_bytes = t_ws_bytes;
    }
    int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epi);
    if (rc != TG_OK)
        return rc;
    if (M == 0 || N == 0)
        return ok();
    DeviceInfo *dev = nullptr;
    rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    if (static_scratch) {
        rc = scratch_address(dev, &user_ws);
        if (rc != TG_OK)
            return rc;
        user_ws_bytes = TG_NOALLOC_SCRATCH_BYTES;
    }
    hipStream_t s = (hipStream_t)stream;
    const OutEpi oe0 = out_epi(epi);
    if (K == 0 || oe0.alpha == 0.0f) {
        // no product term: C = epi(beta * C), A and B untouched (no plan, no workspace)
        const hipError_t e = launch_scale_c(dtype, C, (int)M, (int)N, ldc, oe0, s);
        if (e != hipSuccess)
            return fail(TG_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    const bool aligned = aligned16(A) && aligned16(B);
    Problem p = make_problem(M, N, K, dtype, trans, lda, ldb, ldc, aligned);
    Chip chip = device_chip(*dev);
    tg_plan pl;
    const char *why = "";
    // no options: a benchmark-mode winner for this problem, if one was recorded
    tg_options tuned;
    bool from_cache = false;
    if (!opts && tune_lookup(dev, p, &tuned)) {
        if (make_plan(p, chip, 0, &tuned, device_occ, dev, false, &pl, &why) == TG_OK) {
            opts = &tuned;
            from_cache = true;
        }
    }
    if (!from_cache) {
        rc = make_plan(p, chip, 0, opts, device_occ, dev, false, &pl, &why);
        if (rc != TG_OK)
            return fail(rc, "%s", why);
    }

    void *ws = nullptr;
    bool own_ws = false;
    if (pl.workspace_bytes > 0) {
        if (user_ws && ((uintptr_t)user_ws & 255u) != 0)
            return fail(TG_ERR_ARG, "workspace must be 256-byte aligned");
        if (user_ws) {
            if (user_ws_bytes >= pl.workspace_bytes)
                ws = user_ws;
        } else if (ws_alloc(dev, &ws, pl.workspace_bytes, s) == hipSuccess) {
            own_ws = true;
        } else {
            ws = nullptr;
        }
        if (!ws) {
            if (opts && (opts->split_k > 1 || opts->split_k == TG_SPLIT_STREAM_K) && !from_cache) {
                if (static_scratch)
                    return fail(TG_ERR_ARG,
                                "forced split_k=%d needs %llu bytes of scratch; the static scratch "
                                "holds %llu (TG_NOALLOC_SCRATCH_BYTES)",
                                opts->split_k, (unsigned long long)pl.workspace_bytes,
                                (unsigned long long)TG_NOALLOC_SCRATCH_BYTES);
                return fail(TG_ERR_ARG, "forced split_k=%d needs %llu bytes of workspace",
                            opts->split_k, (unsigned long long)pl.workspace_bytes);
            }
            // without the room: no K split, then no aligned copies either
            tg_options o = opts ? *opts : tg_options{TG_PATH_AUTO, 0, 0, 0};
            o.split_k = 1;
            rc = make_plan(p, chip, 0, &o, device_occ, dev, false, &pl, &why);
            if (rc != TG_OK)
                return fail(rc, "%s", why);
            if (pl.workspace_bytes > 0 && user_ws && user_ws_bytes >= pl.workspace_bytes) {
                ws = user_ws;
            } else if (pl.workspace_bytes > 0) {
                rc = make_plan(p, chip, 0, &o, device_occ, dev, false, &pl, &why, false);
                if (rc != TG_OK)
                    return fail(rc, "%s", why);
            }
        }
    }
    if (pl.vector_io == 4) {
        // the skinny kernel on an aligned, zero-padded copy of B; A in place
        const bool tb = trans & TG_TRANS_B;
        const int64_t brows = tb ? N : K, bcols = tb ? K : N;
        const int64_t bld = skinny_b_ld(p);
        char *w = (char *)ws;
        const hipError_t e = launch_pack(dtype, B, ldb, brows, bcols, w, brows, bld, s, false);
        if (e != hipSuccess) {
            if (own_ws)
                (void)hipFreeAsync(ws, s);
            return fail(TG_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
        }
        tg_plan inner = pl;
        inner.vector_io = 1;
        Problem r = p;
        r.ldb = bld;
        rc = run_plan(inner, r, A, w, C, epi, w + skinny_b_bytes(p), s);
        if (own_ws)
            (void)hipFreeAsync(ws, s);
        if (rc != TG_OK)
            return rc;
        return ok();
    }
    if (pl.vector_io == 2 || pl.vector_io == 3) {
        // copy A and B into zero-padded aligned buffers (3: laid out for the NT
        // product, transposing where needed), then run the aligned plan
        const bool nt = pl.vector_io == 3;
        const PackLayout L = pack_layout(p, nt);
        const Problem q = packed_problem(p, nt);
        const bool ta = trans & TG_TRANS_A, tb = trans & TG_TRANS_B;
        char *w = (char *)ws;
        const void *Ap = L.a_copy ? (const void *)(w + L.a_off) : A;
        const void *Bp = L.b_copy ? (const void *)(w + L.b_off) : B;
        hipError_t e = hipSuccess;
        if (L.a_copy)
            e = launch_pack(dtype, A, lda, ta ? K : M, ta ? M : K, w + L.a_off, L.a_rows, L.a_cols, s,
                            L.a_trans);
        if (e == hipSuccess && L.b_copy)
            e = launch_pack(dtype, B, ldb, tb ? N : K, tb ? K : N, w + L.b_off, L.b_rows, L.b_cols, s,
                            L.b_trans);
        if (e != hipSuccess) {
            if (own_ws)
                (void)hipFreeAsync(ws, s);
            return fail(TG_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
        }
        tg_plan inner = pl;
        inner.vector_io = 1;
        // the copies are read over their padded extent; the M x N result goes
        // straight to C (rows and columns past M and N are computed from the
        // zero padding and never stored)
        Problem r = q;
        r.M = M;
        r.N = N;
        rc = run_plan(inner, r, Ap, Bp, C, epi, w + L.bytes, s, q.M, q.N);
        if (own_ws)
            (void)hipFreeAsync(ws, s);
        if (rc != TG_OK)
            return rc;
        return ok();
    }
    rc = run_plan(pl, p, A, B, C, epi, ws, s);
    if (own_ws)
        (void)hipFreeAsync(ws, s);
    if (rc != TG_OK)
        return rc;
    return ok();
}

}  // namespace tg

// ---------------------------------------------------------------- exported C ABI

using namespace tg;

extern "C" {

int tg_gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
            int64_t ldb, void *C, int64_t ldc, int dtype, int trans, const tg_epilogue *epilogue,
            void *stream)
{
    return gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue, nullptr, nullptr, 0,
                     stream);
}

int tg_gemm_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
               int64_t ldb, void *C, int64_t ldc, int dtype, int trans,
               const tg_epilogue *epilogue, const tg_options *opts, void *workspace,
               size_t workspace_bytes, void *stream)
{
    return gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue, opts, workspace,
                     workspace_bytes, stream);
}

int tg_gemm_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                    int64_t ldb, void *C, int64_t ldc, int dtype, int trans,
                    const tg_epilogue *epilogue, const tg_options *opts, void *stream)
{
    return gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue, opts, nullptr, 0,
                     stream, true);
}

int tg_gemm_plan(int64_t M, int64_t N, int64_t K, int dtype, int trans, const tg_options *opts,
                 tg_plan *out)
{
    if (!out)
        return fail(TG_ERR_NULL, "out is NULL");
    DeviceInfo *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    const bool ta = trans & TG_TRANS_A, tb = trans & TG_TRANS_B;
    Problem p = make_problem(M, N, K, dtype, trans, std::max<int64_t>(1, ta ? M : K),
                             std::max<int64_t>(1, tb ? K : N), std::max<int64_t>(1, N), true);
    const char *why = "";
    tg_options tuned;
    if (!opts && tune_lookup(dev, p, &tuned) &&
        make_plan(p, device_chip(*dev), 0, &tuned, device_occ, dev, false, out, &why) == TG_OK)
        return ok();
    rc = make_plan(p, device_chip(*dev), 0, opts, device_occ, dev, false, out, &why);
    if (rc != TG_OK)
        return fail(rc, "%s", why);
    return ok();
}

int tg_plan_model(int64_t M, int64_t N, int64_t K, int dtype, int trans, int num_cus,
                  int occupancy, const tg_options *opts, tg_plan *out)
{
    if (!out)
        return fail(TG_ERR_NULL, "out is NULL");
    const bool ta = trans & TG_TRANS_A, tb = trans & TG_TRANS_B;
    Problem p = make_problem(M, N, K, dtype, trans, std::max<int64_t>(1, ta ? M : K),
                             std::max<int64_t>(1, tb ? K : N), std::max<int64_t>(1, N), true);
    Chip chip;
    chip.num_cus = num_cus;
    const char *why = "";
    int rc = make_plan(p, chip, occupancy, opts, nullptr, nullptr, true, out, &why);
    if (rc != TG_OK)
        return fail(rc, "%s", why);
    return ok();
}

size_t tg_workspace_size(int64_t M, int64_t N, int64_t K, int dtype, int trans,
                         const tg_options *opts)
{
    tg_plan pl;
    if (tg_gemm_plan(M, N, K, dtype, trans, opts, &pl) != TG_OK)
        return 0;
    return (size_t)pl.workspace_bytes;
}

size_t tg_workspace_bytes(int64_t M, int64_t N, int64_t K, int dtype, int trans)
{
    return tg_workspace_size(M, N, K, dtype, trans, nullptr);
}

int tg_set_workspace(void *workspace, size_t bytes)
{
    if (!workspace && bytes > 0)
        return fail(TG_ERR_ARG, "workspace is NULL but bytes = %zu", bytes);
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(TG_ERR_ARG, "workspace must be 256-byte aligned");
    t_ws = workspace;
    t_ws_bytes = workspace ? bytes : 0;
    return ok();
}

int tg_autotune(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                int64_t ldb, void *C, int64_t ldc, int dtype, int trans,
                const tg_epilogue *epilogue, void *workspace, size_t workspace_bytes, void *stream,
                int reps, tg_options *best, float *best_us)
{
    if (!best)
        return fail(TG_ERR_NULL, "best is NULL");
    if (reps < 1)
        return fail(TG_ERR_ARG, "reps=%d < 1", reps);
    int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, epilogue);
    if (rc != TG_OK)
        return rc;
    *best = tg_options{TG_PATH_AUTO, 0, 0, 0};
    if (best_us)
        *best_us = 0.0f;
    if (M == 0 || N == 0 || K == 0)
        return ok();   // nothing to choose
    DeviceInfo *dev = nullptr;
    rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    // timing runs: the epilogue's kind and slope, no alpha / beta
    tg_epilogue epi{};
    if (epilogue) {
        epi.kind = epilogue->kind;
        epi.slope = epilogue->slope;
    }
    // candidates: the planner's choice, then forced tiles and splits
    std::vector<tg_options> cands;
    cands.push_back(tg_options{TG_PATH_AUTO, 0, 0, 0});
    const TileSpec *menu;
    const int nmenu = tile_menu(dtype, &menu);
    const int splits[] = {1, 2, 3, 4, 6, 8};
    for (int i = 0; i < nmenu; ++i)
        for (int sp : splits)
            cands.push_back(tg_options{TG_PATH_MFMA, menu[i].bm, menu[i].bn, sp, menu[i].kg});
    cands.push_back(tg_options{TG_PATH_MFMA, 64, 64, 1});   // the element-wise tile
    cands.push_back(tg_options{TG_PATH_MFMA, 256, 256, TG_SPLIT_STREAM_K});
    for (int rb : {64, 128})
        for (int sp : {1, 2, 4, 8})
            cands.push_back(tg_options{TG_PATH_SKINNY, rb, 0, sp});

    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0)
            (void)hipEventDestroy(e0);
        return fail(TG_ERR_DEVICE, "hipEventCreate failed");
    }
    const bool aligned = aligned16(A) && aligned16(B);
    Problem p = make_problem(M, N, K, dtype, trans, lda, ldb, ldc, aligned);
    Chip chip = device_chip(*dev);
    float best_t = -1.0f;
    int status = TG_OK;
    for (const tg_options &o : cands) {
        // skip candidates with no kernel for these operands, or without room
        tg_plan pl;
        const char *why = "";
        if (make_plan(p, chip, 0, &o, device_occ, dev, false, &pl, &why) != TG_OK)
            continue;
        if (o.path != TG_PATH_AUTO && o.split_k > 1 && pl.split_k != o.split_k)
            continue;   // the split collapsed to another candidate
        if (workspace && pl.workspace_bytes > workspace_bytes)
            continue;
        if (gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, &epi, &o, workspace,
                      workspace_bytes, stream) != TG_OK)
            continue;   // e.g. a forced split that found no workspace
        bool okrun = hipEventRecord(e0, s) == hipSuccess;
        for (int r = 0; r < reps && okrun; ++r)
            okrun = gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, trans, &epi, &o, workspace,
                              workspace_bytes, stream) == TG_OK;
        okrun = okrun && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
        float ms = 0.0f;
        if (!okrun || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            status = fail(TG_ERR_DEVICE, "timing a candidate failed");
            break;
        }
        const float us = ms * 1000.0f / (float)reps;
        if (best_t < 0.0f || us < best_t) {
            best_t = us;
            *best = o;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (status != TG_OK)
        return status;
    if (best_t < 0.0f)
        return fail(TG_ERR_UNSUPPORTED, "no candidate plan ran");
    if (best_us)
        *best_us = best_t;
    {
        std::lock_guard<std::mutex> lk(g_tune_mu);
        dev->tuned[tune_key(p)] = *best;
    }
    return ok();
}

int tg_tune_cache_clear(void)
{
    DeviceInfo *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    std::lock_guard<std::mutex> lk(g_tune_mu);
    dev->tuned.clear();
    return ok();
}

int64_t tg_tune_cache_size(void)
{
    DeviceInfo *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    std::lock_guard<std::mutex> lk(g_tune_mu);
    return (int64_t)dev->tuned.size();
}

int tg_device_cus(void)
{
    DeviceInfo *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    return dev->cus;
}

int tg_softmax_shape(int64_t N, int dtype, int32_t *waves_per_row, int32_t *chunks_per_lane)
{
    if (!waves_per_row || !chunks_per_lane)
        return fail(TG_ERR_NULL, "output pointer is NULL");
    if (dtype < TG_F32 || dtype > TG_BF16)
        return fail(TG_ERR_ARG, "unknown dtype %d", dtype);
    if (N < 0 || N > INT32_MAX)
        return fail(TG_ERR_ARG, "N=%lld out of range", (long long)N);
    int q = 0, c = 0;
    softmax_shape(dtype, N, &q, &c);
    *waves_per_row = q;
    *chunks_per_lane = c;
    return ok();
}

int tg_softmax(int64_t M, int64_t N, const void *X, int64_t ldx, void *Y, int64_t ldy, int dtype,
               void *stream)
{
    if (dtype < TG_F32 || dtype > TG_BF16)
        return fail(TG_ERR_ARG, "unknown dtype %d", dtype);
    if (M < 0 || N < 0)
        return fail(TG_ERR_ARG, "negative dimension");
    if (N > INT32_MAX || M > INT32_MAX)
        return fail(TG_ERR_ARG, "M and N must be below 2^31");
    const int64_t need = N > 1 ? N : 1;
    if (ldx < need || ldy < need)
        return fail(TG_ERR_ARG, "ldx=%lld / ldy=%lld < max(1, N)=%lld", (long long)ldx,
                    (long long)ldy, (long long)need);
    if (M == 0 || N == 0)
        return ok();
    if (!X || !Y)
        return fail(TG_ERR_NULL, "X or Y is NULL");
    const int64_t span_max = (INT64_MAX / 8 - N) / (M > 1 ? M - 1 : 1);
    if (ldx > span_max || ldy > span_max)
        return fail(TG_ERR_ARG, "leading dimension too large for M=%lld", (long long)M);
    const int64_t es = elem_bytes(dtype);
    const uintptr_t x0 = (uintptr_t)X, y0 = (uintptr_t)Y;
    const uintptr_t x1 = x0 + (uintptr_t)(((M - 1) * ldx + N) * es);
    const uintptr_t y1 = y0 + (uintptr_t)(((M - 1) * ldy + N) * es);
    if (x0 < y1 && y0 < x1 && !(x0 == y0 && ldx == ldy))
        return fail(TG_ERR_ARG, "Y overlaps X other than in place (Y == X, ldy == ldx)");
    DeviceInfo *dev = nullptr;
    int rc = current_device(&dev);
    if (rc != TG_OK)
        return rc;
    int q = 0, c = 0;
    softmax_shape(dtype, N, &q, &c);
    const int E = chunk_elems(dtype);
    const bool vec = (x0 % 16 == 0) && (y0 % 16 == 0) && (ldx % E == 0) && (ldy % E == 0);
    SoftmaxArgs a{};
    a.X = X;
    a.Y = Y;
    a.ldx = ldx;
    a.ldy = ldy;
    a.M = M;
    a.N = (int)N;
    const hipError_t e = launch_softmax(dtype, q, c, vec, a, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(TG_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char *tg_last_error(void) { return g_err.c_str(); }

int tg_version(void) { return TG_VERSION; }

}  // extern "C"
