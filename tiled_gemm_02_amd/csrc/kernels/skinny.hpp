// skinny.hpp -- memory-bound narrow products: M large, N <= 128, K large.
//
// At N = 128 the product does about 124 FLOP per byte moved ("Matrix
// Multiplication Background User's Guide", section 2, works this example),
// below MI355X's ~315 FLOP/byte ridge, so the time is the time to stream A
// from HBM once.  A still needs the matrix cores: at 8 TB/s the multiply-adds
// arrive faster than the vector ALUs retire them.  The kernel is therefore an
// HBM stream that feeds MFMAs:
//   * a workgroup owns 64 rows of C and all (<= 128) of its columns, over a
//     K range (split K across workgroups when M alone gives too few of them);
//   * A goes straight from HBM into MFMA operand registers (each lane loads
//     16 bytes of one row), prefetched two K steps ahead - it is used once,
//     so staging it through LDS would only add traffic;
//   * B (small, L2-resident) is staged per 256-deep K step into LDS as
//     K-contiguous rows (transposed 8 x 8 in registers when B is stored
//     N-contiguous), XOR-swizzled so both the writes and the fragment reads
//     are bank-conflict free, double buffered;
//   * the 8 waves split each K step four ways (and the 64 rows two ways), so
//     LDS traffic per byte of A stays low; their partial tiles are summed in
//     LDS in a fixed order ((w0 + w2) + (w1 + w3)) before the epilogue.
#pragma once

#include "common.hpp"

namespace tg {

struct SkinnyArgs {
    const void *A;
    const void *B;
    void *C;
    float *ws;       // split partials [splits][M][N]
    int64_t lda, ldb, ldc;
    int M, N, K;
    int kps;         // K per split, multiple of 256
    int splits;
    int epi;
    float slope;
    int c_vec;
};

constexpr int kSkRows = 64;     // C rows per workgroup
constexpr int kSkCols = 128;    // C columns covered (N <= 128)
constexpr int kSkBK = 256;      // K per step
constexpr int kSkChunks = kSkBK / 8;  // 16-byte chunks per LDS row (32)

__device__ __forceinline__ int sk_swz(int n) { return (n ^ (n >> 3)) & 15; }

template <typename Tr, bool TB>
__global__ __launch_bounds__(512) void skinny_kernel(SkinnyArgs p)
{
    using T = typename Tr::T;
    constexpr int STAGE = kSkCols * kSkChunks;  // chunks per LDS stage (64 KiB)
    __shared__ u32x4 lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rg = wave & 1;   // row group: rows 32*rg .. 32*rg+31
    const int kg = wave >> 1;  // K group: k 64*kg .. 64*kg+63 of each step
    const int fr = lane & 15, g = lane >> 4;

    const int row0 = blockIdx.x * kSkRows;
    const int z = blockIdx.y;
    const int kbeg = z * p.kps;
    const int kend = min(p.K, kbeg + p.kps);
    const int nsteps = (kend - kbeg + kSkBK - 1) / kSkBK;

    const T *A = (const T *)p.A;
    const T *B = (const T *)p.B;

    // A operand rows of this lane (clamped at the bottom edge; never stored)
    const T *arow[2];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) {
        const int r = min(row0 + 32 * rg + 16 * fm + fr, p.M - 1);
        arow[fm] = A + (int64_t)r * p.lda;
    }
    auto load_a = [&](u32x4 *dst, int k0) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int k = k0 + 64 * kg + 32 * kb + 8 * g;
                dst[fm * 2 + kb] = k < kend ? *(const u32x4 *)(arow[fm] + k) : zero4();
            }
    };

    // B staging: 128 columns x 256 k per step, 512 threads
    u32x4 breg[8];
    auto load_b = [&](int k0) {
        if constexpr (!TB) {
            // B stored K x N (N contiguous): one 8 x 8 block per thread
            const int nb = tid & 15, kb8 = tid >> 4;
            const int gc = min(8 * nb, p.N - 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = k0 + 8 * kb8 + e;
                breg[e] = k < kend ? *(const u32x4 *)(B + (int64_t)k * p.ldb + gc) : zero4();
            }
        } else {
            // B stored N x K (K contiguous): 8 chunks per thread
            const int c = tid & 31;
            const int k = k0 + 8 * c;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int n = min((tid >> 5) + 16 * q, p.N - 1);
                breg[q] = k < kend ? *(const u32x4 *)(B + (int64_t)n * p.ldb + k) : zero4();
            }
        }
    };
    auto store_b = [&](u32x4 *dst) {
        if constexpr (!TB) {
            const int nb = tid & 15, kb8 = tid >> 4;
            u32x4 t[8];
            transpose_block<2>(breg, t);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = 8 * nb + j;
                dst[n * kSkChunks + (kb8 ^ sk_swz(n))] = t[j];
            }
        } else {
            const int c = tid & 31;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int n = (tid >> 5) + 16 * q;
                dst[n * kSkChunks + (c ^ sk_swz(n))] = breg[q];
            }
        }
    };

    f32x4 acc[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const u32x4 *a, const u32x4 *bs) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int c = 8 * kg + 4 * kb + g;
            u32x4 bf[8];
#pragma unroll
            for (int fn = 0; fn < 8; ++fn) {
                const int n = 16 * fn + fr;
                bf[fn] = bs[n * kSkChunks + (c ^ sk_swz(n))];
            }
#pragma unroll
            for (int fm = 0; fm < 2; ++fm)
#pragma unroll
                for (int fn = 0; fn < 8; ++fn)
                    mfma_chunk<Tr>(acc[fm][fn], bf[fn], a[fm * 2 + kb]);
        }
    };

    if (nsteps > 0) {
        // A is prefetched two steps ahead in a 3-slot ring
        u32x4 abuf[3][4];
        load_b(kbeg);
        load_a(abuf[0], kbeg);
        if (nsteps > 1)
            load_a(abuf[1], kbeg + kSkBK);
        store_b(lds);
        __syncthreads();

        auto body = [&](int t, u32x4 *acur, u32x4 *afar) {
            const bool more = t + 1 < nsteps;
            if (more)
                load_b(kbeg + (t + 1) * kSkBK);
            if (t + 2 < nsteps)
                load_a(afar, kbeg + (t + 2) * kSkBK);
            compute(acur, lds + (t & 1) * STAGE);
            if (more)
                store_b(lds + ((t + 1) & 1) * STAGE);
            __syncthreads();
        };
        for (int t = 0; t < nsteps; t += 3) {
            body(t, abuf[0], abuf[2]);
            if (t + 1 < nsteps)
                body(t + 1, abuf[1], abuf[0]);
            if (t + 2 < nsteps)
                body(t + 2, abuf[2], abuf[1]);
        }
    }

    // ---- sum the four K groups: (kg0 + kg2) + (kg1 + kg3), per row group
    float *red = (float *)lds;  // [4 waves][64 values][64 lanes]
    if (kg >= 2) {
        float *dst = red + ((kg - 2) * 2 + rg) * 64 * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[((i * 8 + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (kg < 2) {
        const float *src = red + (kg * 2 + rg) * 64 * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] += src[((i * 8 + j) * 4 + e) * 64 + lane];
    }
    __syncthreads();
    if (kg == 1) {
        float *dst = red + rg * 64 * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[((i * 8 + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    if (kg != 0)
        return;
    {
        const float *src = red + rg * 64 * 64;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][j][e] += src[((i * 8 + j) * 4 + e) * 64 + lane];
    }

    // ---- epilogue: lane holds C[m][n .. n+3]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int m = row0 + 32 * rg + 16 * i + fr;
        if (m >= p.M)
            continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = 16 * j + 4 * g;
            if (n >= p.N)
                continue;
            if (p.splits > 1) {
                float *dst = p.ws + ((int64_t)z * p.M + m) * p.N + n;
                if (n + 3 < p.N && (p.N & 3) == 0) {
                    *(f32x4 *)dst = acc[i][j];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N)
                            dst[e] = acc[i][j][e];
                }
                continue;
            }
            T v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = Tr::from_f32(apply_epi(acc[i][j][e], p.epi, p.slope));
            T *dst = (T *)p.C + (int64_t)m * p.ldc + n;
            if (p.c_vec && n + 3 < p.N) {
                u32x2 w;
                w[0] = __builtin_bit_cast(uint16_t, v[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, v[1]) << 16);
                w[1] = __builtin_bit_cast(uint16_t, v[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, v[3]) << 16);
                *(u32x2 *)dst = w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n + e < p.N)
                        dst[e] = v[e];
            }
        }
    }
}

}  // namespace tg
