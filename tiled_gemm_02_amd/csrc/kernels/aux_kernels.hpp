// aux_kernels.hpp -- split-K reduction and the K == 0 / alpha == 0 output pass.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace tg {

// C[m][n] = out(sum_{z < splits} ws[z * plane + m * wsld + n]), summed in
// increasing z so the result does not depend on which split finished first
// (the partials may be wider than C: padded products).  Splitting K needs
// this final reduction ("Matrix Multiplication Background User's Guide",
// section 2.3).  One thread per 4 consecutive outputs of a row.
template <typename Tr>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws, int splits,
                                                            int64_t wsld, int64_t plane, int M, int N,
                                                            void *C_, int64_t ldc, OutEpi oe,
                                                            int c_vec)
{
    using T = typename Tr::T;
    T *C = (T *)C_;
    const int nq = (N + 3) >> 2;
    const int64_t total = (int64_t)M * nq;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int m = (int)(idx / nq);
        const int n = (int)(idx - (int64_t)m * nq) * 4;
        const float *src = ws + (int64_t)m * wsld + n;
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        // a row of the sums holds wsld >= N floats, so with wsld and plane multiples
        // of 4 a 4-float read at n < N stays inside it
        const bool vec_in = (wsld & 3) == 0 && (plane & 3) == 0;
        // four splits per round: their loads are in flight together, the sum
        // still runs in increasing split order
        for (int z0 = 0; z0 < splits; z0 += 4) {
            f32x4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (z0 + u < splits) {
                    const float *q = src + (int64_t)(z0 + u) * plane;
                    if (vec_in) {
                        v[u] = *(const f32x4 *)q;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N)
                                v[u][e] = q[e];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (z0 + u < splits) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[e] += v[u][e];
                }
        }
        store_out4<Tr>(C + (int64_t)m * ldc + n, f32x4{s[0], s[1], s[2], s[3]}, N - n, c_vec && n + 3 < N, oe);
    }
}

// K == 0 or alpha == 0: the product term is 0, so C = epi(beta * C) (A and B
// are not read; with beta == 0 this writes epi(0) = 0 and does not read C).
template <typename Tr>
__global__ __launch_bounds__(256) void scale_c_kernel(void *C_, int M, int N, int64_t ldc, OutEpi oe)
{
    using T = typename Tr::T;
    T *C = (T *)C_;
    const int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int m = (int)(idx / N);
        const int n = (int)(idx - (int64_t)m * N);
        T *c = C + (int64_t)m * ldc + n;
        const float c_old = oe.beta != 0.0f ? Tr::to_f32(*c) : 0.0f;
        *c = Tr::from_f32(apply_epi(oe.beta != 0.0f ? oe.beta * c_old : 0.0f, oe.kind, oe.slope));
    }
}

// Aligned copy of one operand: dst (drows x dcols, row-major, ld = dcols, a
// multiple of 16 bytes) gets src (rows x cols, ld = lds, any alignment) in
// its top-left corner and zeros elsewhere.  Zero rows and columns past K add
// nothing to the product.  One thread per 16-byte chunk of dst.
template <typename Tr>
__global__ __launch_bounds__(256) void pack_kernel(const void *src_, int64_t lds, int64_t rows,
                                                   int64_t cols, void *dst_, int64_t drows,
                                                   int64_t dcols)
{
    using W = std::conditional_t<Tr::kBytes == 2, uint16_t, uint32_t>;   // the stored bits
    constexpr int E = 16 / Tr::kBytes;
    const W *src = (const W *)src_;
    W *dst = (W *)dst_;
    const int64_t cpr = dcols / E;
    const int64_t total = drows * cpr;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t r = idx / cpr;
        const int64_t c0 = (idx - r * cpr) * E;
        W v[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[e] = (r < rows && c0 + e < cols) ? src[r * lds + c0 + e] : (W)0;
        *(u32x4 *)(dst + r * dcols + c0) = __builtin_bit_cast(u32x4, v);
    }
}

// Transposing aligned copy of one operand: dst (drows x dcols, row-major,
// ld = dcols, a multiple of 16 bytes) gets the transpose of src (rows x cols,
// ld = lds): dst[i][j] = src[j][i] for i < cols, j < rows, zeros elsewhere.
// A workgroup moves one 64 x 64 block of dst through LDS (rows padded by one
// element so the column reads spread over the banks): it reads the block's
// source rows along their contiguous dimension and writes dst rows four
// elements per thread.
template <typename Tr>
__global__ __launch_bounds__(256) void pack_t_kernel(const void *src_, int64_t lds, int64_t rows,
                                                     int64_t cols, void *dst_, int64_t drows,
                                                     int64_t dcols)
{
    using W = std::conditional_t<Tr::kBytes == 2, uint16_t, uint32_t>;
    typedef W w4 __attribute__((ext_vector_type(4)));
    __shared__ W t[64][65];
    const W *src = (const W *)src_;
    W *dst = (W *)dst_;
    const int64_t bcols = (dcols + 63) / 64;
    const int64_t i0 = (int64_t)(blockIdx.x / bcols) * 64;   // dst rows = src columns
    const int64_t j0 = (int64_t)(blockIdx.x % bcols) * 64;   // dst columns = src rows
    const int tr = threadIdx.x >> 4, tc = (threadIdx.x & 15) * 4;
    const bool vec = ((uintptr_t)src_ % sizeof(w4)) == 0 && (lds & 3) == 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = tr + 16 * q;          // source row j0 + r, columns i0 + tc .. + 3
        const int64_t sr = j0 + r;
        if (vec && sr < rows && i0 + tc + 3 < cols) {
            const w4 v = *(const w4 *)(src + sr * lds + i0 + tc);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                t[r][tc + e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t sc = i0 + tc + e;
                t[r][tc + e] = (sr < rows && sc < cols) ? src[sr * lds + sc] : (W)0;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = tr + 16 * q;          // dst row i0 + r, columns j0 + tc .. + 3
        const int64_t di = i0 + r, dj = j0 + tc;
        if (di < drows && dj < dcols) {
            w4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = t[tc + e][r];
            *(w4 *)(dst + di * dcols + dj) = v;
        }
    }
}

}  // namespace tg
