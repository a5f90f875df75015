// aux_kernels.hpp -- split-K reduction and the K == 0 fill.
#pragma once

#include "common.hpp"

namespace tg {

// C[m][n] = epi( sum_{z < splits} ws[z][m][n] ), summed in increasing z so the
// result does not depend on which split finished first.  Splitting K needs
// this final reduction ("Matrix Multiplication Background User's Guide",
// section 2.3).  One thread per 4 consecutive outputs of a row.
template <typename Tr>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws, int splits,
                                                            int M, int N, void *C_, int64_t ldc,
                                                            int epi, float slope, int c_vec)
{
    using T = typename Tr::T;
    T *C = (T *)C_;
    const int nq = (N + 3) >> 2;
    const int64_t total = (int64_t)M * nq;
    const int64_t plane = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int m = (int)(idx / nq);
        const int n = (int)(idx - (int64_t)m * nq) * 4;
        const float *src = ws + (int64_t)m * N + n;
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        const bool vec_in = (N & 3) == 0;
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
        T *dst = C + (int64_t)m * ldc + n;
        T v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = Tr::from_f32(apply_epi(s[e], epi, slope));
        if (c_vec && n + 3 < N) {
            if constexpr (Tr::kBytes == 2) {
                u32x2 w;
                w[0] = __builtin_bit_cast(uint16_t, v[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, v[1]) << 16);
                w[1] = __builtin_bit_cast(uint16_t, v[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, v[3]) << 16);
                *(u32x2 *)dst = w;
            } else {
                *(f32x4 *)dst = f32x4{v[0], v[1], v[2], v[3]};
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N)
                    dst[e] = v[e];
        }
    }
}

// K == 0: the empty sum is 0 and both epilogues map 0 to 0.
template <typename Tr>
__global__ __launch_bounds__(256) void fill_zero_kernel(void *C_, int M, int N, int64_t ldc)
{
    using T = typename Tr::T;
    T *C = (T *)C_;
    const int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int m = (int)(idx / N);
        const int n = (int)(idx - (int64_t)m * N);
        C[(int64_t)m * ldc + n] = Tr::from_f32(0.0f);
    }
}

}  // namespace tg
