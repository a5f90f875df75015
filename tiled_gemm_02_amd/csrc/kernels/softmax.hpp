// softmax.hpp -- fused row softmax on gfx950.
//
// Every row x of an M x N row-major matrix becomes
//     y_j = exp(x_j - m) / sum_k exp(x_k - m),   m = max_k x_k
// (the fused-softmax example of "OpenAI open-sources Triton", programming-model
// section: one program per row, the row kept on chip for the whole
// normalisation, columns past N treated as -inf).  Storage float32, float16 or
// bfloat16; all arithmetic in float32.
//
// Row-resident kernel (N up to 32768, about the longest row the page keeps on
// chip).  Q wave64s share a row (Q = 1: four rows per workgroup, one per
// wave); each lane holds C 16-byte chunks of it in registers, chunk c of lane l in wave q covering elements
// ((c Q + q) 64 + l) E .. + E - 1, so every chunk index is one coalesced
// Q x 1 KiB stretch of the row.  The row is read once and written once: all of
// its loads are issued before the first reduction, the maximum and the sum are
// butterfly reductions across the wave (__shfl_xor) and, for Q > 1, across
// its waves through LDS, and exp(x - m) is evaluated as 2^((x - m) log2 e).
// Each lane sums its own C E <= 32 values in sequence before the tree.
// 16-bit rows stay packed in registers and their exponentials are computed
// twice (for the sum and for the output), which halves the registers a row
// needs; the recomputed values are bit-identical to the first ones.
//
// Long rows (N > 32768): one 1024-thread workgroup per row makes two passes.
// The first keeps, per thread, a running maximum and a sum of exponentials
// rescaled whenever the maximum grows, over steps of four chunks per lane; the
// (max, sum) pairs are then combined across the workgroup.  The second pass
// reads the row again and writes the outputs.
//
// NaN and infinities follow the definition's arithmetic: a row holding NaN or
// +inf, or made only of -inf, comes out NaN; -inf entries of a finite row give
// 0.  Rows are independent, and a row is read completely before any of it is
// written, so Y may be X itself (same leading dimension).
#pragma once

#include "common.hpp"

#include <math.h>

namespace tg {

struct SoftmaxArgs {
    const void *X;
    void *Y;
    int64_t ldx, ldy;  // elements between consecutive rows
    int64_t M;
    int N;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSoftmaxLongThreads = 1024;

__device__ __forceinline__ float sm_wave_max(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ float sm_wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

// Cache policy of the 16-byte row accesses (a bit set: non-temporal, i.e.
// streamed past the caches).  Chosen per launch shape from measurements.
enum : int { kSmNtStore = 1, kSmNtLoad = 2 };

template <int CP>
__device__ __forceinline__ u32x4 sm_ld16(const void *p)
{
    if constexpr ((CP & kSmNtLoad) != 0)
        return __builtin_nontemporal_load((const u32x4 *)p);
    else
        return *(const u32x4 *)p;
}

template <int CP>
__device__ __forceinline__ void sm_st16(void *p, const u32x4 &c)
{
    if constexpr ((CP & kSmNtStore) != 0)
        __builtin_nontemporal_store(c, (u32x4 *)p);
    else
        *(u32x4 *)p = c;
}

// E consecutive elements starting at j0 of a row, as float32; elements at or
// past N read as -inf.  VEC: the row start is 16-byte aligned.  (Indices are
// 32-bit: a row segment holds fewer than 2^31 elements.)
template <typename Tr, bool VEC, int CP = 0>
__device__ __forceinline__ void sm_load(const typename Tr::T *row, int j0, int N,
                                        float (&v)[Tr::E])
{
    constexpr int E = Tr::E;
    if (VEC && j0 + E <= N) {
        const u32x4 c = sm_ld16<CP>(row + j0);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t bits = chunk_elem<Tr::kBytes>(c, e);
            if constexpr (Tr::kBytes == 4)
                v[e] = u32_as_f32(bits);
            else
                v[e] = Tr::to_f32(__builtin_bit_cast(typename Tr::T, (uint16_t)bits));
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[e] = (j0 + e < N) ? Tr::to_f32(row[j0 + e]) : -INFINITY;
    }
}

template <typename Tr, bool VEC, int CP = 0>
__device__ __forceinline__ void sm_store(typename Tr::T *row, int j0, int N,
                                         const float (&v)[Tr::E])
{
    constexpr int E = Tr::E;
    using T = typename Tr::T;
    if (VEC && j0 + E <= N) {
        u32x4 c;
        if constexpr (Tr::kBytes == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                c[e] = __builtin_bit_cast(uint32_t, v[e]);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t lo = __builtin_bit_cast(uint16_t, Tr::from_f32(v[2 * w]));
                const uint32_t hi = __builtin_bit_cast(uint16_t, Tr::from_f32(v[2 * w + 1]));
                c[w] = lo | (hi << 16);
            }
        }
        sm_st16<CP>(row + j0, c);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (j0 + e < N)
                row[j0 + e] = Tr::from_f32(v[e]);
    }
}

template <int Q>
constexpr int sm_rows_per_block() { return Q >= 4 ? 1 : 4 / Q; }

// One 16-byte chunk of a 16-bit row as raw bits (8 elements), elements at or
// past N filled with -inf.  Rows of 16-bit values stay in registers in this
// packed form (half the registers of float32 copies): every pass converts
// them again, and the exponentials are recomputed for the output.
template <typename Tr, bool VEC, int CP>
__device__ __forceinline__ u32x4 sm_load_raw16(const typename Tr::T *row, int j0, int N)
{
    static_assert(Tr::kBytes == 2, "16-bit storage");
    if (VEC && j0 + 8 <= N)
        return sm_ld16<CP>(row + j0);
    const uint32_t ninf = __builtin_bit_cast(uint16_t, Tr::from_f32(-INFINITY));
    const uint16_t *r16 = (const uint16_t *)row;
    u32x4 c;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t lo = (j0 + 2 * w < N) ? r16[j0 + 2 * w] : ninf;
        const uint32_t hi = (j0 + 2 * w + 1 < N) ? r16[j0 + 2 * w + 1] : ninf;
        c[w] = lo | (hi << 16);
    }
    return c;
}

template <typename Tr>
__device__ __forceinline__ float sm_raw16_f32(const u32x4 &c, int e)
{
    return Tr::to_f32(__builtin_bit_cast(typename Tr::T, (uint16_t)chunk_elem<2>(c, e)));
}

// Sixteen-wave rows ask for two resident workgroups per CU (64 registers per
// lane), so that one row's loads overlap the other's reductions and stores
// (the element-wise form, for unaligned rows, would spill at 64).
template <int Q, bool VEC>
constexpr int sm_waves_per_eu() { return Q == 16 && VEC ? 8 : 1; }

// CP: cache policy of the row's 16-byte loads and stores (kSmNt* bits).
template <typename Tr, int Q, int C, bool VEC, int CP>
__global__ __launch_bounds__(64 * Q * sm_rows_per_block<Q>())
__attribute__((amdgpu_waves_per_eu(sm_waves_per_eu<Q, VEC>()))) void softmax_rows_kernel(SoftmaxArgs p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using T = typename Tr::T;
    constexpr int E = Tr::E;
    constexpr bool RAW = Tr::kBytes == 2;
    constexpr int RPB = sm_rows_per_block<Q>();
    static_assert(C * E <= 32, "at most 32 values per lane (registers; sequential part of the sum)");
    __shared__ float red[2][RPB][Q];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rs = wave / Q, qw = wave % Q;
    const int64_t r = (int64_t)blockIdx.x * RPB + rs;
    const bool active = r < p.M;   // every wave still takes part in the barriers
    const T *x = (const T *)p.X + (active ? r : 0) * p.ldx;
    T *y = (T *)p.Y + (active ? r : 0) * p.ldy;
    const int N = active ? p.N : 0;

    // the row: float32 values, or packed 16-bit chunks
    float v[RAW ? 1 : C][E];
    u32x4 raw[RAW ? C : 1];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j0 = ((c * Q + qw) * 64 + lane) * E;
        if constexpr (RAW)
            raw[c] = sm_load_raw16<Tr, VEC, CP>(x, j0, N);
        else
            sm_load<Tr, VEC, CP>(x, j0, N, v[c]);
    }
    auto val = [&](int c, int e) -> float {
        if constexpr (RAW)
            return sm_raw16_f32<Tr>(raw[c], e);
        else
            return v[c][e];
    };

    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e)
            mx = fmaxf(mx, val(c, e));
    mx = sm_wave_max(mx);
    if constexpr (Q > 1) {
        if (lane == 0)
            red[0][rs][qw] = mx;
        __syncthreads();
        mx = red[0][rs][0];
#pragma unroll
        for (int q = 1; q < Q; ++q)
            mx = fmaxf(mx, red[0][rs][q]);
    }

    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float ex = exp2f((val(c, e) - mx) * kLog2e);
            if constexpr (!RAW)
                v[c][e] = ex;
            s += ex;
        }
    s = sm_wave_sum(s);
    if constexpr (Q > 1) {
        if (lane == 0)
            red[1][rs][qw] = s;
        __syncthreads();
        // the same pairwise tree in every wave, so all of them hold the same sum
        float t[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q)
            t[q] = red[1][rs][q];
#pragma unroll
        for (int w = Q / 2; w >= 1; w /= 2)
#pragma unroll
            for (int q = 0; q < w; ++q)
                t[q] += t[q + w];
        s = t[0];
    }
    const float inv = 1.0f / s;

    if (active) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if constexpr (RAW)
                    o[e] = exp2f((val(c, e) - mx) * kLog2e) * inv;
                else
                    o[e] = v[c][e] * inv;
            }
            sm_store<Tr, VEC, CP>(y, ((c * Q + qw) * 64 + lane) * E, N, o);
        }
    }
#endif
}

// Combine per-thread (max, sum) pairs of a 1024-thread workgroup: returns the
// row maximum in *m and the row sum rescaled to it.
__device__ __forceinline__ float sm_block_combine(float &m, float s, float *red_m, float *red_s)
{
    constexpr int NW = kSoftmaxLongThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float M = sm_wave_max(m);
    if (lane == 0)
        red_m[wave] = M;
    __syncthreads();
    M = red_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        M = fmaxf(M, red_m[w]);
    // a thread that saw only -inf has s = 0 and contributes 0 (exp2(-inf) = 0)
    // unless the whole row is -inf, where the definition's NaN comes out
    float t = s * exp2f((m - M) * kLog2e);
    t = sm_wave_sum(t);
    if (lane == 0)
        red_s[wave] = t;
    __syncthreads();
    float u[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w)
        u[w] = red_s[w];
#pragma unroll
    for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
        for (int w = 0; w < h; ++w)
            u[w] += u[w + h];
    m = M;
    return u[0];
}

template <typename Tr, bool VEC>
__global__ __launch_bounds__(kSoftmaxLongThreads) void softmax_long_kernel(SoftmaxArgs p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using T = typename Tr::T;
    constexpr int E = Tr::E;
    constexpr int U = 4;                                  // chunks per lane per step
    constexpr int64_t STEP = (int64_t)kSoftmaxLongThreads * U * E;
    __shared__ float red_m[kSoftmaxLongThreads / 64], red_s[kSoftmaxLongThreads / 64];

    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;   // grid = M
    const T *x = (const T *)p.X + r * p.ldx;
    T *y = (T *)p.Y + r * p.ldy;
    const int64_t N = p.N;

    float m = -INFINITY, s = 0.0f;
    for (int64_t base = 0; base < N; base += STEP) {
        const int rem = (int)min<int64_t>(N - base, STEP);
        float v[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u)
            sm_load<Tr, VEC>(x + base, (u * kSoftmaxLongThreads + tid) * E, rem, v[u]);
        float cm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                cm = fmaxf(cm, v[u][e]);
        const float mn = fmaxf(m, cm);
        if (mn != -INFINITY) {   // nothing but -inf so far: the sum stays 0
            float t = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    t += exp2f((v[u][e] - mn) * kLog2e);
            s = s * exp2f((m - mn) * kLog2e) + t;
            m = mn;
        }
    }
    const float S = sm_block_combine(m, s, red_m, red_s);
    const float inv = 1.0f / S;

    for (int64_t base = 0; base < N; base += STEP) {
        const int rem = (int)min<int64_t>(N - base, STEP);
        float v[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u)
            sm_load<Tr, VEC>(x + base, (u * kSoftmaxLongThreads + tid) * E, rem, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = exp2f((v[u][e] - m) * kLog2e) * inv;
            sm_store<Tr, VEC>(y + base, (u * kSoftmaxLongThreads + tid) * E, rem, v[u]);
        }
    }
#endif
}

}  // namespace tg
