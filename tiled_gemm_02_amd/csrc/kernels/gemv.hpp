// gemv.hpp -- matrix-vector products (M == 1 or N == 1) on the vector ALUs.
//
// A product with M == 1 or N == 1 does about one multiply-add per matrix
// element loaded, an arithmetic intensity below 1 FLOP/byte, so it is bound
// by memory traffic on any GPU ("Matrix Multiplication Background User's
// Guide", section 2).  These kernels use no matrix cores: they stream the
// matrix once with coalesced 128-bit loads, multiply-add in float32 on the
// vector ALUs and reduce across lanes, waves and K-splits.
//
// Two shapes cover every storage combination:
//   cols: out(j) = sum_k v(k) * X[k][j]   X row-major K x n (contiguous along j)
//   rows: out(i) = sum_k X[i][k] * v(k)   X row-major n x K (contiguous along k)
// v(k) = V[k * vs] and out(j) = O[j * os] allow strided vectors.
#pragma once

#include "common.hpp"

namespace tg {

struct GemvArgs {
    const void *X;
    int64_t ldx;
    const void *V;
    int64_t vs;
    void *O;
    int64_t os;
    float *ws;       // [ksplit][n] float32 partials when ksplit > 1
    int n;           // output length
    int K;
    int ksplit;
    int rows_per_split;
    OutEpi oe;       // output transform
};

// out(j) = epi(alpha * acc + beta * out_old(j))
template <typename Tr>
__device__ __forceinline__ void gemv_store(const GemvArgs &p, int64_t j, float acc)
{
    using T = typename Tr::T;
    T *o = (T *)p.O + j * p.os;
    const float c_old = p.oe.beta != 0.0f ? Tr::to_f32(*o) : 0.0f;
    *o = Tr::from_f32(out_value(p.oe, acc, c_old));
}

template <typename Tr>
__device__ __forceinline__ float load_scalar(const void *p, int64_t i)
{
    return Tr::to_f32(((const typename Tr::T *)p)[i]);
}

// Unpack a 16-byte chunk into E floats.
template <typename Tr>
__device__ __forceinline__ void unpack(const u32x4 &c, float *f)
{
    if constexpr (Tr::kBytes == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = c[e];
            f[e] = u32_as_f32(w);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t h = (uint16_t)chunk_elem<2>(c, e);
            f[e] = Tr::to_f32(__builtin_bit_cast(typename Tr::T, h));
        }
    }
}

// cols form, vector path.  A workgroup owns one strip of LPR * E columns
// (each lane 16 bytes of a row, LPR lanes per row, so a row segment is LPR x
// 16 bytes) over a K range; its 256 lanes cover 256 / LPR rows per load, and
// each lane keeps 8 rows in flight.  The matrix is read once, so its loads are
// non-temporal (they do not displace cached data).  Partial column sums are
// combined across the lanes of a wave by a butterfly over the row-selecting
// lane bits, then across the 4 waves in wave order; with one K range the
// result is final, otherwise it is a partial for the reduction kernel.
template <typename Tr, int LPR>
__global__ __launch_bounds__(256) void gemv_cols_kernel(GemvArgs p)
{
    using T = typename Tr::T;
    constexpr int E = Tr::E;
    constexpr int RPW = 64 / LPR;    // row slots per wave
    constexpr int SLOTS = 4 * RPW;   // row slots per workgroup
    constexpr int U = 8;             // rows in flight per lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane % LPR;
    const int slot = wave * RPW + lane / LPR;
    const int col = (blockIdx.x * LPR + q) * E;
    const int k_lo = blockIdx.y * p.rows_per_split;
    const int k_hi = min(p.K, k_lo + p.rows_per_split);
    const T *base = (const T *)p.X + col;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.f;

    // the chunk holding column n - 1 may end past n (n need not be a multiple
    // of E, and the matrix may end at column n of its last row): that lane
    // loads it element by element
    if (col + E <= p.n) {
        int k = k_lo + slot;
        for (; k + (U - 1) * SLOTS < k_hi; k += U * SLOTS) {
            u32x4 x[U];
            float a[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x[u] = __builtin_nontemporal_load((const u32x4 *)(base + (int64_t)(k + u * SLOTS) * p.ldx));
                a[u] = load_scalar<Tr>(p.V, (int64_t)(k + u * SLOTS) * p.vs);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[E];
                unpack<Tr>(x[u], f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    acc[e] += a[u] * f[e];
            }
        }
        for (; k < k_hi; k += SLOTS) {
            const u32x4 x = __builtin_nontemporal_load((const u32x4 *)(base + (int64_t)k * p.ldx));
            const float a = load_scalar<Tr>(p.V, (int64_t)k * p.vs);
            float f[E];
            unpack<Tr>(x, f);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] += a * f[e];
        }
    } else if (col < p.n) {
        for (int k = k_lo + slot; k < k_hi; k += SLOTS) {
            const float a = load_scalar<Tr>(p.V, (int64_t)k * p.vs);
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (col + e < p.n)
                    acc[e] += a * Tr::to_f32(base[(int64_t)k * p.ldx + e]);
        }
    }

    // lanes q, q + LPR, q + 2 LPR, ... hold the same columns
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] += __shfl_xor(acc[e], off, 64);

    __shared__ float red[4][LPR * E];
    if (lane < LPR) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            red[wave][lane * E + e] = acc[e];
    }
    __syncthreads();
    if (wave != 0 || lane >= LPR || col >= p.n)
        return;
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        s[e] = ((red[0][lane * E + e] + red[1][lane * E + e]) + red[2][lane * E + e]) +
               red[3][lane * E + e];
    if (p.ksplit > 1) {
        float *W = p.ws + (int64_t)blockIdx.y * p.n + col;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < p.n)
                W[e] = s[e];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < p.n)
                gemv_store<Tr>(p, col + e, s[e]);
    }
}

// cols form, element-wise path (unaligned or ragged operands).  Grid: x =
// strips of 64 * E columns, y = K-splits; the 4 waves take interleaved rows of
// the split's K range and are summed in wave order through LDS.
template <typename Tr>
__global__ __launch_bounds__(256) void gemv_cols_generic_kernel(GemvArgs p)
{
    using T = typename Tr::T;
    constexpr int E = Tr::E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = (blockIdx.x * 64 + lane) * E;
    const int k_lo = blockIdx.y * p.rows_per_split;
    const int k_hi = min(p.K, k_lo + p.rows_per_split);
    const T *X = (const T *)p.X;

    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.f;
    const bool col_in = col < p.n;
    if (col_in) {
        for (int k = k_lo + wave; k < k_hi; k += 4) {
            const float a = load_scalar<Tr>(p.V, (int64_t)k * p.vs);
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (col + e < p.n)
                    acc[e] += a * Tr::to_f32(X[(int64_t)k * p.ldx + col + e]);
        }
    }

    // sum the 4 waves in order 0..3
    __shared__ float red[4][64 * E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        red[wave][e * 64 + lane] = acc[e];
    __syncthreads();
    if (wave != 0 || !col_in)
        return;
    float s[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        s[e] = ((red[0][e * 64 + lane] + red[1][e * 64 + lane]) + red[2][e * 64 + lane]) +
               red[3][e * 64 + lane];
    if (p.ksplit > 1) {
        float *W = p.ws + (int64_t)blockIdx.y * p.n;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < p.n)
                W[col + e] = s[e];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (col + e < p.n)
                gemv_store<Tr>(p, col + e, s[e]);
    }
}

// out(j) = epi( sum_{z < ksplit} ws[z][j] ), increasing z.
template <typename Tr>
__global__ __launch_bounds__(256) void gemv_reduce_kernel(GemvArgs p)
{
    using T = typename Tr::T;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= p.n)
        return;
    const float *w = p.ws + j;
    float s = 0.f;
    // sixteen splits per round: their loads are in flight together, the sum
    // still runs in increasing z
    for (int z0 = 0; z0 < p.ksplit; z0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            v[u] = z0 + u < p.ksplit ? w[(int64_t)(z0 + u) * p.n] : 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (z0 + u < p.ksplit)
                s += v[u];
    }
    gemv_store<Tr>(p, j, s);
}

// rows form.  One wave per output: lanes stride over 16-byte chunks of the
// row, then a butterfly reduction across the wave.  Grid: n / 4 workgroups.
template <typename Tr, bool VEC>
__global__ __launch_bounds__(256) void gemv_rows_kernel(GemvArgs p)
{
    using T = typename Tr::T;
    constexpr int E = Tr::E;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = blockIdx.x * 4 + wave;
    if (i >= p.n)
        return;
    const T *row = (const T *)p.X + (int64_t)i * p.ldx;
    const T *V = (const T *)p.V;
    float acc = 0.f;
    const int nchunks = VEC ? p.K / E : 0;
    int c = lane;
    for (; c + 192 < nchunks; c += 256) {
        u32x4 x[4], v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            x[u] = __builtin_nontemporal_load((const u32x4 *)(row + (int64_t)(c + 64 * u) * E));
            v[u] = *(const u32x4 *)(V + (int64_t)(c + 64 * u) * E);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float fx[E], fv[E];
            unpack<Tr>(x[u], fx);
            unpack<Tr>(v[u], fv);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc += fx[e] * fv[e];
        }
    }
    for (; c < nchunks; c += 64) {
        const u32x4 x = *(const u32x4 *)(row + (int64_t)c * E);
        const u32x4 v = *(const u32x4 *)(V + (int64_t)c * E);
        float fx[E], fv[E];
        unpack<Tr>(x, fx);
        unpack<Tr>(v, fv);
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc += fx[e] * fv[e];
    }
    // element-wise remainder (or the whole row without vector access)
    for (int k = nchunks * E + lane; k < p.K; k += 64)
        acc += Tr::to_f32(row[k]) * load_scalar<Tr>(p.V, (int64_t)k * p.vs);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        acc += __shfl_xor(acc, off, 64);
    if (lane == 0)
        gemv_store<Tr>(p, i, acc);
}

}  // namespace tg
