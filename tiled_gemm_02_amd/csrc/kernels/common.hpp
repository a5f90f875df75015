// common.hpp -- storage-type traits, conversions and small helpers shared by
// the gfx950 GEMM kernels.  CDNA4 only: 64-lane wavefronts, MFMA matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Epilogue codes (same values as the public tg_epi_kind).
enum : int { kEpiNone = 0, kEpiLeaky = 1 };

__device__ __forceinline__ float apply_epi(float x, int epi, float slope)
{
    // leaky rectifier on the float32 value, before output rounding
    return (epi == kEpiLeaky && x < 0.0f) ? x * slope : x;
}

// The output transform every kernel applies when it writes C:
//     C = epi(alpha * acc + beta * C_old),
// formed in float32 before the single rounding; C_old is read only when
// beta != 0 (with beta == 0 it may hold anything).  alpha = 1, beta = 0 leave
// acc unchanged bit for bit.
struct OutEpi {
    int kind;      // kEpiNone / kEpiLeaky
    float slope;
    float alpha;
    float beta;
};

__device__ __forceinline__ float out_value(const OutEpi &oe, float acc, float c_old)
{
    float x = oe.alpha * acc;
    if (oe.beta != 0.0f)
        x += oe.beta * c_old;
    return apply_epi(x, oe.kind, oe.slope);
}

// out_value where the caller knows beta is 0 (no old C): without that
// knowledge the compiler keeps the beta term's multiply and test per element.
__device__ __forceinline__ float out_value_no_c(const OutEpi &oe, float acc)
{
    return apply_epi(oe.alpha * acc, oe.kind, oe.slope);
}

// Bit reinterpretation of one 32-bit lane value.  The argument is taken by
// value: bit-casting a vector-element expression (v[i]) directly has been seen
// to read element 0 whatever i is, so callers copy the element out first.
__device__ __forceinline__ float u32_as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// ---------------------------------------------------------------- storage types
//
// Each trait describes one storage type: its element, how many elements a
// 16-byte chunk holds (E), the K depth of one 16-byte-per-lane MFMA step, and
// the conversion of a float32 result to storage (round to nearest even).

struct F16 {
    using T = _Float16;
    static constexpr int kBytes = 2;
    static constexpr int E = 8;   // elements per 16-byte chunk
    static constexpr int code = 1;
    __device__ static __forceinline__ T from_f32(float x) { return (T)x; }
    __device__ static __forceinline__ float to_f32(T x) { return (float)x; }
};

struct BF16 {
    using T = __bf16;
    static constexpr int kBytes = 2;
    static constexpr int E = 8;
    static constexpr int code = 2;
    __device__ static __forceinline__ T from_f32(float x) { return (T)x; }
    __device__ static __forceinline__ float to_f32(T x) { return (float)x; }
};

struct F32 {
    using T = float;
    static constexpr int kBytes = 4;
    static constexpr int E = 4;
    static constexpr int code = 0;
    __device__ static __forceinline__ T from_f32(float x) { return x; }
    __device__ static __forceinline__ float to_f32(T x) { return x; }
};

// One 16x16 output block of a 16-byte-per-lane k-step:
//   acc[n-row 4*(lane/16)+i][m-col lane%16] += sum_k bop[n][k] * aop[k][m]
// For 16-bit types this is one v_mfma_f32_16x16x32; for float32 the chunk
// holds four k values, consumed by four v_mfma_f32_16x16x4 steps.  Both
// operands take their k values from the same lane group (lane / 16) and
// element position, so the pairing of A and B along k is consistent.
template <typename Tr>
__device__ __forceinline__ void mfma_chunk(f32x4 &acc, const u32x4 &bop, const u32x4 &aop);

template <>
__device__ __forceinline__ void mfma_chunk<F16>(f32x4 &acc, const u32x4 &bop, const u32x4 &aop)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, bop),
                                                 __builtin_bit_cast(f16x8, aop), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_chunk<BF16>(f32x4 &acc, const u32x4 &bop, const u32x4 &aop)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bop),
                                                  __builtin_bit_cast(bf16x8, aop), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_chunk<F32>(f32x4 &acc, const u32x4 &bop, const u32x4 &aop)
{
#pragma unroll
    for (int e = 0; e < 4; ++e)
    {
        const uint32_t b = bop[e], a = aop[e];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(u32_as_f32(b), u32_as_f32(a), acc, 0, 0, 0);
    }
}

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Element e of a 16-byte chunk, as raw bits of the storage type.
template <int BYTES>
__device__ __forceinline__ uint32_t chunk_elem(const u32x4 &c, int e)
{
    if constexpr (BYTES == 4) {
        return c[e];
    } else {
        uint32_t w = c[e >> 1];
        return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    }
}

// Transpose an E x E block held as E chunks (chunk r = row r, E elements):
// out chunk j holds element j of every input chunk, in row order.
template <int BYTES>
__device__ __forceinline__ void transpose_block(const u32x4 *in, u32x4 *out)
{
    if constexpr (BYTES == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            out[j] = u32x4{in[0][j], in[1][j], in[2][j], in[3][j]};
    } else {
        // 8 x 8 of 16-bit values.  out[j] pairs rows (2p, 2p+1) at column j:
        // low half from row 2p, high half from row 2p+1.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int w = j >> 1;
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            u32x4 o;
#pragma unroll
            for (int p = 0; p < 4; ++p)
                o[p] = __builtin_amdgcn_perm(in[2 * p + 1][w], in[2 * p][w], sel);
            out[j] = o;
        }
    }
}

// Writes out_value(acc[e], C_old[e]) to dst[0 .. 3] of one row of C, skipping
// elements at or past `avail` (columns left in the row).  vec: the four
// elements are one aligned group (8 bytes of 16-bit values, 16 of float32)
// wholly inside the row; then C_old is read and C written with one access each.
template <typename Tr>
__device__ __forceinline__ void store_out4(typename Tr::T *dst, const f32x4 &acc, int avail, bool vec,
                                           const OutEpi &oe)
{
    using T = typename Tr::T;
    float c_old[4] = {0.f, 0.f, 0.f, 0.f};
    if (oe.beta != 0.0f) {
        if (vec) {
            if constexpr (Tr::kBytes == 2) {
                const u32x2 w = *(const u32x2 *)dst;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t word = w[e >> 1];
                    c_old[e] = Tr::to_f32(__builtin_bit_cast(T, (uint16_t)(word >> (16 * (e & 1)))));
                }
            } else {
                const f32x4 v = *(const f32x4 *)dst;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    c_old[e] = v[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < avail)
                    c_old[e] = Tr::to_f32(dst[e]);
        }
    }
    T o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = Tr::from_f32(out_value(oe, acc[e], c_old[e]));
    if (vec) {
        if constexpr (Tr::kBytes == 2) {
            u32x2 w;
            w[0] = (uint32_t)__builtin_bit_cast(uint16_t, o[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, o[1]) << 16);
            w[1] = (uint32_t)__builtin_bit_cast(uint16_t, o[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, o[3]) << 16);
            *(u32x2 *)dst = w;
        } else {
            *(f32x4 *)dst = f32x4{o[0], o[1], o[2], o[3]};
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < avail)
                dst[e] = o[e];
    }
}

// ceil-division on non-negative integers
__host__ __device__ constexpr inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tg
