// launch.hpp -- host-side launchers of the kernel instances (one translation
// unit per storage type instantiates them).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemv.hpp"
#include "mfma_gemm.hpp"
#include "skinny.hpp"
#include "softmax.hpp"

namespace tg {

// The register-staged kernel; kg = K groups per workgroup.  hipErrorInvalidValue:
// no instance for this (type, tile, load width, K groups).
hipError_t launch_mfma(int dtype, int trans, int bm, int bn, bool vec, int kg, const MfmaArgs &a,
                       hipStream_t s);
// Resident workgroups per CU of an instance (0 if none).
int mfma_occupancy(int dtype, int trans, int bm, int bn, bool vec, int kg);
// The LDS-DMA kernel for 16-bit, 16-byte-aligned operands (same tiles); kg = K
// groups per workgroup (1, or 2 for the tiles built with two).
hipError_t launch_mfma2(int dtype, int trans, int bm, int bn, int kg, const MfmaArgs &a, hipStream_t s);
int mfma2_occupancy(int dtype, int trans, int bm, int bn, int kg);
// Stream-K with 256 x 256 tiles on a.splits workgroups (16-bit, aligned), then
// the fix-up of the split tiles; a.ws holds 2 * a.splits float32 tiles.
hipError_t launch_mfma2_sk(int dtype, int trans, const MfmaArgs &a, hipStream_t s);
// C (M x N) = out(sum of `splits` float32 planes of partials, rows wsld apart)
hipError_t launch_splitk_reduce(int dtype, const float *ws, int splits, int64_t wsld, int64_t plane,
                                int M, int N, void *C, int64_t ldc, const OutEpi &oe, int c_vec,
                                hipStream_t s);
// Aligned, zero-padded copy of a rows x cols operand into drows x dcols.
// transposed: dst (drows x dcols) gets the transpose of src (rows x cols) instead.
hipError_t launch_pack(int dtype, const void *src, int64_t lds, int64_t rows, int64_t cols, void *dst,
                       int64_t drows, int64_t dcols, hipStream_t s, bool transposed = false);
// C = epi(beta * C): K == 0 or alpha == 0.
hipError_t launch_scale_c(int dtype, void *C, int M, int N, int64_t ldc, const OutEpi &oe,
                          hipStream_t s);
// rows_form: outputs are contiguous dot products; else column streaming.
// lpr: lanes per row segment of the vector cols kernel (columns per workgroup = lpr x
// elements per 16 bytes).
hipError_t launch_gemv(int dtype, bool rows_form, bool vec, int lpr, const GemvArgs &a,
                       hipStream_t s);
hipError_t launch_skinny(int dtype, bool trans_b, const SkinnyArgs &a, hipStream_t s);
// Row softmax: q waves per row and c 16-byte chunks per lane (row kept in
// registers), or q == 0 for the two-pass long-row kernel.
hipError_t launch_softmax(int dtype, int q, int c, bool vec, const SoftmaxArgs &a, hipStream_t s);

#define TG_DECLARE_TYPE_LAUNCHERS(NAME)                                                          \
    hipError_t launch_mfma_##NAME(int trans, int bm, int bn, bool vec, int kg, const MfmaArgs &a, \
                                  hipStream_t s);                                                \
    int mfma_occupancy_##NAME(int trans, int bm, int bn, bool vec, int kg);                      \
    hipError_t launch_splitk_reduce_##NAME(const float *ws, int splits, int64_t wsld,            \
                                           int64_t plane, int M, int N, void *C, int64_t ldc,    \
                                           OutEpi oe, int c_vec, hipStream_t s);                 \
    hipError_t launch_pack_##NAME(const void *src, int64_t lds, int64_t rows, int64_t cols,      \
                                  void *dst, int64_t drows, int64_t dcols, hipStream_t s);       \
    hipError_t launch_pack_t_##NAME(const void *src, int64_t lds, int64_t rows, int64_t cols,    \
                                    void *dst, int64_t drows, int64_t dcols, hipStream_t s);     \
    hipError_t launch_scale_c_##NAME(void *C, int M, int N, int64_t ldc, OutEpi oe,             \
                                     hipStream_t s);                                             \
    hipError_t launch_gemv_##NAME(bool rows_form, bool vec, int lpr, const GemvArgs &a,          \
                                  hipStream_t s);                                                \
    hipError_t launch_skinny_##NAME(bool trans_b, const SkinnyArgs &a, hipStream_t s);           \
    hipError_t launch_mfma2_##NAME(int trans, int bm, int bn, int kg, const MfmaArgs &a,         \
                                   hipStream_t s);                                               \
    int mfma2_occupancy_##NAME(int trans, int bm, int bn, int kg);                               \
    hipError_t launch_mfma2_sk_##NAME(int trans, const MfmaArgs &a, hipStream_t s);              \
    hipError_t launch_softmax_##NAME(int q, int c, bool vec, const SoftmaxArgs &a, hipStream_t s);

TG_DECLARE_TYPE_LAUNCHERS(f16)
TG_DECLARE_TYPE_LAUNCHERS(bf16)
TG_DECLARE_TYPE_LAUNCHERS(f32)

}  // namespace tg
