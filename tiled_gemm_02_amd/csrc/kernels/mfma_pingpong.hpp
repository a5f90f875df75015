// mfma_pingpong.hpp -- 256 x 256 macro-tile GEMM with two wave groups that
// alternate between loading and multiplying: 16-bit operands in every layout,
// and float32 operands when A and B are both K-contiguous (a float32 value is
// copied as two 16-bit units, so a stage row holds 16 values of K and a phase
// is 128 v_mfma_f32_16x16x4f32 per wave).
//
// Tiling ("Matrix Multiplication Background User's Guide", section 2.1): one
// 256 x 256 tile of C per workgroup, eight wave64s in a 2 x 4 grid, each wave
// owning 128 x 64 of the tile (8 x 4 blocks of v_mfma_f32_16x16x32, fp32
// accumulate, 128 accumulator registers per lane).  K advances in 32-deep stages (one
// MFMA K block each, 32 KiB of LDS), S of them buffered, copied by the LDS-DMA
// path of mfma_gemm3.hpp (K-contiguous rows of 64 bytes).
//
// Schedule.  Waves 0-3 (group 0, tile rows 0-127) and 4-7 (group 1, rows
// 128-255) share the four SIMDs, one wave of each per SIMD.  Time is cut into
// phases separated by a workgroup barrier.  In every phase one group
// multiplies a stage - 32 MFMAs back to back on fragments already in
// registers, at raised wave priority - while the other group loads its next
// stage's fragments from LDS into the same registers.  Group g loads stage b
// in phase 2b + g and multiplies it in phase 2b + g + 1, so each SIMD's matrix
// unit always has one wave with nothing to wait for, and the LDS reads, the
// copy issue and their latencies hide behind the other wave's MFMAs.
//
// 192 x 256 tiles (K-contiguous 16-bit A): each wave owns 96 x 64 (6 x 4
// blocks), group 0 copies three 1 KiB pieces of A per stage and group 1 four
// of B, so each group waits for its own count.
//
// Copies.  Group 0 copies A, group 1 copies B.  In its load phase of stage b a
// group refills the buffer of stage b - 2 with stage b + S - 2.  Stage b - 2
// was last read in phase 2b - 3, and those reads completed before the MFMAs
// of phase 2b - 2 used them, so a load phase never has to wait for its own
// LDS reads: it issues them and goes on to the barrier, and the reads land
// while the phase turns over (the MFMAs that need them wait, if at all, at the
// start of the next phase).  Stage b + S - 2 is first read in phase
// 2b + 2S - 4: the copies have 2S - 5 phases or more to land, enough to cover
// the latency of lines that miss L2 (about a fifth of them for 32 concurrent
// tiles per XCD).  Before the barrier that opens phase 2b + 2 each wave waits
// for its own copies of stage b + 1, leaving the younger stages in flight.
//
// Edges: rows and columns past M and N are clamped (computed, never stored);
// a partial 32-deep stage (K not a multiple of 32) is processed first, loaded
// through registers with a zero mask.
#pragma once

#include "common.hpp"
#include "mfma_gemm.hpp"
#include "mfma_gemm3.hpp"

#include <type_traits>

namespace tg {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// acc (32 x 32 block, 16 floats per lane) += B-fragment x A-fragment on one
// v_mfma_f32_32x32x16, accumulator tied to the destination (see mfma_tied).
// Lane l supplies row / column l % 32 at k = 8 (l / 32) .. + 7 of the 16-deep
// K step, and holds C[m = l % 32][n = 8 q + 4 (l / 32) + e] in element 4 q + e.
template <typename Tr>
__device__ __forceinline__ void mfma32_tied(f32x16 &acc, const u32x4 &bop, const u32x4 &aop)
{
    if constexpr (Tr::code == 1)
        asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(bop), "v"(aop));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(bop), "v"(aop));
}

// K-contiguous 32 x 32 x 16 fragment: rows r0 .. r0+31, K step ks of a 32-deep
// stage (rows of 4 chunks, 32 x 32 swizzle).
__device__ __forceinline__ u32x4 frag32_kc(const char *st, int r0, int ks, int lane)
{
    const int r = r0 + (lane & 31);
    return *(const u32x4 *)(st + r * 64 + 16 * ((2 * ks + (lane >> 5)) ^ kc3_swz<4, 1>(r)));
}

// Per-lane base of a transposed 32 x 32 x 16 fragment read (K step ks, half h):
// within each 16-lane group the read returns 4 k-rows of 16 columns; groups
// 0/1 take columns 0-15 / 16-31 at k 0-7 of the step, groups 2/3 the same
// columns at k 8-15.  The column block only flips chunk bits 2..4 (XOR).
template <int CH>
__device__ __forceinline__ uint32_t mn32_base(uint32_t st, int ks, int h, int lane)
{
    const int gg = lane >> 4, i = lane & 15;
    const int n = 16 * (gg & 1) + 4 * (i & 3);
    const int k = 16 * ks + 8 * (gg >> 1) + 4 * h + (i >> 2);
    const int c = (n >> 3) ^ mn3_swz<CH, 1>(k);
    return st + (uint32_t)((k * CH + c) * 16 + (n & 7) * 2);
}

// EP selects the epilogue the instance carries: 1 = the whole tile to a 16-bit
// C without old C (no K split, beta = 0: the LDS-staged row stores and nothing
// else), 0 = every other case (K-split partials, old C, float32).  The launcher
// picks the instance from the call, so no kernel holds code it cannot run (with
// every epilogue in one kernel, adding the staged split partials had cost 8192^3
// about 1 %, with the K loop unchanged).
template <typename Tr, int S, int MI, bool TA, bool TB, bool SK = false, int BM = 256, int EP = 0>
__global__ __launch_bounds__(512) void mfma_pingpong_kernel(MfmaArgs p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using T = typename Tr::T;
    constexpr int BN = 256, BKS = 32;
    constexpr int WGN = 4;
    constexpr int WM = BM / 2, WN = 64;
    // 192 x 256 tiles (96 x 64 per wave): A K-contiguous (its M/N-contiguous
    // LDS layout needs a power-of-two row of chunks), 16-bit, no stream-K
    static_assert(BM == 256 || (BM == 192 && !TA && !SK && MI == 16 && Tr::kBytes == 2),
                  "192-row tiles: K-contiguous 16-bit A only");
    static_assert(MI == 16 || MI == 32, "MFMA block edge");
    constexpr int FM = WM / MI, FN = WN / MI;            // blocks per wave (8 x 4 or 4 x 2)
    constexpr int KS = BKS * MI / 512;                   // K steps per stage (1 or 2)
    constexpr int SW = MI == 32 ? 1 : 0;                 // LDS layout serving MI x MI reads
    using OpA = Dma3<BM, TA, 4, BKS, SW>;                // copied by group 0
    using OpB = Dma3<BN, !TB, 4, BKS, SW>;               // copied by group 1
    constexpr int A_BYTES = OpA::BYTES, B_BYTES = OpB::BYTES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    // copies per wave per stage: group 0 (A) and group 1 (B); equal for 256 x 256
    constexpr int NDMA_A = OpA::PER_WAVE, NDMA_B = OpB::PER_WAVE;
    static_assert(S >= 3 && S <= 5 && (S - 2) * (NDMA_A > NDMA_B ? NDMA_A : NDMA_B) < 64, "stage count");
    // float32 operands are copied as pairs of 16-bit units: a stage row is
    // then 16 values of K, and only K-contiguous operands are supported (the
    // transposed LDS reads of the M/N-contiguous layouts are 16-bit reads)
    constexpr int EW = Tr::kBytes / 2;
    static_assert(EW == 1 || (!TA && TB && !SK && MI == 16), "float32: K-contiguous A and B only");

    __shared__ __attribute__((aligned(1024))) char lds[S * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int grp = wm;            // group = row half of the tile
    const int gwave = wave & 3;    // wave index within its group

    // One work item: the K range [kbeg, kbeg + klen) of the tile at (m0, n0),
    // stored to C (through the output transform), to split z's float32 plane
    // of the workspace (K split), or as a tile-local float32 partial at Wt
    // (stream-K).  Every wave executes the same barriers, so items can follow
    // one another in a workgroup: all LDS reads of an item are consumed before
    // its last barrier.
    auto item = [&](const int m0, const int n0, const int z, const int kbeg, const int klen,
                    float *const Wt) {
        // K in 16-bit units from here on (float32: twice the element count)
        const int nfull = klen * EW / BKS;
        const int has_tail = (klen * EW % BKS) != 0;
        const int nst = nfull + has_tail;

        OpA oa;
        OpB ob;
        if (grp == 0)
            oa.init((const uint16_t *)p.A, p.lda * EW, p.rows_a, m0, kbeg * EW, gwave, lane);
        else
            ob.init((const uint16_t *)p.B, p.ldb * EW, p.cols_b, n0, kbeg * EW, gwave, lane);
        const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
        // this group's operand of processing stage t into its buffer: the K tail
        // (stage 0 when there is one) through registers, the rest by DMA
        auto issue = [&](int t) {
            const int slot = t % S;
            if (has_tail && t == 0) {
                char *st = lds + slot * STAGE;
                const int krel = klen * EW - nfull * BKS;
                if (grp == 0)
                    oa.tail(nfull, krel, st, gwave, lane);
                else
                    ob.tail(nfull, krel, st + A_BYTES, gwave, lane);
            } else if (grp == 0) {
                oa.dma(t - has_tail, lds_base + slot * STAGE, gwave);
            } else {
                ob.dma(t - has_tail, lds_base + slot * STAGE + A_BYTES, gwave);
            }
        };
        // Wait until this wave's copies of stage t have landed, stages up to
        // `last` having been issued: the younger stages (all DMA) may stay in
        // flight.  `lds` also waits for this wave's LDS traffic (the prologue's
        // register-path writes).
        auto wait_stage_n = [&](auto ndma, int t, int last, bool lds_too) {
            constexpr int NDMA = decltype(ndma)::value;
            const int younger = max(0, min(last - t, S - 2));
            if (lds_too) {
                if (S >= 5 && younger >= 3)
                    wait_vm_lgkm<(S >= 5 ? 3 : 0) * NDMA>();
                else if (S >= 4 && younger == 2)
                    wait_vm_lgkm<(S >= 4 ? 2 : 0) * NDMA>();
                else if (younger == 1)
                    wait_vm_lgkm<NDMA>();
                else
                    wait_vm_lgkm<0>();
            } else {
                if (S >= 5 && younger >= 3)
                    wait_vm<(S >= 5 ? 3 : 0) * NDMA>();
                else if (S >= 4 && younger == 2)
                    wait_vm<(S >= 4 ? 2 : 0) * NDMA>();
                else if (younger == 1)
                    wait_vm<NDMA>();
                else
                    wait_vm<0>();
            }
        };
        auto wait_stage = [&](int t, int last, bool lds_too) {
            if constexpr (NDMA_A == NDMA_B)
                wait_stage_n(std::integral_constant<int, NDMA_A>{}, t, last, lds_too);
            else if (grp == 0)
                wait_stage_n(std::integral_constant<int, NDMA_A>{}, t, last, lds_too);
            else
                wait_stage_n(std::integral_constant<int, NDMA_B>{}, t, last, lds_too);
        };

        // fragment reads of one stage: (K step, row block) for A, (K step,
        // column block) for B
        uint32_t mnA[KS][2], mnB[KS][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if constexpr (MI == 16) {
                    mnA[ks][h] = mn3_base<BM / 8>(lds_base, 0, h, lane);
                    mnB[ks][h] = mn3_base<BN / 8>(lds_base + A_BYTES, 0, h, lane);
                } else {
                    mnA[ks][h] = mn32_base<BM / 8>(lds_base, ks, h, lane);
                    mnB[ks][h] = mn32_base<BN / 8>(lds_base + A_BYTES, ks, h, lane);
                }
            }
        auto read_a = [&](const char *st, int ks, int i) -> u32x4 {
            const int r0 = wm * WM + MI * i;
            if constexpr (!TA) {
                if constexpr (MI == 16)
                    return frag3_kc<BKS / 8>(st, r0, 0, lane);
                else
                    return frag32_kc(st, r0, ks, lane);
            } else {
                const uint32_t so = (uint32_t)(st - lds);
                return frag3_mn<BM / 8>(mnA[ks][0] + so, mnA[ks][1] + so, r0);
            }
        };
        auto read_b = [&](const char *st, int ks, int j) -> u32x4 {
            const int c0 = wn * WN + MI * j;
            if constexpr (TB) {
                if constexpr (MI == 16)
                    return frag3_kc<BKS / 8>(st + A_BYTES, c0, 0, lane);
                else
                    return frag32_kc(st + A_BYTES, c0, ks, lane);
            } else {
                const uint32_t so = (uint32_t)(st - lds);
                return frag3_mn<BN / 8>(mnB[ks][0] + so, mnB[ks][1] + so, c0);
            }
        };

        using AccT = typename std::conditional<MI == 16, f32x4, f32x16>::type;
        AccT acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = AccT{};

        if (nst > 0) {
            u32x4 fa[KS][FM], fb[KS][FN];   // one stage of fragments

            // stages 0 .. S - 2 come first; stage b + S - 2 follows with stage b
            const int pro = min(nst, S - 1);
#pragma unroll
            for (int t = 0; t < S - 1; ++t)
                if (t < pro)
                    issue(t);
            wait_stage(0, pro - 1, true);
            lds_barrier();

            // load stage b into (fa, fb), after refilling the buffer of stage
            // b - 2 with stage b + S - 2; the reads are left in flight
            auto load = [&](int b) {
                if (b >= 1 && b + S - 2 < nst)
                    issue(b + S - 2);
                const char *st = lds + (b % S) * STAGE;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        fb[ks][j] = read_b(st, ks, j);
#pragma unroll
                    for (int i = 0; i < FM; ++i)
                        fa[ks][i] = read_a(st, ks, i);
                }
            };
            // multiply the stage in (fa, fb): 32 (16 x 16) or 16 (32 x 32) MFMAs
            // with nothing to wait for (float32: 128 v_mfma_f32_16x16x4f32,
            // element e of every fragment chunk at a time, so that no MFMA
            // waits for the one before it)
            auto multiply = [&]() {
                __builtin_amdgcn_s_setprio(2);
                if constexpr (EW == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int i = 0; i < FM; ++i)
#pragma unroll
                            for (int j = 0; j < FN; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    u32_as_f32(fb[0][j][e]), u32_as_f32(fa[0][i][e]), acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_s_setprio(0);
                    return;
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int i = 0; i < FM; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            // 16 x 16 blocks: the compiler's own MFMA, accumulators in
                            // VGPRs (measured as fast as tied AGPR accumulators, with
                            // no spills, and the compiler sees and covers every
                            // hazard of a register it moves)
                            if constexpr (MI == 16)
                                mfma_chunk<Tr>(acc[i][j], fb[ks][j], fa[ks][i]);
                            else
                                mfma32_tied<Tr>(acc[i][j], fb[ks][j], fa[ks][i]);
                        }
                __builtin_amdgcn_s_setprio(0);
            };
            // before the barrier that opens phase 2b + 2 (stage b + 1 first read)
            auto sync_next = [&](int b) {
                if (b + 1 < nst)
                    wait_stage(b + 1, min(nst - 1, b + S - 2), false);
            };
            // Each group runs its own straight-line loop (no role branches, so
            // the accumulators stay in their AGPRs); both execute 2 nst + 1
            // barriers, group 1 one phase behind group 0.
            if (grp == 0) {
                for (int b = 0; b < nst; ++b) {
                    load(b);
                    lds_barrier();
                    multiply();
                    sync_next(b);
                    lds_barrier();
                }
                lds_barrier();
            } else {
                lds_barrier();
                for (int b = 0; b < nst; ++b) {
                    load(b);
                    sync_next(b);
                    lds_barrier();
                    multiply();
                    lds_barrier();
                }
            }
            if constexpr (MI != 16)
                mfma_drain();   // tied asm accumulators: the hazard the compiler cannot see
        }

        T *C = (T *)p.C;
        // ---- epilogue through LDS (16-bit C, written directly, no old C):
        // the waves park their results in the ring as a row-major BM x 256
        // tile, then every store instruction writes two whole rows of the
        // tile, 16 bytes per lane.  The MFMA layout stores 16 rows x 32 bytes
        // per instruction instead, four times the L2 requests for the same
        // bytes, and all workgroups of a wave of tiles store at once.
        if constexpr (EP == 1) {
            static_assert(!SK && MI == 16 && Tr::kBytes == 2 && BM * 512 <= S * STAGE,
                          "the staged 16-bit epilogue needs 16 x 16 blocks and a ring of the tile's size");
            // Every LDS read of the ring was consumed by an MFMA before the
            // last barrier of the loop, and every copy had landed.  Chunk q
            // (16 bytes) of row r sits at chunk q ^ (r & 15): the 8-byte
            // writes below and the 16-byte reads after are bank-conflict-free.
            char *ct = lds;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int r = wm * WM + 16 * i + (lane & 15);
                    const int c = wn * WN + 16 * j + 4 * (lane >> 4);
                    T o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = Tr::from_f32(out_value_no_c(p.oe, acc[i][j][e]));
                    u32x2 w;
                    w[0] = (uint32_t)__builtin_bit_cast(uint16_t, o[0]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, o[1]) << 16);
                    w[1] = (uint32_t)__builtin_bit_cast(uint16_t, o[2]) |
                           ((uint32_t)__builtin_bit_cast(uint16_t, o[3]) << 16);
                    *(u32x2 *)(ct + r * 512 + (((c >> 3) ^ (r & 15)) << 4) + ((c >> 2) & 1) * 8) = w;
                }
            __syncthreads();
            const bool vec8 = (((uintptr_t)p.C) & 15) == 0 && (p.ldc & 7) == 0;
            constexpr int RW = BM / 8;   // tile rows per wave
#pragma unroll
            for (int it = 0; it < RW / 2; ++it) {
                const int r = wave * RW + 2 * it + (lane >> 5), q = lane & 31;
                const u32x4 v = *(const u32x4 *)(ct + r * 512 + ((q ^ (r & 15)) << 4));
                const int m = m0 + r, n = n0 + 8 * q;
                if (m < p.M) {
                    T *dst = C + (int64_t)m * p.ldc + n;
                    if (vec8 && n + 7 < p.N) {
                        *(u32x4 *)dst = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t word = v[e >> 1];
                            if (n + e < p.N)
                                dst[e] = __builtin_bit_cast(T, (uint16_t)(word >> (16 * (e & 1))));
                        }
                    }
                }
            }
            return;
        } else {
            // ---- K split: this split's float32 partial through LDS, one group's
            // half of the tile (the whole ring) at a time: row-major rows of 16-byte
            // chunks, chunk q of row r at q ^ (r & 15), then every wave stores rows
            // of the half, 16 bytes per lane
            if constexpr (!SK && MI == 16 && (BM / 2) * BN * 4 <= S * STAGE) {
                if (p.splits > 1) {
                    constexpr int CH = BN / 4;      // 16-byte chunks per row
                    constexpr int RW = WM / 8;      // rows of a half per wave
                    char *ct = lds;
                    float *Wz = p.ws + (int64_t)z * p.M * p.N;
                    const bool wvec = (p.N & 3) == 0;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        __syncthreads();   // the ring is idle (or the last half is stored)
                        if (grp == h) {
#pragma unroll
                            for (int i = 0; i < FM; ++i)
#pragma unroll
                                for (int j = 0; j < FN; ++j) {
                                    const int r = 16 * i + (lane & 15);
                                    const int q = (wn * WN + 16 * j) / 4 + (lane >> 4);
                                    *(f32x4 *)(ct + r * (BN * 4) + ((q ^ (r & 15)) << 4)) = acc[i][j];
                                }
                        }
                        __syncthreads();
#pragma unroll
                        for (int it = 0; it < RW * CH / 64; ++it) {
                            const int r = wave * RW + (it * 64 + lane) / CH, q = (it * 64 + lane) % CH;
                            const f32x4 v = *(const f32x4 *)(ct + r * (BN * 4) + ((q ^ (r & 15)) << 4));
                            const int m = m0 + h * WM + r, n = n0 + 4 * q;
                            if (m < p.M && n < p.N) {
                                float *dst = Wz + (int64_t)m * p.N + n;
                                if (wvec && n + 3 < p.N) {
                                    *(f32x4 *)dst = v;
                                } else {
#pragma unroll
                                    for (int e = 0; e < 4; ++e) {
                                        const float x = v[e];
                                        if (n + e < p.N)
                                            dst[e] = x;
                                    }
                                }
                            }
                        }
                    }
                    return;
                }
            }
            // ---- epilogue: each lane holds runs of 4 consecutive columns of C
            float *W = p.ws + (int64_t)z * p.M * p.N;
            auto store4 = [&](int m, int n, const f32x4 &v) {
                if constexpr (SK) {
                    if (Wt) {   // the whole tile, rows and columns past M and N included
                        *(f32x4 *)(Wt + (m - m0) * BN + (n - n0)) = v;
                        return;
                    }
                }
                if (m >= p.M || n >= p.N)
                    return;
                if (!SK && p.splits > 1) {
                    float *dst = W + (int64_t)m * p.N + n;
                    if (n + 3 < p.N && (p.N & 3) == 0) {
                        *(f32x4 *)dst = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N)
                                dst[e] = v[e];
                    }
                    return;
                }
                store_out4<Tr>(C + (int64_t)m * p.ldc + n, v, p.N - n, p.c_vec && n + 3 < p.N, p.oe);
            };
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (MI == 16) {
                        // C[m0 + .. + (lane & 15)][n0 + .. + 4 (lane >> 4) .. + 3]
                        store4(m0 + wm * WM + 16 * i + (lane & 15), n0 + wn * WN + 16 * j + 4 * (lane >> 4),
                               acc[i][j]);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                             acc[i][j][4 * q + 3]};
                            store4(m0 + wm * WM + 32 * i + (lane & 31),
                                   n0 + wn * WN + 32 * j + 8 * q + 4 * (lane >> 5), v);
                        }
                    }
                }
        }
    };

    if constexpr (!SK) {
        int tm, tn;
        tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
        const int z = blockIdx.y;
        const int kbeg = z * p.kps;
        item(tm * BM, tn * BN, z, kbeg, max(0, min(p.K, kbeg + p.kps) - kbeg), nullptr);
    } else {
        // stream-K: this workgroup's run of the tiles' stages, one item per
        // tile it touches (at most two: runs are shorter than a tile); a
        // whole tile goes straight to C, a piece to slot 2 g + j (g: the run)
        // run g of the sequence goes to workgroup ids that share an XCD (ids
        // go round-robin over the 8 XCDs): each XCD takes a contiguous
        // stretch of runs, i.e. of neighbouring tiles
        const int G = gridDim.x;
        const int q = G >> 3, rr = G & 7, x = blockIdx.x & 7;
        const int64_t g = x * q + min(x, rr) + (blockIdx.x >> 3);
        const int64_t beg = sk_start(g, p.sk_total, G), end = sk_start(g + 1, p.sk_total, G);
        int j = 0;
        for (int64_t it = beg; it < end; ++j) {
            const int t = (int)(it / p.sk_ipt);
            const int s0 = (int)(it - (int64_t)t * p.sk_ipt);
            const int s1 = (int)min<int64_t>(p.sk_ipt, s0 + (end - it));
            int tm, tn;
            tile_coords(t, p.tiles_m, p.tiles_n, tm, tn);
            const bool whole = s0 == 0 && s1 == p.sk_ipt;
            float *Wt = whole ? nullptr : p.ws + (2 * g + j) * (int64_t)(BM * BN);
            const int kbeg = s0 * BKS;
            item(tm * BM, tn * BN, 0, kbeg, min(p.K, s1 * BKS) - kbeg, Wt);
            it += s1 - s0;
        }
    }
#else
    (void)p;
#endif
}

// Stream-K fix-up.  Tile t whose stages were split between workgroups
// g0 .. g1 gets the sum of their float32 pieces, in stage order (g0 first),
// through the output transform; a tile one workgroup finished is already in
// C.  Run g's piece of its j-th tile is slot 2 g + j.  Grid: x = tiles,
// y = bands of p.sk_rows rows of a tile; the pieces of an element are loaded
// eight at a time and added in order.
template <typename Tr, int BM, int BN>
__global__ __launch_bounds__(256) void sk_fixup_kernel(MfmaArgs p)
{
    using T = typename Tr::T;
    constexpr int U = 8;
    const int t = blockIdx.x;
    const int64_t G = p.splits;   // workgroups of the stream-K launch
    const int64_t g0 = sk_owner((int64_t)t * p.sk_ipt, p.sk_total, G);
    const int64_t g1 = sk_owner((int64_t)(t + 1) * p.sk_ipt - 1, p.sk_total, G);
    if (g0 == g1)
        return;
    int tm, tn;
    tile_coords(t, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    T *C = (T *)p.C;
    constexpr int NQ = BN / 4;
    for (int idx = threadIdx.x; idx < p.sk_rows * NQ; idx += 256) {
        const int r = blockIdx.y * p.sk_rows + idx / NQ, c = (idx % NQ) * 4;
        const int m = m0 + r, n = n0 + c;
        if (m >= p.M || n >= p.N)
            continue;
        const float *base = p.ws + r * BN + c;
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int64_t g = g0; g <= g1; g += U) {
            f32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t gg = g + u;
                if (gg <= g1) {
                    const int64_t j = t - sk_start(gg, p.sk_total, G) / p.sk_ipt;
                    v[u] = *(const f32x4 *)(base + (2 * gg + j) * (int64_t)(BM * BN));
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (g + u <= g1)
                    s += v[u];
        }
        store_out4<Tr>(C + (int64_t)m * p.ldc + n, s, p.N - n, p.c_vec && n + 3 < p.N, p.oe);
    }
}

}  // namespace tg
