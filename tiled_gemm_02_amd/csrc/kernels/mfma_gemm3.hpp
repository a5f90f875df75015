// mfma_gemm3.hpp -- macro-tile GEMM for 16-bit operands: LDS-DMA pipeline with
// explicitly placed waits.
//
// Tiling ("Matrix Multiplication Background User's Guide", section 2.1): one
// BM x BN tile of C per workgroup, four wave64s in a 2 x 2 grid, each wave
// owning a (BM/2) x (BN/2) sub-tile of 16 x 16 blocks computed with
// v_mfma_f32_16x16x32_{f16,bf16} (fp32 accumulate).  K advances in stages of
// 64 elements: every K-contiguous operand row contributes one whole 128-byte
// line per stage.
//
// Data movement:
//   * global_load_lds_dwordx4 copies 16 bytes per lane from memory straight
//     into LDS (lane l lands at M0 + 16 l).  The copies are issued from inline
//     assembly so that the compiler, which cannot tell an LDS-DMA target from
//     the buffer a later LDS read touches, does not drain the copy queue before
//     every LDS read; the kernel places its own s_waitcnt instead, counting the
//     copies still allowed in flight exactly.
//   * K-contiguous tiles (A stored M x K, B stored N x K) are read with
//     ds_read_b128; M/N-contiguous tiles (A stored K x M, B stored K x N) are
//     copied as they lie and read transposed with ds_read_b64_tr_b16.
//
// LDS layouts of one stage (16-byte chunks), chosen against gfx950's banking
// (64 banks of 4 bytes; a ds_read_b128 serves 16 lanes per pass, lanes
// {0-3,12-15,20-23,24-27} together, a ds_read_b64(_tr) 32 lanes, a
// ds_write_b128 8 lanes), so that fragment reads and copies are conflict free:
//   K-contiguous: ROWS rows x 8 chunks, chunk c of row r at r*8 + (c ^ (r & 6));
//   M/N-contiguous: 64 k-rows x ROWS/8 chunks, chunk c of row k at
//       k*(ROWS/8) + (c ^ mn_swz(k)).
// A lane's copy picks the global chunk that belongs at its LDS position, so
// every copy instruction writes 1 KiB of LDS linearly.
//
// Pipeline (S stages in LDS, fragments double-buffered in registers, one
// barrier per stage): while the MFMAs of one 32-deep K block run, the
// fragments of the next block are read from LDS - B fragments during the first
// half of the MFMA rows, A fragments during the second.  When the next block
// starts a new stage, the wave first issues one row of MFMAs, then waits for
// its own copies of that stage, waits for its outstanding LDS reads, meets the
// other waves at the barrier (after which every copy of the stage has landed
// and nobody reads the stage just finished), and refills the finished stage's
// buffer with the copy of the stage S ahead.
//
// Edges: M/N rows past the edge are clamped (computed, never stored); a
// partial 64-deep K stage is loaded through registers with a zero mask and
// written with ds_write_b128 into the same swizzled positions, as the first
// stage processed, so the main loop issues nothing but DMA.
#pragma once

#include "common.hpp"
#include "mfma_gemm.hpp"

namespace tg {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK3 = 64;   // K per stage (16-bit elements) of the pipelined kernel, by default

// Chunk swizzle of a K-contiguous LDS row of KCH 16-byte chunks (KCH = 8:
// 128-byte rows, 64-deep stages; KCH = 4: 64-byte rows, 32-deep stages).  SW
// selects the fragment shape the layout serves: 0 for 16 x 16 x 32 MFMA
// fragments (16 rows x 4 chunks per read), 1 for 32 x 32 x 16 ones (32 rows x
// 2 chunks per read); each is conflict free for its own reads.
template <int KCH, int SW = 0>
__device__ __forceinline__ int kc3_swz(int r)
{
    static_assert(KCH == 4 || KCH == 8, "row of 4 or 8 chunks");
    static_assert(SW == 0 || KCH == 4, "32 x 32 layout only for 64-byte rows");
    if constexpr (KCH == 8)
        return r & 6;
    else if constexpr (SW == 0)
        return (r >> 1) & 3;
    else
        return (r >> 2) & 3;
}

// Chunk swizzle of an M/N-contiguous k-row of CH chunks.  SW = 0: a
// transposed 16 x 16 x 32 fragment read touches 8 k-rows x 32 bytes per pass,
// spread by 32-byte steps; SW = 1: a 32 x 32 x 16 one touches 4 k-rows x 64
// bytes, spread by 64-byte steps.
template <int CH, int SW = 0>
__device__ __forceinline__ int mn3_swz(int k)
{
    if constexpr (SW == 1)
        return (4 * (k & 3)) & (CH - 1);
    else if constexpr (CH >= 16)
        return (2 * (k & 3) + 8 * ((k >> 3) & 3)) & (CH - 1);
    else
        return (2 * ((k & 3) ^ ((k >> 3) & 3))) & (CH - 1);
}

// s_waitcnt vmcnt(N) lgkmcnt(0), as a compiler memory barrier.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(N) alone (LDS reads may stay in flight).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte-per-lane copy from global memory into LDS at m0 + 16 * lane.
// The base address and the LDS address are wave-uniform; they are passed
// through readfirstlane so that they are SGPR operands whatever the compiler
// concluded about their uniformity.
__device__ __forceinline__ void dma16(uint32_t voff, const void *sbase, uint32_t lds_addr)
{
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                 :
                 : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"(sb)
                 : "memory", "m0");
}

// acc += B-fragment x A-fragment on one 16 x 16 x 32 MFMA (same operand
// roles as mfma_chunk), with the accumulator tied to the destination.  As a
// builtin, the compiler's MFMA register rewriting gives most of these
// instructions a destination other than their accumulator and then copies
// whole accumulators between AGPRs and VGPRs every iteration; the tied asm
// form keeps every accumulator in one AGPR quad.  The compiler still places
// the LDS waits for the VGPR inputs; the one hazard it cannot see (MFMA result
// -> v_accvgpr_read) is covered by mfma_drain() before the accumulators are
// read.
template <typename Tr>
__device__ __forceinline__ void mfma_tied(f32x4 &acc, const u32x4 &bop, const u32x4 &aop)
{
    if constexpr (Tr::code == 1)
        asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(bop), "v"(aop));
    else
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(bop), "v"(aop));
}

// Wait states between the last MFMA and any read of its accumulator (an
// 8-pass MFMA needs fewer than 20; 64 are given).
__device__ __forceinline__ void mfma_drain()
{
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
}

// One operand's stage traffic: ROWS tile rows (m for A, n for B) by BKS of K,
// copied by NW waves.  MN: the operand is contiguous along the tile rows in
// memory.
template <int ROWS, bool MN, int NW, int BKS = kBK3, int SW = 0>
struct Dma3 {
    static constexpr int BYTES = ROWS * BKS * 2;                // LDS bytes per stage
    static constexpr int PER_WAVE = BYTES / 1024 / NW;          // 1 KiB copies per wave per stage
    static constexpr int CH = ROWS / 8;                         // chunks per k-row (MN layout)
    static constexpr int KCH = BKS / 8;                         // chunks per row (KC layout)
    static_assert(PER_WAVE >= 1 && PER_WAVE * NW * 1024 == BYTES, "stage does not split over the waves");

    const char *base;        // byte address of (row0, kbeg) / (kbeg, row0)
    int64_t step;            // bytes to advance per stage
    uint32_t off[PER_WAVE];  // this lane's byte offsets from base

    __device__ static __forceinline__ int pos(int wave, int lane, int u) { return (wave + NW * u) * 64 + lane; }

    __device__ __forceinline__ void init(const uint16_t *X, int64_t ld, int rows_total, int row0,
                                         int kbeg, int wave, int lane)
    {
        if constexpr (!MN) {
            base = (const char *)(X + (int64_t)row0 * ld + kbeg);
            step = BKS * 2;
        } else {
            base = (const char *)(X + (int64_t)kbeg * ld + row0);
            step = (int64_t)BKS * ld * 2;
        }
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u) {
            const int P = pos(wave, lane, u);
            if constexpr (!MN) {
                const int r = P / KCH;
                const int c = (P % KCH) ^ kc3_swz<KCH, SW>(r);
                const int gr = min(row0 + r, rows_total - 1) - row0;
                off[u] = (uint32_t)(((int64_t)gr * ld + 8 * c) * 2);
            } else {
                const int k = P / CH;
                const int c = (P % CH) ^ mn3_swz<CH, SW>(k);
                const int gc = min(row0 + 8 * c, rows_total - 8) - row0;
                off[u] = (uint32_t)(((int64_t)k * ld + gc) * 2);
            }
        }
    }

    // Copy stage t into the LDS region at byte address `dst` (uniform).
    __device__ __forceinline__ void dma(int t, uint32_t dst, int wave) const
    {
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u)
            dma_one(t, u, dst, wave);
    }
    // The u-th of this wave's copies of stage t.
    __device__ __forceinline__ void dma_one(int t, int u, uint32_t dst, int wave) const
    {
        dma16(off[u], base + (int64_t)t * step, dst + (uint32_t)(wave + NW * u) * 1024u);
    }

    // Partial last stage: masked register loads into the same LDS positions.
    // krel_end = valid K elements in this stage (1 .. BKS - 1).
    __device__ __forceinline__ void tail(int t, int krel_end, char *dst, int wave, int lane) const
    {
        const char *b = base + (int64_t)t * step;
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u) {
            const int P = pos(wave, lane, u);
            int kp;  // K offset of this lane's chunk within the stage
            if constexpr (!MN)
                kp = 8 * ((P % KCH) ^ kc3_swz<KCH, SW>(P / KCH));
            else
                kp = P / CH;
            const u32x4 v = kp < krel_end ? *(const u32x4 *)(b + off[u]) : zero4();
            *(u32x4 *)(dst + (wave + NW * u) * 1024 + lane * 16) = v;
        }
    }
};

// K-contiguous fragment: rows r0 .. r0+15, 32-deep K block kb of the stage
// (rows of KCH chunks).
template <int KCH = 8>
__device__ __forceinline__ u32x4 frag3_kc(const char *st, int r0, int kb, int lane)
{
    const int r = r0 + (lane & 15), g = lane >> 4;
    return *(const u32x4 *)(st + r * (KCH * 16) + 16 * ((4 * kb + g) ^ kc3_swz<KCH>(r)));
}

// M/N-contiguous fragment: two transposed 64-bit reads give 8 k values of
// column n0 + (lane & 15) for K block kb.  Column block n0 / 16 only flips
// address bits 5..8 (chunk bits 1..4, untouched by the row base), so the
// address is the lane's base for (kb, h) XOR a constant; the XOR is issued
// where it is used, which keeps a handful of base registers live instead of
// one address per (block, kb, h).
template <int CH>
__device__ __forceinline__ uint32_t mn3_base(uint32_t st, int kb, int h, int lane)
{
    const int g = lane >> 4, i = lane & 15;
    const int n = 4 * (i & 3);
    const int k = 32 * kb + 8 * g + 4 * h + (i >> 2);
    const int c = (n >> 3) ^ mn3_swz<CH>(k);
    return st + (uint32_t)((k * CH + c) * 16 + (n & 7) * 2);
}

template <int CH>
__device__ __forceinline__ u32x4 frag3_mn(uint32_t b0, uint32_t b1, int n0)
{
    static_assert(CH <= 32, "chunk bits above 4 would reach the row base");
    const uint32_t flip = (uint32_t)(n0 >> 3) * 16u;  // n0 is a multiple of 16
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t a;
        asm volatile("v_xor_b32 %0, %1, %2" : "=v"(a) : "v"(h ? b1 : b0), "s"(flip));
        const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t *)(uintptr_t)a);
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        out[2 * h] = w[0];
        out[2 * h + 1] = w[1];
    }
    return out;
}

// KG K groups per workgroup (1, 2 or 4): the workgroup holds KG sets of
// WGM x WGN waves, each running the pipeline above over its own part of the
// workgroup's K range in its own LDS ring; at the end groups 1 .. KG-1 add
// their sums to group 0's through LDS (in group order, a fixed order) and the
// whole workgroup stores the tile.  It is a K split whose reduction stays on
// the CU: no float32 partials in memory and no second launch.  The groups meet
// at the same barriers, so all run the same number of stages: the workgroup's
// 64-deep stages are dealt out in consecutive runs, ceil(n / KG) to the first
// groups and one fewer to the rest, the partial stage of a K tail being the
// last of group 0's run (groups 1 .. KG-1 start on the 16-byte grid, since K is
// a multiple of 8); a group one whole stage short processes an all-zero tail
// stage first, with no K to load.
//
// BKS: K depth of a stage, 64 (every K-contiguous row contributes a whole
// 128-byte line per stage) or 32 (half-line rows, twice the stages in the same
// LDS, so more of them in flight); a stage is BKS / 32 blocks of 32-deep MFMAs.
template <typename Tr, int BM, int BN, int S, int WGM, int WGN, bool TA, bool TB, int KG = 1, int BKS = kBK3>
__global__ __launch_bounds__(64 * WGM * WGN * KG) void mfma_gemm3_kernel(MfmaArgs p)
{
    // The LDS-DMA and transposed-read builtins exist on the device side only;
    // the host pass needs nothing but the signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using T = typename Tr::T;
    static_assert(KG == 1 || KG == 2 || KG == 4, "1, 2 or 4 K groups");
    static_assert(BKS == 32 || BKS == 64, "32- or 64-deep stages");
    constexpr int KB = BKS / 32;                          // 32-deep K blocks per stage
    constexpr int KCH = BKS / 8;                          // 16-byte chunks per K-contiguous row
    constexpr int NW = WGM * WGN;                         // waves per K group
    constexpr int NWALL = NW * KG;                        // waves per workgroup
    constexpr int WM = BM / WGM, WN = BN / WGN;           // wave sub-tile
    constexpr int FM = WM / 16, FN = WN / 16;
    using OpA = Dma3<BM, TA, NW, BKS>;
    using OpB = Dma3<BN, !TB, NW, BKS>;
    constexpr int A_BYTES = OpA::BYTES, B_BYTES = OpB::BYTES;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int NDMA = OpA::PER_WAVE + OpB::PER_WAVE;  // copies per wave per stage
    constexpr int HALF = FM > 1 ? FM / 2 : 1;            // MFMA rows that carry B reads
    static_assert(FM >= 2 && FN >= 2, "wave sub-tile of at least 32 x 32");
    static_assert(S >= 2 && (S - 2) * NDMA < 64, "stage count");

    constexpr int LDS_BYTES = KG * S * STAGE;
    __shared__ __attribute__((aligned(1024))) char lds_all[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kgrp = wave_all / NW;                       // K group of this wave
    const int wave = wave_all % NW;                       // wave within its group
    const int wm = wave / WGN, wn = wave % WGN;
    char *const lds = lds_all + kgrp * (S * STAGE);       // this group's ring

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int z = blockIdx.y;
    const int kbeg_wg = z * p.kps;
    const int klen_wg = max(0, min(p.K, kbeg_wg + p.kps) - kbeg_wg);
    // this group's run of the workgroup's stages (KG = 1: all of them)
    const int nstg = (klen_wg + BKS - 1) / BKS;           // stages, the partial one included
    const int short0 = (klen_wg % BKS) ? BKS - klen_wg % BKS : 0;   // missing from the partial one
    const int nst = (nstg + KG - 1) / KG;                  // stages every group processes
    const int nhi = nst > 0 ? nstg - (nst - 1) * KG : KG;  // groups with nst stages of K
    const int cnt = kgrp < nhi ? nst : nst - 1;            // this group's stages of K
    const int first = kgrp < nhi ? kgrp * nst : nhi * nst + (kgrp - nhi) * (nst - 1);
    const int kbeg = kbeg_wg + (kgrp == 0 ? 0 : BKS * first - short0);
    const int klen = cnt <= 0 ? 0 : BKS * cnt - (kgrp == 0 ? short0 : 0);
    // A partial stage (group 0's last, when K is not a multiple of BKS)
    // is processed first, as stage 0, through the masked register path; the
    // whole stages follow, all copied by DMA.  Summation order over K is
    // immaterial.  A group with one stage fewer processes an all-zero stage 0
    // the same way (no valid K).
    const int nfull = klen / BKS;                 // whole stages
    const int has_tail = nst - nfull;             // 0 or 1
    OpA oa;
    OpB ob;
    oa.init((const uint16_t *)p.A, p.lda, p.rows_a, m0, kbeg, wave, lane);
    ob.init((const uint16_t *)p.B, p.ldb, p.cols_b, n0, kbeg, wave, lane);

    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    // Load processing stage t into its buffer: the K-tail (stage 0 when there
    // is one) through registers, every other stage by DMA.
    auto issue = [&](int t) {
        const int slot = t % S;
        if (has_tail && t == 0) {
            char *st = lds + slot * STAGE;
            const int krel = klen - nfull * BKS;
            oa.tail(nfull, krel, st, wave, lane);
            ob.tail(nfull, krel, st + A_BYTES, wave, lane);
        } else {
            oa.dma(t - has_tail, lds_base + slot * STAGE, wave);
            ob.dma(t - has_tail, lds_base + slot * STAGE + A_BYTES, wave);
        }
    };
    // Wait until this wave's copies of stage t have landed (and its LDS reads
    // completed), given that stages up to `last` have been issued.  Stages
    // loaded through registers were already complete when written.
    auto wait_stage = [&](int t, int last) {
        int younger = 0;
#pragma unroll
        for (int d = 1; d <= S - 2; ++d)
            if (t + d <= last)   // stages after t are all DMA stages
                ++younger;
        if constexpr (S >= 4) {
            if (younger >= 2) {
                wait_vm_lgkm<(S >= 4 ? 2 : 0) * NDMA>();
                return;
            }
        }
        if constexpr (S >= 3) {
            if (younger == 1) {
                wait_vm_lgkm<NDMA>();
                return;
            }
        }
        wait_vm_lgkm<0>();
    };

    const int fr = lane & 15, fg = lane >> 4;
    // per-lane bases of the transposed reads, by (K block, half), at stage 0
    uint32_t mnA[KB][2], mnB[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            mnA[kb][h] = mn3_base<BM / 8>(lds_base, kb, h, lane);
            mnB[kb][h] = mn3_base<BN / 8>(lds_base + A_BYTES, kb, h, lane);
        }
    auto read_a = [&](const char *st, int kb, int i) -> u32x4 {
        if constexpr (!TA) {
            return frag3_kc<KCH>(st, wm * WM + 16 * i, kb, lane);
        } else {
            const uint32_t so = (uint32_t)(st - lds);
            return frag3_mn<BM / 8>(mnA[kb][0] + so, mnA[kb][1] + so, wm * WM + 16 * i);
        }
    };
    auto read_b = [&](const char *st, int kb, int j) -> u32x4 {
        if constexpr (TB) {
            return frag3_kc<KCH>(st + A_BYTES, wn * WN + 16 * j, kb, lane);
        } else {
            const uint32_t so = (uint32_t)(st - lds);
            return frag3_mn<BN / 8>(mnB[kb][0] + so, mnB[kb][1] + so, wn * WN + 16 * j);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nst > 0) {
        u32x4 fa[FM], fb0[FN], fb1[FN];
        const int pro = min(nst, S);
#pragma unroll
        for (int t = 0; t < S; ++t)
            if (t < pro)
                issue(t);
        wait_stage(0, pro - 1);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[i] = read_a(lds, 0, i);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb0[j] = read_b(lds, 0, j);

        // K block kb of stage t.  The A fragments (fa) and the B fragments (fb)
        // of this block are in registers.  Row i of MFMAs is followed by the
        // refill of fa[i] with the next block's fragment, and each of the first
        // HALF rows also by a share of the next block's B fragments (into nb).
        // When the next block starts stage t + 1, the wave synchronises after
        // its first row of MFMAs, and the copies of stage t + S into the buffer
        // just released are spread one per row over the rest of the block, so
        // the matrix unit is never left waiting behind a burst of copy issues.
        auto body = [&](int t, int kb, const u32x4 *fb, u32x4 *nb, bool more) {
            const bool last = kb == KB - 1;        // the next block starts stage t + 1
            const int tn1 = last ? t + 1 : t;      // stage of the next block
            const int kbn = last ? 0 : kb + 1;
            const char *nst_p = lds + (tn1 % S) * STAGE;
            const bool refill = more && last && t + S < nst;
            const uint32_t rslot = lds_base + ((t + S) % S) * STAGE;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    mfma_tied<Tr>(acc[i][j], fb[j], fa[i]);
                if (more) {
                    if (i == 0 && last) {
                        // stages up to t + S - 1 have been issued
                        wait_stage(t + 1, min(nst - 1, t + S - 1));
                        lds_barrier();
                    }
                    if (last) {
                        // copies q = i, i + FM, ... of stage t + S (DMA: t + S >= 1)
#pragma unroll
                        for (int q = i; q < NDMA; q += FM) {
                            if (refill) {
                                if (q < OpA::PER_WAVE)
                                    oa.dma_one(t + S - has_tail, q, rslot, wave);
                                else
                                    ob.dma_one(t + S - has_tail, q - OpA::PER_WAVE, rslot + A_BYTES, wave);
                            }
                        }
                    }
                    if (i < HALF) {
#pragma unroll
                        for (int j = i * FN / HALF; j < (i + 1) * FN / HALF; ++j)
                            nb[j] = read_b(nst_p, kbn, j);
                    }
                    fa[i] = read_a(nst_p, kbn, i);
                }
                // keep each row's MFMAs and reads where they are
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // Two K blocks per trip (one 64-deep stage, or two 32-deep ones); the B
        // fragments ping-pong between two register sets, so every accumulator
        // keeps one register home.
        if constexpr (KB == 2) {
            for (int t = 0; t < nst; ++t) {
                body(t, 0, fb0, fb1, true);
                body(t, 1, fb1, fb0, t + 1 < nst);
            }
        } else {
            for (int t = 0; t < nst; t += 2) {
                body(t, 0, fb0, fb1, t + 1 < nst);
                if (t + 1 < nst)
                    body(t + 1, 0, fb1, fb0, t + 2 < nst);
            }
        }
        mfma_drain();
    }

    // ---- epilogue: lane holds C[m][n .. n+3] of every 16 x 16 block
    if constexpr (KG > 1) {
        // groups 1 .. KG-1 join group 0: each of their waves parks its
        // accumulators in LDS (16 bytes per lane, lane-linear: no bank
        // conflicts) and the wave of group 0 with the same sub-tile adds them,
        // group by group
        static_assert((KG - 1) * NW * FM * FN * 1024 <= LDS_BYTES, "reduction area");
        f32x4 *xs = (f32x4 *)lds_all + wave * (FM * FN * 64) + lane;
        constexpr int GSTRIDE = NW * FM * FN * 64;   // f32x4 slots per group
        __syncthreads();   // every wave's last fragment reads are done
        if (kgrp > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    xs[(kgrp - 1) * GSTRIDE + (i * FN + j) * 64] = acc[i][j];
        }
        __syncthreads();
        if (kgrp == 0) {
#pragma unroll
            for (int g = 1; g < KG; ++g)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const f32x4 v = xs[(g - 1) * GSTRIDE + (i * FN + j) * 64];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][j][e] += v[e];
                    }
        }
    }
    // From here on the sums are group 0's; every wave of the workgroup meets
    // the barriers of the LDS-staged stores (their branches depend on kernel
    // arguments only), and group 1 leaves before the direct stores.
    if constexpr (BM * BN * 4 <= LDS_BYTES) {
        if (p.splits > 1) {
            // this split's float32 partial through LDS, like the 16-bit C below:
            // a row-major BM x BN tile (chunk q of row r at q ^ (r & 15), rows of
            // 16 or 32 chunks), then rows of 16-byte chunks per lane
            constexpr int CH = BN / 4;
            static_assert(CH >= 16, "float32 staging: rows of 16 or more chunks");
            char *ct = lds_all;
            __syncthreads();   // every wave's last fragment reads are done
            if (kgrp == 0) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int r = wm * WM + i * 16 + fr;
                        const int q = (wn * WN + j * 16) / 4 + fg;
                        *(f32x4 *)(ct + r * (BN * 4) + ((q ^ (r & 15)) << 4)) = acc[i][j];
                    }
            }
            __syncthreads();
            float *W = p.ws + (int64_t)z * p.M * p.N;
            const bool wvec = (p.N & 3) == 0;
            constexpr int RPI = 64 / CH;                     // rows per read instruction
            constexpr int NI = BM / RPI;                     // read instructions per tile
            static_assert(NI * RPI == BM, "whole read instructions per tile");
#pragma unroll
            for (int it = 0; it < (NI + NWALL - 1) / NWALL; ++it) {
                const int ins = it * NWALL + wave_all;       // instruction of this wave (uniform)
                if (NI % NWALL != 0 && ins >= NI)
                    break;
                const int r = ins * RPI + lane / CH, q = lane % CH;
                const f32x4 v = *(const f32x4 *)(ct + r * (BN * 4) + ((q ^ (r & 15)) << 4));
                const int m = m0 + r, n = n0 + 4 * q;
                if (m < p.M && n < p.N) {
                    float *dst = W + (int64_t)m * p.N + n;
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
            return;
        }
    }
    if (p.splits > 1) {
        if (kgrp != 0)
            return;
        float *W = p.ws + (int64_t)z * p.M * p.N;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * WM + i * 16 + fr;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WN + j * 16 + 4 * fg;
                float *dst = W + (int64_t)m * p.N + n;
                if (n + 3 < p.N && (p.N & 3) == 0) {
                    *(f32x4 *)dst = acc[i][j];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N)
                            dst[e] = acc[i][j][e];
                }
            }
        }
        return;
    }
    T *C = (T *)p.C;
    // 16-bit C without old C: through LDS as a row-major BM x BN tile, then
    // whole rows, 16 bytes per lane (the MFMA layout stores 16 rows x 32 bytes
    // per instruction).  Chunk q of row r sits at q ^ sw(r): XOR of the row's
    // low four bits for rows of 16 or 32 chunks, of bits 1..3 for rows of 8
    // (two such rows share one pass over the 64 banks), so the 8-byte writes
    // and the 16-byte reads are both free of bank conflicts.
    if constexpr (Tr::kBytes == 2 && BM * BN * 2 <= LDS_BYTES) {
        if (p.oe.beta == 0.0f) {
            constexpr int CH = BN / 8;                       // 16-byte chunks per row
            auto sw = [](int r) { return CH >= 16 ? (r & 15) : ((r >> 1) & 7); };
            char *ct = lds_all;
            __syncthreads();   // every wave's last fragment reads are done
            if (kgrp == 0) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int r = wm * WM + i * 16 + fr;
                        const int c = wn * WN + j * 16 + 4 * fg;
                        T o[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            o[e] = Tr::from_f32(out_value_no_c(p.oe, acc[i][j][e]));
                        u32x2 w;
                        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, o[0]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, o[1]) << 16);
                        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, o[2]) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, o[3]) << 16);
                        *(u32x2 *)(ct + r * (BN * 2) + (((c >> 3) ^ sw(r)) << 4) + ((c >> 2) & 1) * 8) = w;
                    }
            }
            __syncthreads();
            const bool vec8 = (((uintptr_t)p.C) & 15) == 0 && (p.ldc & 7) == 0;
            constexpr int RPI = 64 / CH;                     // rows per read instruction
            constexpr int NI = BM / RPI;                     // read instructions per tile
            static_assert(NI * RPI == BM, "whole read instructions per tile");
#pragma unroll
            for (int it = 0; it < (NI + NWALL - 1) / NWALL; ++it) {
                const int ins = it * NWALL + wave_all;       // instruction of this wave (uniform)
                if (NI % NWALL != 0 && ins >= NI)
                    break;
                const int r = ins * RPI + lane / CH, q = lane % CH;
                const u32x4 v = *(const u32x4 *)(ct + r * (BN * 2) + ((q ^ sw(r)) << 4));
                const int m = m0 + r, n = n0 + 8 * q;
                if (m < p.M && n < p.N) {
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
        }
    }
    if (kgrp != 0)
        return;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + i * 16 + fr;
        if (m >= p.M)
            continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + j * 16 + 4 * fg;
            if (n >= p.N)
                continue;
            store_out4<Tr>(C + (int64_t)m * p.ldc + n, acc[i][j], p.N - n, p.c_vec && n + 3 < p.N, p.oe);
        }
    }
#else
    (void)p;
#endif
}

}  // namespace tg
