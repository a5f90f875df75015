// mfma_gemm2.hpp -- macro-tile GEMM for 16-bit operands, LDS-DMA pipeline.
//
// Same tiling as mfma_gemm.hpp (one BM x BN tile of C per workgroup, four
// wave64s in a 2 x 2 grid, 16 x 16 x 32 MFMA blocks; "Matrix Multiplication
// Background User's Guide", section 2.1), with the data movement rebuilt
// around two gfx950 features:
//
//   * global_load_lds_dwordx4 copies 16 bytes per lane from HBM/L2 straight
//     into LDS (lane l lands at base + 16 l) without passing through
//     registers, so a stage costs no VGPRs and four stages of BK = 32 can be in
//     flight (4 x (BM + BN) x 64 bytes of LDS: 128 KiB at 256 x 256);
//   * ds_read_b64_tr_b16 reads an N-contiguous (or M-contiguous) tile
//     transposed: within each 16-lane group, lane 4j + q supplies the address
//     of row k0 + j, columns n0 + 4q .. n0 + 4q + 3, and lane i receives
//     column n0 + i at rows k0 .. k0 + 3 - exactly an MFMA operand.  So a
//     plain-stored B (or a transposed-stored A) is copied to LDS as it lies
//     in memory and transposed by the read, not by the ALUs.
//
// LDS layouts of one stage (16-byte chunks, XOR-swizzled so that the DMA
// writes - always 1 KiB contiguous per wave instruction - and the fragment
// reads are both bank-conflict free; the swizzle is applied by choosing which
// global chunk each lane fetches):
//   K-contiguous operand: ROWS rows x 4 chunks (64 bytes of K per row),
//       chunk c of row r at r*4 + (c ^ ((r ^ r>>2) & 3));
//   M/N-contiguous operand: 32 k-rows x ROWS/8 chunks,
//       chunk c of row k at k*(ROWS/8) + (c ^ mn_swz(k)).
//
// Pipeline, per K step t (one barrier each): wait for this wave's DMA of step
// t+1, barrier (now every wave's copy of step t+1 has landed and every wave is
// done reading the buffer about to be refilled), issue the DMA of step t+3
// into that buffer, read step t+1's fragments into the spare register set
// while the MFMAs of step t run on the other set.  The waits are explicit
// (s_waitcnt vmcnt) because the compiler does not track LDS-DMA hazards.
//
// Edges: M/N rows past the edge are clamped (computed, never stored); a
// partial last K step is loaded through registers with a zero mask and
// written with ds_write_b128 into the same swizzled positions.
#pragma once

#include "common.hpp"
#include "mfma_gemm.hpp"

namespace tg {

typedef short s16x4 __attribute__((ext_vector_type(4)));

#define TG_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int kStages = 4;   // LDS pipeline depth
constexpr int kBK2 = 32;     // K per stage (16-bit elements)

__device__ __forceinline__ int kc_swz(int r) { return (r ^ (r >> 2)) & 3; }

template <int CH>
__device__ __forceinline__ int mn_swz(int k)
{
    if constexpr (CH >= 16)
        return (2 * (k & 3) + 8 * ((k >> 3) & 3)) & (CH - 1);
    else
        return (2 * ((k & 3) ^ ((k >> 3) & 3))) & (CH - 1);
}

// s_waitcnt immediate: wait until at most n vector-memory ops are outstanding,
// and until every LDS op has completed.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    constexpr int imm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8);
    __builtin_amdgcn_s_waitcnt(imm);
}

// One operand's stage traffic: ROWS tile rows (m for A, n for B).
// MN: the operand is contiguous along the tile rows in memory.  Offsets are
// 32-bit element offsets from the operand's base (the launcher only picks
// this kernel when every operand spans fewer than 2^31 elements).
template <int ROWS, bool MN>
struct DmaOperand {
    static constexpr int PER_WAVE = ROWS / 64;   // 1 KiB wave instructions per wave per stage
    static constexpr int CH = ROWS / 8;          // chunks per k-row (MN layout)
    static_assert(ROWS % 64 == 0, "tile rows must be a multiple of 64");

    const uint16_t *X;
    uint32_t off[PER_WAVE];  // this lane's source (elements from X) for K step 0
    uint32_t step;           // elements to advance per K step

    // chunk position -> (tile row, logical chunk) of this lane's u-th copy
    __device__ static __forceinline__ int pos(int wave, int lane, int u) { return (wave + 4 * u) * 64 + lane; }

    __device__ __forceinline__ void init(const uint16_t *X_, int64_t ld, int rows_total, int row0,
                                         int kbeg, int wave, int lane)
    {
        X = X_;
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u) {
            const int P = pos(wave, lane, u);
            if constexpr (!MN) {
                const int r = P >> 2;
                const int c = (P & 3) ^ kc_swz(r);
                const int gr = min(row0 + r, rows_total - 1);
                off[u] = (uint32_t)((int64_t)gr * ld + kbeg + 8 * c);
            } else {
                const int k = P / CH;
                const int c = (P % CH) ^ mn_swz<CH>(k);
                const int gc = min(row0 + 8 * c, rows_total - 8);
                off[u] = (uint32_t)((int64_t)(kbeg + k) * ld + gc);
            }
        }
        step = MN ? (uint32_t)(kBK2 * ld) : (uint32_t)kBK2;
    }

    // DMA of K step t into the stage at `dst` (this operand's region).
    __device__ __forceinline__ void dma(int t, char *dst, int wave) const
    {
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u)
            __builtin_amdgcn_global_load_lds(X + (off[u] + (uint32_t)t * step),
                                             TG_LDS(dst + (wave + 4 * u) * 1024), 16, 0, 0);
    }

    // Partial last step: masked register loads into the same LDS positions.
    __device__ __forceinline__ void tail(int t, int krel_end, char *dst, int wave, int lane) const
    {
#pragma unroll
        for (int u = 0; u < PER_WAVE; ++u) {
            const int P = pos(wave, lane, u);
            int kp;  // K offset of this lane's chunk within the step
            if constexpr (!MN)
                kp = 8 * ((P & 3) ^ kc_swz(P >> 2));
            else
                kp = P / CH;
            const bool ok = kp < krel_end;
            const u32x4 v = ok ? *(const u32x4 *)(X + (off[u] + (uint32_t)t * step)) : zero4();
            *(u32x4 *)(dst + (wave + 4 * u) * 1024 + lane * 16) = v;
        }
    }
};

// Fragment reads.  K-contiguous: one ds_read_b128 per 16-row block.
__device__ __forceinline__ u32x4 frag_kc(const char *base, int r, int g)
{
    return *(const u32x4 *)(base + (r * 4 + (g ^ kc_swz(r))) * 16);
}

// M/N-contiguous: two transposed 64-bit reads give 8 k values of column n0 + (lane & 15).
template <int CH>
__device__ __forceinline__ u32x4 frag_mn(const char *base, int n0, int lane)
{
    const int g = lane >> 4, i = lane & 15;
    const int n = n0 + 4 * (i & 3);
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int k = 8 * g + 4 * h + (i >> 2);
        const int c = (n >> 3) ^ mn_swz<CH>(k);
        const char *p = base + (k * CH + c) * 16 + (n & 7) * 2;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        out[2 * h] = w[0];
        out[2 * h + 1] = w[1];
    }
    return out;
}

template <typename Tr, int BM, int BN, bool TA, bool TB>
__global__ __launch_bounds__(256) void mfma_gemm2_kernel(MfmaArgs p)
{
    // The host compilation pass only needs this kernel's signature for its
    // launch stub; the LDS-DMA and transpose-read builtins exist on the device
    // side only, so the body is compiled for the device alone.
#if defined(__HIP_DEVICE_COMPILE__)
    using T = typename Tr::T;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64;
    constexpr int STAGE = A_BYTES + B_BYTES;
    using OpA = DmaOperand<BM, TA>;
    using OpB = DmaOperand<BN, !TB>;
    constexpr int NDMA = OpA::PER_WAVE + OpB::PER_WAVE;  // vm ops per wave per stage

    __shared__ __attribute__((aligned(1024))) char lds[kStages * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int z = blockIdx.y;
    const int kbeg = z * p.kps;
    const int kend = min(p.K, kbeg + p.kps);
    const int klen = max(0, kend - kbeg);
    // Steps are processed in pairs; an odd count gets one more step that lies
    // wholly past K (loaded as zeros), so the main loop has no peeled remainder.
    const int nk0 = (klen + kBK2 - 1) / kBK2;
    const int nk = nk0 + (nk0 & 1);
    // step t is copied by DMA when it lies wholly inside K, else through the
    // masked register path (the partial last step and the padding step)
    auto is_dma = [&](int t) { return (t + 1) * kBK2 <= klen; };

    OpA oa;
    OpB ob;
    oa.init((const uint16_t *)p.A, p.lda, p.M, m0, kbeg, wave, lane);
    ob.init((const uint16_t *)p.B, p.ldb, p.N, n0, kbeg, wave, lane);

    auto issue = [&](int t) {
        char *st = lds + (t % kStages) * STAGE;
        if (!is_dma(t)) {
            const int krel = klen - t * kBK2;  // <= 0 for the padding step
            oa.tail(t, krel, st, wave, lane);
            ob.tail(t, krel, st + A_BYTES, wave, lane);
        } else {
            oa.dma(t, st, wave);
            ob.dma(t, st + A_BYTES, wave);
        }
    };
    // Wait until step t's copies (this wave's) have landed.  `last` is the
    // newest step issued so far; DMA steps t+1 .. last may stay in flight (a
    // partial tail step was loaded through registers and is already done).
    auto wait_for = [&](int t, int last) {
        int younger = 0;
#pragma unroll
        for (int d = 1; d <= kStages - 2; ++d)
            if (t + d <= last && is_dma(t + d))
                ++younger;
        if (younger >= 2)
            wait_vm_lgkm0<2 * NDMA>();
        else if (younger == 1)
            wait_vm_lgkm0<NDMA>();
        else
            wait_vm_lgkm0<0>();
    };

    const int fr = lane & 15, fg = lane >> 4;
    u32x4 fa[FM], fb0[FN], fb1[FN];

    auto read_a = [&](const char *st, int i) -> u32x4 {
        if constexpr (!TA)
            return frag_kc(st, wm * WM + 16 * i + fr, fg);
        else
            return frag_mn<BM / 8>(st, wm * WM + 16 * i, lane);
    };
    auto read_b = [&](const char *st, int j) -> u32x4 {
        if constexpr (TB)
            return frag_kc(st + A_BYTES, wn * WN + 16 * j + fr, fg);
        else
            return frag_mn<BN / 8>(st + A_BYTES, wn * WN + 16 * j, lane);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
#pragma unroll
        for (int t = 0; t < kStages - 1; ++t)
            if (t < nk)
                issue(t);
        wait_for(0, min(nk - 1, kStages - 2));
        __builtin_amdgcn_s_barrier();
        {
            const char *st = lds;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = read_a(st, i);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb0[j] = read_b(st, j);
        }

        // Step t: fragments of step t are in (fa, fb).  After the barrier the
        // next step's B fragments are read into nb, then the DMA of step
        // t + kStages - 1 is issued (after the reads: the compiler cannot tell
        // a transposed read from an LDS-DMA target and drains the DMA queue
        // before one, so the reads go first and only the older copies are
        // waited for).  Each A fragment is refilled with the next step's as soon
        // as its row of MFMAs has been issued.
        auto body = [&](int t, u32x4 *fb, u32x4 *nb) {
            const bool more = t + 1 < nk;
            const char *nst = lds + ((t + 1) % kStages) * STAGE;
            if (more) {
                // issued so far: steps 0 .. t + kStages - 2
                wait_for(t + 1, min(nk - 1, t + kStages - 2));
                __builtin_amdgcn_s_barrier();
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    nb[j] = read_b(nst, j);
                if (t + kStages - 1 < nk)
                    issue(t + kStages - 1);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    mfma_chunk<Tr>(acc[i][j], fb[j], fa[i]);
                if (more)
                    fa[i] = read_a(nst, i);
            }
        };
        // Two steps per trip, both unconditional (nk is even), so the B
        // fragments ping-pong between two register sets without copies and
        // every accumulator keeps one register home.
        for (int t = 0; t < nk; t += 2) {
            body(t, fb0, fb1);
            body(t + 1, fb1, fb0);
        }
    }

    // ---- epilogue: lane holds C[m][n .. n+3] of every 16 x 16 block
    if (p.splits > 1) {
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
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WM + i * 16 + fr;
        if (m >= p.M)
            continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WN + j * 16 + 4 * fg;
            T *dst = C + (int64_t)m * p.ldc + n;
            T v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = Tr::from_f32(apply_epi(acc[i][j][e], p.epi, p.slope));
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
#else
    (void)p;
#endif
}

}  // namespace tg
