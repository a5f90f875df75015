// mfma_gemm.hpp -- macro-tile GEMM on gfx950 matrix cores.
//
// The output is cut into BM x BN tiles, one workgroup each; every workgroup
// walks the contraction dimension in BK-deep steps, multiplying the A and B
// slices it has staged in LDS into accumulators it keeps in registers (the
// tiled outer-product scheme of "Matrix Multiplication Background User's
// Guide", section 2.1, and the blocked GEMM of "Learning Triton One Kernel at
// a Time: Matrix Multiplication", sections on tiled and parallel tiled GEMM).
//
// gfx950 specifics:
//   * 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a
//     (BM/2) x (BN/2) sub-tile made of 16 x 16 MFMA blocks;
//   * one BK step is 128 bytes of K per row (64 fp16/bf16 or 32 fp32
//     values), i.e. 8 16-byte chunks per LDS row;
//   * global -> register loads are 128-bit and coalesced along the operand's
//     contiguous dimension; an operand that is contiguous along M or N (A
//     stored transposed, B stored plain) is transposed in registers 8 x 8
//     (4 x 4 for fp32) on its way into LDS, so LDS always holds K-contiguous
//     rows and the MFMA fragment reads are single ds_read_b128s;
//   * LDS rows are XOR-swizzled at 16-byte granularity so that the fragment
//     reads (16 rows, one chunk each) and both kinds of writes spread over all
//     banks: the transposed-store stall the Triton tutorial profiles is what
//     this avoids;
//   * two LDS stages: the loads for step t+1 are in flight while step t
//     multiplies, one barrier per step;
//   * tiles are handed out XCD-major: the hardware deals consecutive workgroup
//     ids round-robin over the 8 XCDs, so ids are remapped to give every XCD a
//     contiguous run of tiles, walked in groups of 8 tile rows, keeping the A
//     and B panels of concurrently running tiles in one XCD's L2.
//
// M and N edges clamp the row index (rows past the edge are computed but never
// stored); the last partial K step is zero-filled; split-K writes float32
// partial tiles that a separate pass reduces in a fixed order.
//
// K groups (KG = 2 or 4): the workgroup holds KG sets of the four waves, each
// with its own two LDS stages, taking consecutive runs of ceil(steps / KG)
// BK-deep steps of the workgroup's K range; every group runs the same number of
// steps (they share the barriers), loads past the end of its run being
// zero-filled like any K tail.  Groups 1 .. KG-1 then park their sums in LDS
// and group 0 adds them in group order (a fixed order) and stores the tile: a
// split of K whose reduction stays on the CU.
#pragma once

#include "common.hpp"

namespace tg {

struct MfmaArgs {
    const void *A;
    const void *B;
    void *C;
    float *ws;        // split-K partials [splits][M][N], or null
    int64_t lda, ldb, ldc;
    int M, N, K;
    int kps;          // K range per split (multiple of BK)
    int splits;
    int tiles_m, tiles_n;
    OutEpi oe;        // output transform
    int c_vec;        // 1: C rows are 16-byte aligned and ldc % 4 == 0
    int rows_a;       // rows of A(i, k) the loads may touch, >= M (padded copies: M rounded up)
    int cols_b;       // columns of B(k, j) the loads may touch, >= N
    // stream-K schedule (ping-pong kernel only): the tiles' K stages laid end
    // to end, sk_total = tiles * sk_ipt, cut into gridDim.x equal runs
    int sk_ipt;       // K stages per tile
    int sk_rows;      // fix-up: tile rows per workgroup
    int64_t sk_total;
};

// Stream-K bookkeeping shared by the kernel and its fix-up: workgroup g of G
// owns stages [sk_start(g), sk_start(g + 1)) of the end-to-end sequence.
__host__ __device__ inline int64_t sk_start(int64_t g, int64_t total, int64_t G)
{
    const int64_t base = total / G, rem = total % G;
    return g * base + (g < rem ? g : rem);
}

// The workgroup that owns stage `it`.
__host__ __device__ inline int64_t sk_owner(int64_t it, int64_t total, int64_t G)
{
    const int64_t base = total / G, rem = total % G;
    const int64_t big = rem * (base + 1);
    return it < big ? it / (base + 1) : rem + (it - big) / base;
}

// 16-byte-chunk XOR swizzle of an LDS row (8 chunks per row).
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// Stages one operand's BK-deep slice (ROWS rows of the tile) into registers and
// then into LDS.  MN_CONTIG: the operand's contiguous dimension runs along the
// tile rows (A stored transposed, or B stored plain).
template <typename Tr, int ROWS, bool MN_CONTIG, bool VEC>
struct Stager {
    using T = typename Tr::T;
    static constexpr int E = Tr::E;
    static constexpr int BK = 8 * E;
    static constexpr int NBLK = 8 * ROWS / E;                 // E x E blocks per slice
    static constexpr int BPT = (NBLK + 255) / 256;            // blocks per thread
    static constexpr int NREG = MN_CONTIG ? BPT * E : ROWS / 32;

    u32x4 reg[NREG];
    const T *X;
    int64_t ld;
    int rows_total;  // M (for A) or N (for B)
    int row0;        // first tile row

    __device__ __forceinline__ void load(int tid, int k0, int kend, bool full)
    {
        if constexpr (!MN_CONTIG) {
            const int c = tid & 7;
            const int k = k0 + c * E;
#pragma unroll
            for (int p = 0; p < ROWS / 32; ++p) {
                const int r = (tid >> 3) + 32 * p;
                if constexpr (VEC) {
                    const int gr = min(row0 + r, rows_total - 1);
                    const T *ptr = X + (int64_t)gr * ld + k;
                    reg[p] = (full || k < kend) ? *(const u32x4 *)ptr : zero4();
                } else {
                    reg[p] = load_elems(row0 + r, k, kend, /*k_contig=*/true);
                }
            }
        } else {
            constexpr int PER_K = ROWS / E;  // blocks along the rows of one k-block
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int b = tid + 256 * q;
                const bool on = (NBLK % 256 == 0) || (b < NBLK);
                const int kb = b / PER_K, mb = b % PER_K;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int k = k0 + kb * E + e;
                    if constexpr (VEC) {
                        const int gc = min(row0 + mb * E, rows_total - E);
                        const T *ptr = X + (int64_t)k * ld + gc;
                        reg[q * E + e] = (on && (full || k < kend)) ? *(const u32x4 *)ptr : zero4();
                    } else {
                        reg[q * E + e] = on ? load_elems(row0 + mb * E, k, kend, false) : zero4();
                    }
                }
            }
        }
    }

    // Element-wise chunk load for operands without 16-byte alignment.
    // k_contig: E consecutive k of tile row `r`; else E consecutive rows at depth k.
    __device__ __forceinline__ u32x4 load_elems(int r, int k, int kend, bool k_contig) const
    {
        uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int rr = k_contig ? r : r + e;
            const int kk = k_contig ? k + e : k;
            if (rr < rows_total && kk < kend) {
                const T *ptr = k_contig ? X + (int64_t)rr * ld + kk : X + (int64_t)kk * ld + rr;
                if constexpr (Tr::kBytes == 4)
                    w[e] = __builtin_bit_cast(uint32_t, *ptr);
                else
                    h[e] = __builtin_bit_cast(uint16_t, *ptr);
            }
        }
        if constexpr (Tr::kBytes == 4)
            return u32x4{w[0], w[1], w[2], w[3]};
        else
            return u32x4{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                         h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16)};
    }

    __device__ __forceinline__ void store(int tid, u32x4 *lds) const
    {
        if constexpr (!MN_CONTIG) {
            const int c = tid & 7;
#pragma unroll
            for (int p = 0; p < ROWS / 32; ++p) {
                const int r = (tid >> 3) + 32 * p;
                lds[r * 8 + (c ^ swz(r))] = reg[p];
            }
        } else {
            constexpr int PER_K = ROWS / E;
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int b = tid + 256 * q;
                if ((NBLK % 256 == 0) || (b < NBLK)) {
                    const int kb = b / PER_K, mb = b % PER_K;
                    u32x4 t[E];
                    transpose_block<Tr::kBytes>(&reg[q * E], t);
#pragma unroll
                    for (int j = 0; j < E; ++j) {
                        const int r = mb * E + j;
                        lds[r * 8 + (kb ^ swz(r))] = t[j];
                    }
                }
            }
        }
    }
};

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int ntiles = tiles_m * tiles_n;
    // XCD-major remap: id -> (xcd = id % 8, slot = id / 8) -> contiguous run per XCD
    const int q = ntiles >> 3, r = ntiles & 7;
    const int x = bid & 7, s = bid >> 3;
    int lin = x * q + min(x, r) + s;
    // grouped raster: 8 tile rows at a time, walked down the columns
    constexpr int G = 8;
    const int width = G * tiles_n;
    const int g = lin / width;
    const int first = g * G;
    const int gs = min(tiles_m - first, G);
    const int in = lin - g * width;
    tm = first + in % gs;
    tn = in / gs;
}

template <typename Tr, int BM, int BN, bool TA, bool TB, bool VEC, int KG = 1>
__global__ __launch_bounds__(256 * KG) void mfma_gemm_kernel(MfmaArgs p)
{
    using T = typename Tr::T;
    constexpr int E = Tr::E;
    constexpr int BK = 8 * E;
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 16, FN = WN / 16;
    constexpr int STAGE = (BM + BN) * 8;  // 16-byte chunks per stage
    static_assert(KG == 1 || KG == 2 || KG == 4, "1, 2 or 4 K groups");

    __shared__ u32x4 lds_all[KG * 2 * STAGE];

    const int tid = threadIdx.x & 255;                 // thread within its K group
    const int kgrp = threadIdx.x >> 8;                 // K group (uniform per wave)
    u32x4 *const lds = lds_all + kgrp * (2 * STAGE);   // the group's two stages
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int z = blockIdx.y;
    const int kbeg_wg = z * p.kps;
    const int kend_wg = min(p.K, kbeg_wg + p.kps);
    const int nk = ((kend_wg - kbeg_wg + BK - 1) / BK + KG - 1) / KG;   // steps per group
    const int kbeg = kbeg_wg + kgrp * nk * BK;
    const int kend = min(kend_wg, kbeg + nk * BK);   // below kbeg for a group with no K

    Stager<Tr, BM, TA, VEC> sa;
    sa.X = (const T *)p.A; sa.ld = p.lda; sa.rows_total = p.rows_a; sa.row0 = m0;
    Stager<Tr, BN, !TB, VEC> sb;
    sb.X = (const T *)p.B; sb.ld = p.ldb; sb.rows_total = p.cols_b; sb.row0 = n0;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nk > 0) {
        {
            const bool full = kbeg + BK <= kend;
            sa.load(tid, kbeg, kend, full);
            sb.load(tid, kbeg, kend, full);
            sa.store(tid, lds);
            sb.store(tid, lds + BM * 8);
        }
        __syncthreads();

        const int fr = lane & 15;   // fragment row within a 16-row block
        const int fg = lane >> 4;   // lane group -> chunk within a k-block

        for (int t = 0; t < nk; ++t) {
            const int cur = t & 1;
            const bool more = t + 1 < nk;
            if (more) {
                const int k0 = kbeg + (t + 1) * BK;
                const bool full = k0 + BK <= kend;
                sa.load(tid, k0, kend, full);
                sb.load(tid, k0, kend, full);
            }
            const u32x4 *As = lds + cur * STAGE;
            const u32x4 *Bs = As + BM * 8;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int c = kb * 4 + fg;
                u32x4 af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int r = wm * WM + i * 16 + fr;
                    af[i] = As[r * 8 + (c ^ swz(r))];
                }
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int r = wn * WN + j * 16 + fr;
                    bfr[j] = Bs[r * 8 + (c ^ swz(r))];
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        mfma_chunk<Tr>(acc[i][j], bfr[j], af[i]);
            }
            if (more) {
                u32x4 *nxt = lds + (cur ^ 1) * STAGE;
                sa.store(tid, nxt);
                sb.store(tid, nxt + BM * 8);
            }
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds C[m][n .. n+3] of every 16 x 16 block
    if constexpr (KG > 1) {
        // groups 1 .. KG-1 park their sums in LDS (16 bytes per lane, lane-
        // linear), group 0 adds them in group order; the K loop ended with a
        // barrier, so the stages are free
        static_assert((KG - 1) * 4 * FM * FN * 64 <= KG * 2 * STAGE, "reduction area");
        f32x4 *xs = (f32x4 *)lds_all;
        auto slot = [&](int g, int i, int j) { return (((g - 1) * 4 + wave) * (FM * FN) + i * FN + j) * 64 + lane; };
        if (kgrp > 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    xs[slot(kgrp, i, j)] = acc[i][j];
        }
        __syncthreads();
        if (kgrp > 0)
            return;
#pragma unroll
        for (int g = 1; g < KG; ++g)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const f32x4 v = xs[slot(g, i, j)];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j][e] += v[e];
                }
    }
    const int fr = lane & 15, fg = lane >> 4;
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
            if (n >= p.N)
                continue;
            store_out4<Tr>(C + (int64_t)m * p.ldc + n, acc[i][j], p.N - n, p.c_vec && n + 3 < p.N, p.oe);
        }
    }
}

}  // namespace tg
