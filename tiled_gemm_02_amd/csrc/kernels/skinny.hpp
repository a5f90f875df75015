// skinny.hpp -- memory-bound narrow products: M large, N <= 128, K large.
//
// At N = 128 the product does about 124 FLOP per byte moved ("Matrix
// Multiplication Background User's Guide", section 2, works this example),
// below MI355X's ~315 FLOP/byte ridge, so the time is the time to stream A
// from HBM once.  A still needs the matrix cores: at 8 TB/s the multiply-adds
// arrive faster than the vector ALUs retire them.  The kernel is an HBM stream
// that feeds MFMAs, shaped by what the memory system rewards:
//   * every CU streams its own slice of A: a CU keeps only a bounded number of
//     cache lines in flight, so the full rate needs all 256 CUs reading
//     distinct data (two workgroups reading the same lines each wait a full
//     HBM round trip); a workgroup owns 64 rows of C and all of its columns
//     (64 or 128), and K is split across workgroups when the row blocks alone
//     leave CUs idle;
//   * B (small, L2-resident) is re-read by every row block; its lines come
//     from L2 with a short round trip;
//   * A and B move into LDS by buffer loads that write LDS directly
//     (buffer_load ... lds) in 64-deep K stages.  The two operands have rings
//     of their own: A, whose lines take an HBM round trip, keeps 9 to 13
//     stages in flight; B keeps 3.  Each copy instruction covers 1 KiB (8 rows
//     x 128 contiguous bytes of A).  The buffer bound turns rows past M,
//     columns past N and K past the range into zeros with no branch and no
//     tail path;
//   * one wave sustains only a few GB/s of such copies and its waits are in
//     issue order, so a 16-wave workgroup gives A and B separate copy waves
//     (8 each); four of the B waves also run the MFMAs (2 x 2 grid, each
//     32 rows x CN/2 columns of v_mfma_f32_16x16x32, fp32 accumulate);
//   * row blocks start their K sweep at different stages, which spreads the
//     concurrent requests over the memory channels (rows of A are a power of
//     two apart, so requests for one K offset crowd the same channels);
//   * LDS layouts are swizzled for gfx950's banks: A (and B stored N x K) as
//     K-contiguous rows of 8 chunks, B stored K x N as M/N-contiguous k-rows
//     read back transposed (ds_read_b64_tr_b16).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "mfma_gemm3.hpp"

namespace tg {

struct SkinnyArgs {
    const void *A;
    const void *B;
    void *C;
    float *ws;       // split partials [splits][M][N]
    int64_t lda, ldb, ldc;
    int M, N, K;
    int kps;         // K per split (multiple of kSkBK)
    int splits;
    int nrb;         // row blocks, ceil(M / rb)
    int rb;          // rows per block: 64 or 128
    int skew;        // stages between the start points of consecutive XCDs
    OutEpi oe;       // output transform
    int c_vec;
};

constexpr int kSkRows = 64;     // C rows per workgroup (the default; 128 is also built)
constexpr int kSkBK = 64;       // K per stage
constexpr int kSkLds = 144 * 1024;   // LDS of the two rings
constexpr int kSkStagesB = 4;        // B ring stages (A gets the rest)

// Raw buffer resource over [base, base + bytes): offsets at or past `bytes`
// read as zeros.  Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ u32x4 sk_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// One 16-byte-per-lane buffer load written straight into LDS at m0 + 16 lane.
// Its completion is counted by vmcnt; the compiler does not see it as a
// memory operation, so the waits are the caller's.
__device__ __forceinline__ void sk_copy(const u32x4 &rs, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "s"(rs)
                 : "memory", "m0");
}

// s_waitcnt leaving the copies of the y youngest stages (ND per stage) in
// flight, y <= Y.
template <int ND, int Y>
__device__ __forceinline__ void sk_wait_younger(int y)
{
    if constexpr (Y > 0) {
        if (y >= Y) {
            wait_vm_lgkm<Y * ND>();
            return;
        }
        sk_wait_younger<ND, Y - 1>(y);
    } else {
        wait_vm_lgkm<0>();
    }
}

// RB: rows of C (and of A) per workgroup, 64 or 128.  Taller blocks read each
// B stage for more rows: fewer of the CU's outstanding line requests go to B.
template <typename Tr, bool TB, int CN, int RB = kSkRows>
__global__ __launch_bounds__(1024) void skinny_kernel(SkinnyArgs p)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using T = typename Tr::T;
    constexpr int BK = kSkBK;
    constexpr int KS = BK / 32;                           // MFMA K steps per stage
    constexpr int WR = 2, WC = 2;                         // compute waves: a 2 x 2 grid
    static_assert(RB == 64 || RB == 128, "row block");
    constexpr int MB = RB / 16 / WR, NBK = CN / 16 / WC;  // 16 x 16 blocks per compute wave
    constexpr int A_BYTES = RB * BK * 2;                  // 8 or 16 KiB: copies of 1 KiB
    constexpr int NAC = RB / 64;                          // A copies per A wave per stage
    constexpr int B_BYTES = CN * BK * 2;                  // 8 or 16 KiB
    constexpr int SB = kSkStagesB;                        // B ring
    constexpr int SA = (kSkLds - SB * B_BYTES) / A_BYTES; // A ring: the rest of LDS
    constexpr int NBW = 8, NAW = 8;                       // B-copy waves 0..7, A-copy waves 8..15
    constexpr int NBC = B_BYTES / 1024 / NBW;             // B copies per B wave per stage
    constexpr int BCH = CN / 8;                           // chunks per k-row of B stored K x N
    constexpr uint32_t kOut = 0x80000000u;                // past every bound (bounds < 2^31)
    static_assert(NBC >= 1 && SA >= 3 && SB >= 2 && SA - 2 < 64, "rings");
    __shared__ __attribute__((aligned(1024))) char lds[SA * A_BYTES + SB * B_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fr = lane & 15, fg = lane >> 4;

    const int rb = blockIdx.x;
    const int row0 = rb * RB;
    const int z = blockIdx.y;
    const int kbeg = z * p.kps;
    const int kend = min(p.K, kbeg + p.kps);
    const int nst = max(0, (kend - kbeg + BK - 1) / BK);
    // start stage: row blocks rb and rb + 8 share an XCD (ids go round-robin
    // over the 8 XCDs); XCDs start skew stages apart, row blocks within one
    // XCD one stage apart
    const int s0 = nst > 0 ? (int)(((int64_t)(rb & 7) * p.skew + (rb >> 3)) % nst) : 0;

    const T *A = (const T *)p.A;
    const T *B = (const T *)p.B;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    const uint32_t ldsB = lds_base + SA * A_BYTES;

    // K offset of stage t: row blocks start their sweep at stage s0
    auto stage_k0 = [&](int t) {
        int ts = t + s0;
        ts = ts >= nst ? ts - nst : ts;
        return kbeg + ts * BK;
    };

    // A copy u of wave 8 + c (RB / 64 per stage): A rows 64 u + 8c .. + 7,
    // 128 bytes each; lane l stores chunk l % 8 of row 64 u + 8c + l / 8, i.e.
    // logical chunk (l % 8) ^ swz(row), into bytes [8192 u + 1024 c, + 1024)
    // of the stage (row r at 128 r).
    // B copy u of wave w (0..7): copy j = w + 8 u of the stage's B tile.  Stored
    // N x K, like A (rows are columns); stored K x N, k-rows of BCH chunks, lane
    // l storing chunk l % BCH of k-row (64 / BCH) j + l / BCH.
    // Per lane: the byte offset at K offset 0 and the stage-relative K it reads.
    constexpr int NC = NBC > NAC ? NBC : NAC;
    uint32_t c_off[NC];
    int c_k[NC];
    u32x4 rs;
    if (wave >= NBW) {
        const int c = wave - NBW;
        const int rows_here = min(RB, p.M - row0);
        rs = sk_rsrc(A + (int64_t)row0 * p.lda, (uint32_t)((int64_t)rows_here * p.lda * 2));
#pragma unroll
        for (int u = 0; u < NAC; ++u) {
            const int r = 64 * u + 8 * c + (lane >> 3);
            const int lc = (lane & 7) ^ kc3_swz<8>(r);
            c_k[u] = 8 * lc;
            c_off[u] = (uint32_t)(r * p.lda * 2 + 16 * lc);
        }
    } else {
        rs = TB ? sk_rsrc(B, (uint32_t)((int64_t)p.N * p.ldb * 2)) : sk_rsrc(B, (uint32_t)((int64_t)p.K * p.ldb * 2));
#pragma unroll
        for (int u = 0; u < NBC; ++u) {
            const int j = wave + NBW * u;
            if constexpr (TB) {
                const int n = 8 * j + (lane >> 3);
                const int lc = (lane & 7) ^ kc3_swz<8>(n);
                c_k[u] = 8 * lc;
                c_off[u] = n < p.N ? (uint32_t)(n * p.ldb * 2 + 16 * lc) : kOut;
            } else {
                const int k = (64 / BCH) * j + lane / BCH;
                const int n = 8 * ((lane % BCH) ^ mn3_swz<BCH>(k));
                c_k[u] = k;
                c_off[u] = n < p.N ? (uint32_t)(k * p.ldb * 2 + n * 2) : kOut;
            }
        }
    }
    auto issue_a = [&](int t) {
        const int k0 = stage_k0(t);
#pragma unroll
        for (int u = 0; u < NAC; ++u) {
            const uint32_t off = c_k[u] < kend - k0 ? c_off[u] + 2u * (uint32_t)k0 : kOut;
            sk_copy(rs, off, lds_base + (uint32_t)((t % SA) * A_BYTES + u * 8192 + (wave - NBW) * 1024));
        }
    };
    auto issue_b = [&](int t) {
        const int k0 = stage_k0(t);
        const uint32_t step = TB ? 2u * (uint32_t)k0 : (uint32_t)((int64_t)k0 * p.ldb * 2);
#pragma unroll
        for (int u = 0; u < NBC; ++u) {
            const uint32_t off = (c_k[u] < kend - k0 && c_off[u] != kOut) ? c_off[u] + step : kOut;
            sk_copy(rs, off, ldsB + (uint32_t)((t % SB) * B_BYTES + (wave + NBW * u) * 1024));
        }
    };

    const int wr = (wave >> 1) & 1, wc = wave & 1;
    uint32_t mnb[KS][2];
    if constexpr (!TB) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                mnb[ks][h] = mn3_base<BCH>(ldsB, ks, h, lane);
    }

    f32x4 acc[MB][NBK];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBK; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One straight-line loop per role (a role branch inside the loop would
    // make the compiler move the accumulators out of AGPRs every iteration).
    // Every role meets the same barrier once per stage: after it, stage t of
    // both rings has landed and every read of stage t - 1 is done, so the
    // slots of stage t - 1 are refilled.  A waves keep SA - 1 stages in flight
    // (HBM latency), B waves SB - 1 (L2 latency); each wave's vmcnt counts its
    // own copies only.
    if (wave >= NBW) {
#pragma unroll
        for (int t = 0; t < SA - 1; ++t)
            if (t < nst)
                issue_a(t);
        for (int t = 0; t < nst; ++t) {
            sk_wait_younger<NAC, SA - 2>(min(nst - 1, t + SA - 2) - t);
            lds_barrier();
            if (t + SA - 1 < nst)
                issue_a(t + SA - 1);
        }
        return;
    }
    auto b_loop = [&](auto compute) {
        constexpr bool kCompute = decltype(compute)::value;
#pragma unroll
        for (int t = 0; t < SB - 1; ++t)
            if (t < nst)
                issue_b(t);
        for (int t = 0; t < nst; ++t) {
            sk_wait_younger<NBC, SB - 2>(min(nst - 1, t + SB - 2) - t);
            lds_barrier();
            if (t + SB - 1 < nst)
                issue_b(t + SB - 1);
            if constexpr (kCompute) {
                const char *sa = lds + (t % SA) * A_BYTES;
                const char *sb = lds + SA * A_BYTES + (t % SB) * B_BYTES;
                const uint32_t so = (uint32_t)((t % SB) * B_BYTES);
                u32x4 fa[KS][MB], fb[KS][NBK];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int x = 0; x < MB; ++x)
                        fa[ks][x] = frag3_kc<8>(sa, 16 * (MB * wr + x), ks, lane);
#pragma unroll
                    for (int x = 0; x < NBK; ++x) {
                        if constexpr (TB)
                            fb[ks][x] = frag3_kc<8>(sb, 16 * (NBK * wc + x), ks, lane);
                        else
                            fb[ks][x] = frag3_mn<BCH>(mnb[ks][0] + so, mnb[ks][1] + so, 16 * (NBK * wc + x));
                    }
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int i = 0; i < MB; ++i)
#pragma unroll
                        for (int j = 0; j < NBK; ++j)
                            // the compiler's MFMA (accumulators in VGPRs): 6 % faster
                            // here than tied AGPR accumulators
                            mfma_chunk<Tr>(acc[i][j], fb[ks][j], fa[ks][i]);
            }
        }
    };
    if (wave >= WR * WC) {
        b_loop(std::false_type{});
        return;
    }
    b_loop(std::true_type{});

    // ---- epilogue: lane holds C[m][n .. n + 3] of each of its blocks
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int m = row0 + 16 * (MB * wr + i) + fr;
        if (m >= p.M)
            continue;
#pragma unroll
        for (int j = 0; j < NBK; ++j) {
            const int ncol = 16 * (NBK * wc + j) + 4 * fg;
            if (ncol >= p.N)
                continue;
            const f32x4 s = acc[i][j];
            if (p.splits > 1) {
                float *dst = p.ws + ((int64_t)z * p.M + m) * p.N + ncol;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (ncol + e < p.N)
                        dst[e] = s[e];
                continue;
            }
            store_out4<Tr>((T *)p.C + (int64_t)m * p.ldc + ncol, s, p.N - ncol, p.c_vec && ncol + 3 < p.N, p.oe);
        }
    }
#else
    (void)p;
#endif
}

}  // namespace tg
