// plan.h -- host-side planner: path choice, tile choice, split-K, and the
// tile/wave quantization model behind them.  Pure C++ (no HIP), so the model
// can be exercised on a machine without a GPU.
#pragma once

#include <stdint.h>

#include "../../include/tg_gemm.h"

namespace tg {

// Chip description the model plans against.
struct Chip {
    int num_cus = 256;            // MI355X: 8 XCDs x 32 CUs
    double clock_ghz = 2.4;       // peak engine clock
    double mfma16_flop_clk = 4096;  // dense fp16/bf16 matrix-core FLOP per clock per CU
    double mfma32_flop_clk = 256;   // fp32 matrix-core FLOP per clock per CU
    double valu_flop_clk = 256;     // fp32 vector FMA FLOP per clock per CU
    double hbm_gbs = 8000.0;      // HBM3E bandwidth, GB/s
    double launch_us = 3.0;       // cost charged per extra kernel launch
    double reduce_gbs = 2500.0;   // streaming rate of the split-K reduction kernel
};

// Everything the planner may look at for one call.
struct Problem {
    int64_t M, N, K;
    int dtype;       // tg_dtype
    int trans;       // tg_trans
    int64_t lda, ldb, ldc;
    bool ptrs_aligned;  // A, B (and C) 16-byte aligned
};

// Macro-tile kernels compiled into the library (tile_m x tile_n), per
// storage type, with their per-CU efficiency relative to the largest tile
// and the LDS each workgroup holds.  Element-wise ("generic") loads exist for
// one tile only.
struct TileSpec {
    int bm, bn;
    double eff;      // fraction of the dense matrix peak a saturated CU sustains
    int lds_kib;     // LDS per workgroup (2 stages)
    double sat;      // workgroups one CU needs at once to sustain eff (a lone small
                     // tile cannot hide its own load latency)
    int kg = 1;      // K groups: 2 or 4 sets of waves per workgroup, each over a part of
                     // the workgroup's K range, their sums added in LDS
    double fixed_us = 0.0;  // time per workgroup beyond its K loop (the K groups' LDS
                            // reduction, their fills), charged on top of the FLOP time
};

int tile_menu(int dtype, const TileSpec **out);       // vector-load tiles, largest first

// Residency of a tile kernel on one CU when no measured value is given:
// limited by LDS (160 KiB per CU) and the kernels' register use.
int model_occupancy(int dtype, int bm, int bn, bool vec, int kg = 1);

// Skinny kernel geometry (N <= kSkinnyMaxN): a workgroup covers 64 rows and
// all columns (64 or 128); K is split until the row blocks fill the CUs.
constexpr int kSkinnyRows = 64;        // output rows per workgroup (default)
constexpr int kSkinnyMaxRows = 128;    // the taller row block the kernel also offers
constexpr int kSkinnyMaxN = 128;       // widest output it covers in one pass
constexpr int kSkinnyBK = 64;          // K per pipeline stage, the granularity of a split
constexpr int kSkinnySkew = 16;        // stages between the K start points of consecutive XCDs
constexpr bool kSkinnyEnabled = true;

// Occupancy lookup: returns workgroups per CU for a tile kernel; the device
// path fills this from the runtime, the model from model_occupancy().
typedef int (*OccFn)(int dtype, int trans, int bm, int bn, bool vec, int kg, void *ctx);

// Plan one call.  occupancy > 0 forces that residency for every kernel.
// Returns TG_OK or a tg_status; `why` receives a static description on error.
// model: called from the pure model, which may price tiles no kernel offers.
int make_plan(const Problem &p, const Chip &chip, int occupancy, const tg_options *opts,
              OccFn occ, void *occ_ctx, bool model, tg_plan *out, const char **why,
              bool allow_pack = true);

// Operands that cannot take 16-byte loads (M, N, K, a leading dimension or a
// base pointer off the 16-byte grid) are copied, when the product is large
// enough, into zero-padded aligned buffers at the start of the workspace (plan
// vector_io == 2).  PackLayout describes those buffers; packed_problem() is
// the problem the kernels then see (M, N and K rounded up to 16 bytes, packed
// leading dimensions, aligned).  When M or N was rounded up only the
// macro-tile kernel runs the product: it reads the copies over their padded
// extent and stores the M x N result straight into C (its stores are bounded
// by M and N, its loads by M' and N').
//
// nt (float32 in a layout other than NT, plan vector_io == 3): the copies are
// laid out K-contiguous, A' = M' x K' and B' = N' x K', transposing the
// operands stored the other way, and the product runs as NT.  An aligned
// problem copies only the operands that need the transpose (no padding); the
// other is read in place.
struct PackLayout {
    int64_t a_rows, a_cols;   // stored A' (row-major): (trans_a ? K' x M' : M' x K'); nt: M' x K'
    int64_t b_rows, b_cols;   // stored B': (trans_b ? N' x K' : K' x N'); nt: N' x K'
    uint64_t a_off, b_off;    // byte offsets in the workspace
    uint64_t bytes;           // the copies; the kernels' own workspace follows
    bool padded_mn;           // M or N rounded up
    bool a_copy, b_copy;      // operand copied (else read in place)
    bool a_trans, b_trans;    // copy transposes the stored operand
};
PackLayout pack_layout(const Problem &p, bool nt = false);
Problem packed_problem(const Problem &p, bool nt = false);

// Widest leading dimension (elements) of a 16-bit operand the LDS-DMA
// kernels read in place: a tile's 256 rows then span less than 2^31 bytes.
constexpr int64_t kDmaMaxLd16 = (int64_t)1 << 22;

// The aligned copy of B behind a vector_io 4 plan (the skinny kernel with B's
// rows off the 16-byte grid): B stored K x N is copied with rows of N rounded
// up to 8 elements, B stored N x K with rows of K; zero-padded, at the start
// of the workspace, 256-byte aligned size.
inline int64_t skinny_b_ld(const Problem &p) { return (p.trans & TG_TRANS_B) ? p.K : (p.N + 7) / 8 * 8; }
inline uint64_t skinny_b_bytes(const Problem &p)
{
    const int64_t rows = (p.trans & TG_TRANS_B) ? p.N : p.K;
    return ((uint64_t)(rows * skinny_b_ld(p) * 2) + 255) & ~(uint64_t)255;
}

// 16-byte-chunk element count of a storage type.
inline int chunk_elems(int dtype) { return dtype == TG_F32 ? 4 : 8; }
inline int elem_bytes(int dtype) { return dtype == TG_F32 ? 4 : 2; }

// Row softmax launch shape for rows of N elements: the smallest register-
// resident form (q wave64s per row, c 16-byte chunks per lane, capacity
// q * 64 * c * chunk_elems) that holds the row, or q = c = 0 for the two-pass
// long-row kernel (N above kSoftmaxMaxResident).
constexpr int64_t kSoftmaxMaxResident = 32768;

// K depth of one stage of the 256 x 256 ping-pong kernel: the unit in which
// stream-K shares the tiles' K loops between workgroups.
constexpr int kStreamKStage = 32;
void softmax_shape(int dtype, int64_t N, int *q, int *c);

}  // namespace tg
