// plan.cpp -- the planner: which kernel, which tile, how many K-splits.
//
// The model follows "Matrix Multiplication Background User's Guide":
//   * section 2: arithmetic intensity 2MNK / (bytes of A, B, C) against the
//     chip's FLOP:byte ratio separates memory-bound calls (GEMV when M or N
//     is 1, the skinny kernel when one output dimension is small) from
//     math-bound ones;
//   * section 2.3: larger tiles reuse more data and run more efficiently,
//     smaller tiles give more parallel work; K may be split when M and N are
//     small and K large, at the price of a final reduction;
//   * section 3.1 (tile quantization): ceil(M/Mt) * ceil(N/Nt) tiles each do
//     a full tile of math, however little of it is useful;
//   * section 3.2 (wave quantization): tiles run in waves of
//     (compute units x tiles resident per unit); a partial last wave costs
//     about as much as a full one.
// Every candidate (tile, split) is priced as waves x time-per-wave, floored by
// the HBM time of the algorithmic bytes; ties (within 3%) go to the larger
// tile, then to fewer tiles, then to fewer splits.
#include "plan.h"

#include <algorithm>
#include <cmath>

namespace tg {

// Relative per-CU efficiencies are measured values of these kernels on
// MI355X (largest tile = 1); LDS is 2 stages x (BM + BN) rows x 128 bytes.
// eff: the fraction of the chip's dense matrix peak one saturated CU sustains
// with that tile's kernel, measured at 8192^3 fp16 on MI355X (256 x 256: the
// ping-pong kernel, about 1250 TFLOP/s under the board's power limit; the
// others: the 4-wave LDS-DMA kernel).
// sat: fitted to MI355X timings with one to four workgroups per CU (fp16
// 2304 x N x 4096 for N = 1536 .. 2560, 1024 x 1024 x 4096,
// 512 x 512 x 16384, 256 x 256 x 65536; float32 256^3 and 512^3): the small
// tiles need two or three workgroups per CU to hide their load latency.
// The two-group 128 x 128 kernel (eight waves, one workgroup per CU) keeps a K
// split of two on the CU: measured at 2304 x 1536..1792 x 4096, one workgroup
// per tile, it sustains 0.375 of a CU's peak, plus about 4 us per workgroup
// (the reduction in LDS and both groups' fills), which decides against it for
// short K (measured over 78 fp16 shapes x every tile and split: the picks with
// the fixed charge average 1.009x the best candidate's time, 1.011x without).
// 64 x 64 with four K groups (sixteen waves): small outputs with long K, where
// each group's chain of stages is a quarter of the one-group kernel's
// (256 x 256 x 65536 split 16: 35.8 against 40.4 us; 1024 x 1024 x 4096 in one
// launch: 20.6 against 21.8 us for split 4).
static const TileSpec kTiles16[] = {
    {256, 256, 0.50, 160, 1.0}, {192, 256, 0.42, 140, 1.0}, {256, 128, 0.355, 96, 1.0},
    {128, 128, 0.385, 64, 2.0}, {128, 128, 0.375, 128, 1.0, 2, 4.0},
    {128, 64, 0.31, 48, 2.5},   {64, 64, 0.22, 32, 2.0},    {64, 64, 0.20, 128, 1.0, 4, 4.0},
};
// float32: 256 x 256 is the ping-pong kernel, K-contiguous A and B only
// (tile_fits); the smaller tiles are the register-staged kernel.  Measured at
// 8192^3 on MI355X: 137.6 TFLOP/s (NT, 256 x 256) and 126 (NN, 128 x 128) of
// the 157.3 TFLOP/s float32 matrix peak.  With K groups (one workgroup per CU):
// 128 x 128 x 2 groups at 2048^3 and 1024 x 1024 x 4096 split 4, 0.68-0.71;
// 64 x 64 x 4 groups at 512^3 and 1024^3, 0.57; 32 x 32 x 4 groups (the
// smallest products, one launch on up to 256 CUs) set to 0.30, which makes it
// the plan for 128^3 to 512^3 (measured 256^3: 7.1 us against 10.1 us for
// 64 x 64 x 4 groups split 4).
static const TileSpec kTiles32[] = {
    {256, 256, 0.87, 160, 1.0},
    {128, 128, 0.80, 64, 2.0},
    {128, 128, 0.70, 128, 1.0, 2},
    {64, 64, 0.57, 128, 1.0, 4},
    {32, 32, 0.30, 64, 1.0, 4},
    {64, 64, 0.48, 32, 2.0},
};

int tile_menu(int dtype, const TileSpec **out)
{
    if (dtype == TG_F32) {
        *out = kTiles32;
        return (int)(sizeof kTiles32 / sizeof kTiles32[0]);
    }
    *out = kTiles16;
    return (int)(sizeof kTiles16 / sizeof kTiles16[0]);
}

// Whether the kernel behind a menu tile takes this problem's layout.
static bool tile_fits(const Problem &p, int bm, int bn)
{
    if (p.dtype == TG_F32 && bm == 256 && bn == 256)
        return p.trans == TG_NT && p.lda <= (1 << 21) && p.ldb <= (1 << 21);
    // 192 x 256: the ping-pong kernel with K-contiguous A
    if (bm == 192 && bn == 256)
        return p.dtype != TG_F32 && !(p.trans & TG_TRANS_A) && p.lda <= (1 << 22) && p.ldb <= (1 << 22);
    return true;
}

static const TileSpec *find_tile(int dtype, int bm, int bn, int kg = 1)
{
    const TileSpec *t;
    int n = tile_menu(dtype, &t);
    for (int i = 0; i < n; ++i)
        if (t[i].bm == bm && t[i].bn == bn && t[i].kg == kg)
            return &t[i];
    return nullptr;
}

int model_occupancy(int dtype, int bm, int bn, bool vec, int kg)
{
    (void)vec;
    kg = std::max(1, kg);
    const int lds_kib = kg * 2 * (bm + bn) * 128 / 1024;
    int by_lds = 160 / std::max(1, lds_kib);
    // register-limited residency (waves per SIMD) of each tile's wave sub-tile
    int by_regs;
    const int area = bm * bn;
    if (area >= 256 * 256)
        by_regs = 1;
    else if (area >= 256 * 128)
        by_regs = dtype == TG_F32 ? 2 : 1;
    else if (area >= 128 * 128)
        by_regs = 2;
    else if (area >= 128 * 64)
        by_regs = 3;
    else
        by_regs = 4;
    by_regs /= kg;   // each K group is a full set of waves
    return std::max(1, std::min(by_lds, by_regs));
}

static double flop_rate_cu(const Chip &c, int dtype)
{
    const double per_clk = dtype == TG_F32 ? c.mfma32_flop_clk : c.mfma16_flop_clk;
    return per_clk * c.clock_ghz * 1e9;
}

static double chip_peak(const Chip &c, int dtype) { return flop_rate_cu(c, dtype) * c.num_cus; }

static double alg_bytes(const Problem &p)
{
    const double s = elem_bytes(p.dtype);
    return s * ((double)p.M * p.K + (double)p.K * p.N + (double)p.M * p.N);
}

static void fill_common(const Problem &p, const Chip &chip, tg_plan *out)
{
    out->num_cus = chip.num_cus;
    const double bytes = alg_bytes(p);
    out->arith_intensity = bytes > 0 ? 2.0 * p.M * p.N * p.K / bytes : 0.0;
}

// Operands the 128-bit-load kernels take as they lie: leading dimensions,
// base pointers and the dimensions the 16-byte chunks run along on the
// 16-byte grid.  16-bit operands run on the LDS-DMA kernels, whose chunks run
// along each operand's contiguous dimension (K for A plain and B transposed,
// M for A transposed, N for B plain) and which clamp the rows past M and N, so
// M (A plain) and N (B transposed) may be ragged; they address a tile's rows
// by 32-bit byte offsets from a per-tile base: leading dimensions up to
// kDmaMaxLd16 elements.  Float32 keeps every dimension on the grid.  Other
// operands are read through aligned copies (or element-wise loads).
static bool vec_ok(const Problem &p)
{
    const int E = chunk_elems(p.dtype);
    if (p.dtype != TG_F32 && (p.lda > kDmaMaxLd16 || p.ldb > kDmaMaxLd16))
        return false;
    const bool ta = (p.trans & TG_TRANS_A) != 0, tb = (p.trans & TG_TRANS_B) != 0;
    const bool m_ok = p.M % E == 0 || (p.dtype != TG_F32 && !ta);
    const bool n_ok = p.N % E == 0 || (p.dtype != TG_F32 && tb);
    return p.ptrs_aligned && m_ok && n_ok && p.K % E == 0 && p.lda % E == 0 && p.ldb % E == 0;
}

// ---------------------------------------------------------------- GEMV

static int plan_gemv(const Problem &p, const Chip &chip, const tg_options *opts, tg_plan *out,
                     const char **why)
{
    (void)opts;
    if (!(p.M == 1 || p.N == 1)) {
        *why = "GEMV path needs M == 1 or N == 1";
        return TG_ERR_UNSUPPORTED;
    }
    const int E = chunk_elems(p.dtype);
    const bool ta = p.trans & TG_TRANS_A, tb = p.trans & TG_TRANS_B;
    // rows form: output elements are contiguous dot products
    const bool rows_form = (p.M == 1) ? tb : !ta;
    const int64_t n = (p.M == 1) ? p.N : p.M;
    out->path = TG_PATH_GEMV;
    out->tile_k = 0;
    out->occupancy = 8;
    if (rows_form) {
        out->tile_m = 4;   // outputs per workgroup (one per wave)
        out->tile_n = 1;
        out->split_k = 1;
        out->tiles = (n + 3) / 4;
        out->workgroups = out->tiles;
        out->workspace_bytes = 0;
        // vector loads need a unit-stride, aligned vector and aligned rows
        const int64_t vs = (p.M == 1) ? (ta ? p.lda : 1) : (tb ? 1 : p.ldb);
        const int64_t ldx = (p.M == 1) ? p.ldb : p.lda;
        // (the kernel reads a K tail past the last whole chunk element by element)
        out->vector_io = p.ptrs_aligned && vs == 1 && ldx % E == 0;
    } else {
        const int64_t ldx = (p.M == 1) ? p.ldb : p.lda;
        // (the chunk that straddles column n is read element by element)
        const bool vec = p.ptrs_aligned && ldx % E == 0;
        int64_t cols_per_wg = 64LL * E;  // element-wise kernel: 64 lanes x E columns
        int64_t rows_per_pass = 4;       // rows its workgroup covers per load
        if (vec) {
            // vector kernel: strips of lpr lanes x 16 bytes.  Wide row segments
            // (a wave reads up to 1 KiB of a row) keep the stream close to
            // sequential; the K split then gives every CU a workgroup, and the
            // narrower strips serve outputs too short for a full one.
            int lpr = 0;
            if (opts && opts->tile_n > 0) {
                lpr = opts->tile_n / E;
                if (lpr * E != opts->tile_n || (lpr != 8 && lpr != 16 && lpr != 32 && lpr != 64)) {
                    *why = "GEMV strips are 8, 16, 32 or 64 lanes of 16 bytes wide";
                    return TG_ERR_UNSUPPORTED;
                }
            } else {
                // 512-byte row segments measured fastest at 1 x 8192 x 8192
                lpr = 32;
                while (lpr > 8 && (int64_t)lpr * E / 2 >= n)
                    lpr /= 2;
            }
            cols_per_wg = (int64_t)lpr * E;
            rows_per_pass = 256 / lpr;
        }
        const int64_t strips = (n + cols_per_wg - 1) / cols_per_wg;
        int64_t ks;
        if (opts && opts->split_k > 0) {
            ks = std::min<int64_t>(opts->split_k, std::max<int64_t>(1, p.K));
        } else if (vec) {
            // about two workgroups per CU, each lane keeping 8 rows in flight;
            // keep at least that many rows per split
            ks = std::max<int64_t>(1, (2LL * chip.num_cus + strips - 1) / strips);
            ks = std::min<int64_t>(ks, std::max<int64_t>(1, p.K / (8 * rows_per_pass)));
        } else {
            // element-wise kernel: about 8 workgroups per CU
            const int64_t want = 8LL * chip.num_cus;
            ks = std::max<int64_t>(1, (want + strips - 1) / strips);
            ks = std::min<int64_t>(ks, std::max<int64_t>(1, p.K / 32));
        }
        int64_t rps = (p.K + ks - 1) / ks;
        rps = (rps + 3) / 4 * 4;
        ks = (p.K + rps - 1) / rps;
        out->tile_m = 1;
        out->tile_n = (int)cols_per_wg;
        out->split_k = (int)ks;
        out->tiles = strips;
        out->workgroups = strips * ks;
        out->workspace_bytes = ks > 1 ? (uint64_t)ks * (uint64_t)n * 4u : 0;
        out->vector_io = vec ? 1 : 0;
    }
    const int64_t slots = (int64_t)chip.num_cus * out->occupancy;
    out->waves = (out->workgroups + slots - 1) / slots;
    out->tile_eff = 1.0;
    out->wave_eff = (double)out->workgroups / (double)(out->waves * slots);
    const double bytes = alg_bytes(p) + (double)out->workspace_bytes * 2;
    out->pred_us = bytes / (chip.hbm_gbs * 1e3) + (out->split_k > 1 ? chip.launch_us : 0.0);
    out->pred_eff = (2.0 * p.M * p.N * p.K / (out->pred_us * 1e-6)) / chip_peak(chip, p.dtype);
    return TG_OK;
}

// ---------------------------------------------------------------- macro tiles

struct Cand {
    int bm, bn, s, occ, kps, kg;
    int64_t tiles, units, waves;
    double t, eff;
};

static Cand price(const Problem &p, const Chip &chip, int bm, int bn, int s, int occ, double eff,
                  double sat, double fixed_us = 0.0)
{
    Cand c{};
    const int BK = 8 * chunk_elems(p.dtype);
    c.kg = 1;
    c.bm = bm;
    c.bn = bn;
    c.occ = occ;
    c.eff = eff;
    int64_t kps = (p.K + s - 1) / s;
    kps = (kps + BK - 1) / BK * BK;
    c.kps = (int)kps;
    c.s = (int)((p.K + kps - 1) / kps);
    c.tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    c.units = c.tiles * c.s;
    const int64_t slots = (int64_t)chip.num_cus * occ;
    c.waves = (c.units + slots - 1) / slots;
    // A CU holding c workgroups at once runs at eff * min(1, c / sat) of its
    // peak (eff is measured with the tile's full residency, so sat <= occ),
    // shared among the c: one workgroup takes max(c, sat) times its work at
    // eff.  c is occ when the grid fills every slot, fewer when it is smaller.
    const int64_t per_cu = (c.units + chip.num_cus - 1) / chip.num_cus;
    const double conc = (double)std::min<int64_t>(occ, per_cu);
    const double t_unit = std::max(conc, std::min(sat, (double)occ)) *
                          ((2.0 * bm * bn * (double)kps) / (flop_rate_cu(chip, p.dtype) * eff) + fixed_us * 1e-6);
    // the tile kernel: waves of tiles, or its own HBM traffic (operands, and
    // the float32 partials it writes when K is split), whichever is longer
    const double partials = c.s > 1 ? (double)c.s * p.M * p.N * 4.0 : 0.0;
    double t = std::max(c.waves * t_unit, (alg_bytes(p) + partials) / (chip.hbm_gbs * 1e9));
    // a split adds the reduction kernel after it: partials in, C out
    if (c.s > 1)
        t += (partials + (double)p.M * p.N * elem_bytes(p.dtype)) / (chip.reduce_gbs * 1e9) +
             chip.launch_us * 1e-6;
    c.t = t;
    return c;
}

// Stream-K on 256 x 256 tiles (the ping-pong kernel: 16-bit, 16-byte-aligned
// operands, 32-deep K stages): G = one workgroup per CU shares the tiles' K
// stages evenly.  Only for fewer tiles than CUs, where a tile wave leaves CUs
// idle; each run is then shorter than a tile and touches at most two tiles.
static bool sk_ok(const Problem &p, const Chip &chip)
{
    const int64_t tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    return vec_ok(p) && p.dtype != TG_F32 && p.lda <= (1 << 22) && p.ldb <= (1 << 22) &&
           find_tile(p.dtype, 256, 256) != nullptr && tiles < chip.num_cus;
}

// Measured on MI355X (fp16, 2304 x N x 4096, 72-216 tiles): a stream-K stage
// takes about 1.9x a whole-tile stage.  The runs of one XCD sit at unrelated
// K offsets of their tiles, so the panel reuse in L2 that a wave of whole
// tiles gets (neighbouring tiles at the same K) is lost; the fix-up then reads
// every piece once at about 70 % of the HBM rate.
constexpr double kStreamKStageCost = 1.9;
constexpr double kStreamKFixupHbm = 0.7;

static Cand price_sk(const Problem &p, const Chip &chip, double eff)
{
    Cand c{};
    c.bm = c.bn = 256;
    c.occ = 1;
    c.eff = eff;
    c.s = -1;
    c.tiles = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    const int64_t ipt = (p.K + kStreamKStage - 1) / kStreamKStage;
    const int64_t total = c.tiles * ipt;
    const int64_t G = std::min<int64_t>(chip.num_cus, total);
    c.units = G;
    c.waves = 1;
    c.kps = kStreamKStage;
    const double t_stage =
        kStreamKStageCost * (2.0 * 256 * 256 * kStreamKStage) / (flop_rate_cu(chip, p.dtype) * eff);
    const double tile_f32 = 256.0 * 256.0 * 4.0;
    // longest run, then the last pieces written by every workgroup at once,
    // then the fix-up: every piece read once, the split tiles' C written
    const double pieces = (double)std::min<int64_t>(2 * G, G + c.tiles);
    double t = (double)((total + G - 1) / G) * t_stage;
    t = std::max(t, alg_bytes(p) / (chip.hbm_gbs * 1e9));
    t += (double)G * tile_f32 / (chip.hbm_gbs * 1e9);
    t += (pieces * tile_f32 + (double)p.M * p.N * elem_bytes(p.dtype)) /
             (kStreamKFixupHbm * chip.hbm_gbs * 1e9) +
         chip.launch_us * 1e-6;
    c.t = t;
    return c;
}

static int plan_mfma(const Problem &p, const Chip &chip, int occupancy, const tg_options *opts,
                     OccFn occ_fn, void *occ_ctx, bool model, tg_plan *out, const char **why)
{
    const bool vec = vec_ok(p);
    const int E = chunk_elems(p.dtype);
    const int BK = 8 * E;
    const TileSpec generic = {64, 64, 0.42, 32, 2.0};
    const TileSpec *menu;
    int nmenu;
    if (vec) {
        nmenu = tile_menu(p.dtype, &menu);
    } else {
        menu = &generic;
        nmenu = 1;
    }
    // K groups asked for: 0 = any offered (one when the tile is forced), 1, 2 or 4
    const int kg_req = opts ? opts->k_groups : 0;
    if (kg_req > 1 && !vec) {
        *why = "K groups need operands the 128-bit-load kernels read";
        return TG_ERR_UNSUPPORTED;
    }
    // forced tile
    TileSpec forced{};
    if (opts && (opts->tile_m > 0 || opts->tile_n > 0)) {
        if (opts->tile_m <= 0 || opts->tile_n <= 0) {
            *why = "a forced tile needs both tile_m and tile_n";
            return TG_ERR_ARG;
        }
        const int kg = std::max(1, kg_req);
        const TileSpec *f = vec ? find_tile(p.dtype, opts->tile_m, opts->tile_n, kg) : nullptr;
        if (f && !tile_fits(p, f->bm, f->bn))
            f = nullptr;
        if (!vec && opts->tile_m == 64 && opts->tile_n == 64)
            f = &generic;
        if (!f) {
            if (!model) {
                *why = kg > 1 ? "no kernel of the forced size with these K groups for these operands"
                              : "no macro-tile kernel of the forced size for these operands";
                return TG_ERR_UNSUPPORTED;
            }
            // the model prices any tile (e.g. another chip's tile menu)
            forced = TileSpec{opts->tile_m, opts->tile_n, 1.0, 0, 1.0, kg};
            f = &forced;
        }
        menu = f;
        nmenu = 1;
    }
    const bool force_sk = opts && opts->split_k == TG_SPLIT_STREAM_K;
    if (opts && opts->split_k < 0 && !force_sk) {
        *why = "split_k must be 0, positive, or TG_SPLIT_STREAM_K";
        return TG_ERR_ARG;
    }
    const bool tile_256 = !(opts && (opts->tile_m > 0 || opts->tile_n > 0)) ||
                          (opts->tile_m == 256 && opts->tile_n == 256);
    if (force_sk && !(tile_256 && sk_ok(p, chip))) {
        *why = "stream-K needs 16-bit, 16-byte-aligned operands with 256 x 256 tiles, "
               "and fewer tiles than compute units";
        return TG_ERR_UNSUPPORTED;
    }
    int splits[16];
    int nsplit = 0;
    if (force_sk) {
        // priced below
    } else if (opts && opts->split_k > 0) {
        splits[nsplit++] = opts->split_k;
    } else {
        const int cand[] = {1, 2, 3, 4, 6, 8, 12, 16};
        for (int s : cand)
            if (s == 1 || (int64_t)s * 2 * BK <= p.K)
                splits[nsplit++] = s;
    }
    bool have = false;
    Cand best{};
    // offered (not forced) only where each tile is shared by at most eight
    // workgroups: more pieces per tile cost more in the fix-up than they save
    const int64_t tiles256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    if (tile_256 && !(opts && opts->split_k > 0) && kg_req <= 1 && sk_ok(p, chip) &&
        (force_sk || tiles256 * 8 >= chip.num_cus)) {
        best = price_sk(p, chip, find_tile(p.dtype, 256, 256)->eff);
        have = true;
    }
    for (int i = 0; i < nmenu && !force_sk; ++i) {
        const TileSpec &ts = menu[i];
        if (!tile_fits(p, ts.bm, ts.bn) || (kg_req > 0 && ts.kg != kg_req))
            continue;
        int occ = occupancy > 0 ? occupancy
                                : (occ_fn ? occ_fn(p.dtype, p.trans, ts.bm, ts.bn, vec, ts.kg, occ_ctx)
                                          : model_occupancy(p.dtype, ts.bm, ts.bn, vec, ts.kg));
        occ = std::max(1, occ);
        for (int j = 0; j < nsplit; ++j) {
            Cand c = price(p, chip, ts.bm, ts.bn, splits[j], occ, ts.eff, ts.sat, ts.fixed_us);
            c.kg = ts.kg;
            if (!have) {
                best = c;
                have = true;
                continue;
            }
            const double tol = 0.03;
            if (c.t < best.t * (1 - tol)) {
                best = c;
            } else if (c.t <= best.t * (1 + tol)) {
                // near-tie: larger tile, then fewer tiles, then fewer splits
                const int64_t ac = (int64_t)c.bm * c.bn, ab = (int64_t)best.bm * best.bn;
                if (ac > ab || (ac == ab && (c.tiles < best.tiles ||
                                             (c.tiles == best.tiles && c.s < best.s))))
                    best = c;
            }
        }
    }
    if (!have) {
        *why = kg_req > 1 ? "no kernel with these K groups for these operands" : "no macro-tile kernel for these operands";
        return TG_ERR_UNSUPPORTED;
    }
    out->path = TG_PATH_MFMA;
    out->tile_m = best.bm;
    out->tile_n = best.bn;
    out->tile_k = BK;
    out->split_k = best.s;
    out->k_groups = best.s == TG_SPLIT_STREAM_K ? 1 : best.kg;
    out->occupancy = best.occ;
    out->vector_io = vec ? 1 : 0;
    out->tiles = best.tiles;
    out->workgroups = best.units;
    out->waves = best.waves;
    out->tile_eff = (double)p.M * p.N / ((double)best.tiles * best.bm * best.bn);
    out->wave_eff = (double)best.units / ((double)best.waves * chip.num_cus * best.occ);
    out->pred_us = best.t * 1e6;
    out->pred_eff = (2.0 * p.M * p.N * p.K / best.t) / chip_peak(chip, p.dtype);
    out->workspace_bytes = best.s > 1 ? (uint64_t)best.s * p.M * p.N * 4u : 0;
    if (best.s == TG_SPLIT_STREAM_K) {
        out->tile_k = kStreamKStage;
        out->wave_eff = (double)best.units / chip.num_cus;
        out->workspace_bytes = (uint64_t)2 * best.units * 256 * 256 * 4;
    }
    return TG_OK;
}

// ---------------------------------------------------------------- skinny

// The skinny kernel reads A in place as K-contiguous rows of 16-byte chunks
// (K and lda multiples of 8, A's pointer aligned) and B by 16-byte chunks of
// its rows (ldb a multiple of 8, B's pointer aligned).  M and N may be ragged:
// the buffer bounds read rows past M as zeros, the B copies skip chunks past
// N, and the C stores are masked (any ldc).  Buffer offsets are 32-bit with
// bit 31 reserved as "out of range": one row block of A, and all of B, must
// span less than 2^31 bytes.
static bool skinny_a_ok(const Problem &p)
{
    const int64_t lim = (int64_t)1 << 31;
    return p.dtype != TG_F32 && !(p.trans & TG_TRANS_A) && p.N >= 1 && p.N <= kSkinnyMaxN &&
           p.M >= 2 * kSkinnyRows && p.K % 8 == 0 && p.lda % 8 == 0 && p.ptrs_aligned &&
           (int64_t)kSkinnyMaxRows * p.lda * 2 < lim;
}

static bool skinny_fits(const Problem &p)
{
    const int64_t lim = (int64_t)1 << 31;
    const bool tb = (p.trans & TG_TRANS_B) != 0;
    return skinny_a_ok(p) && p.ldb % 8 == 0 && (tb ? p.N : p.K) * p.ldb * 2 < lim;
}

// B stored with rows off the 16-byte grid (ldb not a multiple of 8, e.g. a
// K x N matrix with a few columns): the skinny kernel runs on an aligned,
// zero-padded copy of B (skinny_b_ld).
static bool skinny_b_copy(const Problem &p) { return skinny_a_ok(p) && p.N >= 2 && p.ldb % 8 != 0; }

static int plan_skinny(const Problem &p, const Chip &chip, const tg_options *opts, tg_plan *out,
                       const char **why)
{
    if (!kSkinnyEnabled) {
        *why = "skinny kernel not built";
        return TG_ERR_UNSUPPORTED;
    }
    if (!skinny_fits(p)) {
        *why = "skinny path needs 16-bit operands, A not transposed, 1 <= N <= 128, M >= 128, "
               "K, lda and ldb multiples of 8, A and B 16-byte aligned, and operand spans below "
               "2 GiB";
        return TG_ERR_UNSUPPORTED;
    }
    const int BK = kSkinnyBK;
    // 128-row blocks read each B stage for twice the rows, so fewer of the
    // CU's outstanding requests go to B; measured on MI355X with 128-wide
    // outputs: 8192 x 128 x 8192 +9 %, 16384 x 128 x 8192 +8 %, but
    // 8192 x 128 x 16384 -15 % (rows of 32 KiB); 64-wide outputs: no change
    int rb = (p.N > 64 && p.K <= 8192 && p.M >= 2 * kSkinnyMaxRows) ? kSkinnyMaxRows : kSkinnyRows;
    if (opts && opts->tile_m > 0) {
        if (opts->tile_m != 64 && opts->tile_m != 128) {
            *why = "skinny row blocks are 64 or 128 rows";
            return TG_ERR_UNSUPPORTED;
        }
        rb = opts->tile_m;
    }
    const int64_t tm = (p.M + rb - 1) / rb;
    // split K until every CU streams its own part of A, four stages per split at least
    int s = 1;
    if (opts && opts->split_k > 0) {
        s = opts->split_k;
    } else {
        while (tm * s < (int64_t)chip.num_cus && (int64_t)(s * 2) * 4 * BK <= p.K && s < 16)
            s *= 2;
    }
    int64_t kps = (p.K + s - 1) / s;
    kps = (kps + BK - 1) / BK * BK;
    s = (int)((p.K + kps - 1) / kps);
    out->path = TG_PATH_SKINNY;
    out->tile_m = rb;
    out->tile_n = p.N > 64 ? 128 : 64;
    out->tile_k = BK;
    out->split_k = s;
    out->occupancy = 1;
    out->vector_io = 1;
    out->tiles = tm;
    out->workgroups = tm * s;
    const int64_t slots = (int64_t)chip.num_cus * out->occupancy;
    out->waves = (out->workgroups + slots - 1) / slots;
    out->tile_eff = (double)p.N / out->tile_n * (double)p.M / (tm * rb);
    out->wave_eff = (double)out->workgroups / (double)(out->waves * slots);
    out->workspace_bytes = s > 1 ? (uint64_t)s * p.M * p.N * 4u : 0;
    const double bytes = alg_bytes(p) + 2.0 * (double)out->workspace_bytes;
    out->pred_us = bytes / (chip.hbm_gbs * 1e3) + (s > 1 ? chip.launch_us : 0.0);
    out->pred_eff = (2.0 * p.M * p.N * p.K / (out->pred_us * 1e-6)) / chip_peak(chip, p.dtype);
    return TG_OK;
}

// ---------------------------------------------------------------- entry

// ---------------------------------------------------------------- row softmax

void softmax_shape(int dtype, int64_t N, int *q, int *c)
{
    // capacities 256 .. 32768 elements; one wave per row up to 1 KiB-4 KiB rows,
    // then more waves per row before more chunks per lane (more loads in flight
    // per row, the same registers per lane).  32 values per lane at most: a
    // 1024-thread workgroup has 128 registers per lane, and 64 values spill.
    static const int f32_shapes[][2] = {{1, 1}, {1, 2}, {1, 4}, {2, 4}, {4, 4},
                                        {8, 4}, {16, 4}, {16, 8}};
    static const int h16_shapes[][2] = {{1, 1}, {1, 2}, {2, 2}, {4, 2},
                                        {8, 2}, {16, 2}, {16, 4}};
    const int E = chunk_elems(dtype);
    const int (*shapes)[2] = E == 4 ? f32_shapes : h16_shapes;
    const int n = E == 4 ? 8 : 7;
    for (int i = 0; i < n; ++i) {
        if ((int64_t)shapes[i][0] * 64 * shapes[i][1] * E >= N) {
            *q = shapes[i][0];
            *c = shapes[i][1];
            return;
        }
    }
    *q = 0;
    *c = 0;
}

// ---------------------------------------------------------------- aligned copies

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Which operands the (non-transposing) aligned copies must copy.  A K tail
// off the 16-byte grid pads K in both (the padding must be zeros in both).
// Otherwise a 16-bit operand is copied only when the LDS-DMA kernels cannot
// read it as it lies (vec_ok's rules for that operand); float32 copies both.
static void copy_needs(const Problem &p, bool *a, bool *b)
{
    const int E = chunk_elems(p.dtype);
    const bool ta = (p.trans & TG_TRANS_A) != 0, tb = (p.trans & TG_TRANS_B) != 0;
    if (p.dtype == TG_F32 || p.K % E != 0 || !p.ptrs_aligned) {
        *a = *b = true;
        return;
    }
    *a = p.lda % E != 0 || (ta && p.M % E != 0) || p.lda > kDmaMaxLd16;
    *b = p.ldb % E != 0 || (!tb && p.N % E != 0) || p.ldb > kDmaMaxLd16;
}

Problem packed_problem(const Problem &p, bool nt)
{
    const int E = chunk_elems(p.dtype);
    Problem q = p;
    if (nt && vec_ok(p)) {
        // aligned: only the operands stored the other way are copied
        q.trans = TG_NT;
        if (p.trans & TG_TRANS_A)
            q.lda = p.K;
        if (!(p.trans & TG_TRANS_B))
            q.ldb = p.K;
        return q;
    }
    if (nt) {
        q.M = round_up(p.M, E);
        q.N = round_up(p.N, E);
        q.K = round_up(p.K, E);
        q.trans = TG_NT;
        q.lda = q.K;
        q.ldb = q.K;
        q.ptrs_aligned = true;
        return q;
    }
    // an operand read in place keeps its sizes and leading dimension, so no
    // kernel reads it past its own M or N
    bool a, b;
    copy_needs(p, &a, &b);
    q.K = round_up(p.K, E);
    q.M = a ? round_up(p.M, E) : p.M;
    q.N = b ? round_up(p.N, E) : p.N;
    if (a)
        q.lda = (p.trans & TG_TRANS_A) ? q.M : q.K;
    if (b)
        q.ldb = (p.trans & TG_TRANS_B) ? q.K : q.N;
    q.ptrs_aligned = true;
    return q;
}

PackLayout pack_layout(const Problem &p, bool nt)
{
    const Problem q = packed_problem(p, nt);
    const int64_t es = elem_bytes(p.dtype);
    PackLayout L;
    const bool ta = p.trans & TG_TRANS_A, tb = p.trans & TG_TRANS_B;
    if (nt) {
        const bool all = !vec_ok(p);
        L.a_copy = all || ta;
        L.b_copy = all || !tb;
        L.a_trans = ta;
        L.b_trans = !tb;
        L.a_rows = q.M;
        L.a_cols = q.K;
        L.b_rows = q.N;
        L.b_cols = q.K;
    } else {
        copy_needs(p, &L.a_copy, &L.b_copy);
        L.a_trans = L.b_trans = false;
        L.a_rows = ta ? q.K : q.M;
        L.a_cols = ta ? q.M : q.K;
        L.b_rows = tb ? q.N : q.K;
        L.b_cols = tb ? q.K : q.N;
    }
    L.a_off = 0;
    L.b_off = L.a_copy ? (uint64_t)round_up(L.a_rows * L.a_cols * es, 256) : 0;
    L.bytes = L.b_off + (L.b_copy ? (uint64_t)round_up(L.b_rows * L.b_cols * es, 256) : 0);
    L.padded_mn = q.M != p.M || q.N != p.N;
    return L;
}

// Worth copying: the element-wise kernel runs at a few percent of the vector
// ones, so above about 1 GFLOP (20 us of element-wise work) the copies (short
// launches and one pass over what they copy) pay for themselves many times.
// For 16-bit operands they also pay above 4 MB of operands: the element-wise
// kernel streams about 0.5 TB/s, a tenth of a copy pass, and the copies take
// only the operands the LDS-DMA kernels cannot read in place.  Float32
// copies are laid out for the NT kernel, transposing whole operands, which
// measured slower than the element-wise kernel on narrow products below
// 1 GFLOP (8192 x 7 x 8192: 205 against 160 us).  Below both, the launches
// would cost more than they save.  The transposing copy moves 64 x 64 blocks
// through LDS; it is priced at this fraction of the HBM rate.
static constexpr double kTransposeHbmFrac = 0.6;

static bool pack_worthwhile(const Problem &p)
{
    return p.M > 1 && p.N > 1 &&
           (2.0 * (double)p.M * (double)p.N * (double)p.K >= 1e9 ||
            (p.dtype != TG_F32 && alg_bytes(p) >= 4e6));
}

int make_plan(const Problem &p, const Chip &chip, int occupancy, const tg_options *opts,
              OccFn occ, void *occ_ctx, bool model, tg_plan *out, const char **why,
              bool allow_pack)
{
    static const char *none = "";
    *why = none;
    *out = tg_plan{};
    out->k_groups = 1;
    if (opts && !(opts->k_groups >= 0 && opts->k_groups <= 2) && opts->k_groups != 4) {
        *why = "k_groups must be 0, 1, 2 or 4";
        return TG_ERR_ARG;
    }
    if (p.M < 0 || p.N < 0 || p.K < 0) {
        *why = "negative dimension";
        return TG_ERR_ARG;
    }
    if (p.dtype < TG_F32 || p.dtype > TG_BF16) {
        *why = "unknown dtype";
        return TG_ERR_ARG;
    }
    if (p.trans < 0 || p.trans > 3) {
        *why = "unknown trans";
        return TG_ERR_ARG;
    }
    if (chip.num_cus <= 0) {
        *why = "num_cus must be positive";
        return TG_ERR_ARG;
    }
    fill_common(p, chip, out);
    out->split_k = 1;
    if (p.M == 0 || p.N == 0 || p.K == 0) {
        out->path = TG_PATH_NONE;
        out->pred_us = 0.0;
        return TG_OK;
    }
    // float32 copies are laid out for the NT product, whose 256 x 256 kernel
    // is the fastest float32 one
    const bool nt = p.dtype == TG_F32 && p.trans != TG_NT;
    const bool forced_other = opts && opts->path != TG_PATH_AUTO && opts->path != TG_PATH_MFMA;
    if (allow_pack && nt && vec_ok(p) && pack_worthwhile(p) && !forced_other) {
        // aligned float32 in another layout: the direct plan, or a transposed
        // copy of the operand(s) stored M/N-contiguous and the NT plan,
        // whichever the model prices lower
        tg_plan direct;
        const int rc_d = make_plan(p, chip, occupancy, opts, occ, occ_ctx, model, &direct, why, false);
        const Problem q = packed_problem(p, true);
        const PackLayout L = pack_layout(p, true);
        tg_plan inner;
        const char *why_n = none;
        const int rc_n = make_plan(q, chip, occupancy, opts, occ, occ_ctx, model, &inner, &why_n, false);
        const double copy_us = 2.0 * (double)L.bytes / (chip.hbm_gbs * 1e3 * kTransposeHbmFrac) +
                               (L.a_copy + L.b_copy) * chip.launch_us;
        if (rc_n == TG_OK && inner.vector_io == 1 &&
            (rc_d != TG_OK || inner.pred_us + copy_us < direct.pred_us)) {
            *out = inner;
            out->vector_io = 3;
            out->workspace_bytes = L.bytes + inner.workspace_bytes;
            out->pred_us += copy_us;
            fill_common(p, chip, out);
            *why = none;
            return TG_OK;
        }
        if (rc_d == TG_OK)
            *out = direct;
        return rc_d;
    }
    // a forced tile or two K groups ask for the macro-tile kernel
    const bool tile_forced = opts && (opts->tile_m > 0 || opts->tile_n > 0 || opts->k_groups > 1);
    const bool skinny_ok = kSkinnyEnabled &&
                           ((!opts || opts->path == TG_PATH_AUTO) ? !tile_forced : opts->path == TG_PATH_SKINNY);
    const double ridge = chip_peak(chip, p.dtype) / (chip.hbm_gbs * 1e9);
    const bool narrow = p.M > 1 && p.N > 1 && out->arith_intensity < ridge;
    if (allow_pack && skinny_ok && narrow && skinny_b_copy(p)) {
        // a narrow product whose B rows are off the 16-byte grid: copy B alone
        // (K x N is small) and stream A in place with the skinny kernel
        Problem q = p;
        q.ldb = skinny_b_ld(p);
        tg_plan inner;
        const char *why_s = none;
        if (plan_skinny(q, chip, opts, &inner, &why_s) == TG_OK) {
            const uint64_t bbytes = skinny_b_bytes(p);
            *out = inner;
            out->vector_io = 4;
            out->workspace_bytes = bbytes + inner.workspace_bytes;
            out->pred_us += 2.0 * (double)bbytes / (chip.hbm_gbs * 1e3) + chip.launch_us;
            fill_common(p, chip, out);
            return TG_OK;
        }
    }
    // (a narrow product the skinny kernel reads as it lies needs no copies)
    if (allow_pack && !vec_ok(p) && pack_worthwhile(p) && !(opts && opts->path == TG_PATH_GEMV) &&
        !(skinny_ok && narrow && skinny_fits(p))) {
        // plan the padded, aligned copy ("Matrix Multiplication Background
        // User's Guide", section 2.2, Table 1 and Figure 2: 16-bit products run
        // best with sizes that are multiples of 8 elements; padding is how a
        // caller gets there)
        const Problem q = packed_problem(p, nt);
        const PackLayout L = pack_layout(p, nt);
        tg_plan inner;
        int rc = make_plan(q, chip, occupancy, opts, occ, occ_ctx, model, &inner, why, false);
        if (L.padded_mn && forced_other)
            rc = TG_ERR_UNSUPPORTED;  // the forced path keeps its own element-wise form
        else if (rc == TG_OK && L.padded_mn && inner.path != TG_PATH_MFMA) {
            // only the macro-tile kernel reads past M and N
            tg_options o = opts ? *opts : tg_options{TG_PATH_AUTO, 0, 0, 0};
            o.path = TG_PATH_MFMA;
            rc = make_plan(q, chip, occupancy, &o, occ, occ_ctx, model, &inner, why, false);
        }
        if (rc == TG_OK && inner.vector_io == 1) {
            *out = inner;
            out->vector_io = nt ? 3 : 2;
            out->workspace_bytes = L.bytes + inner.workspace_bytes;
            out->pred_us += 2.0 * (double)L.bytes / (chip.hbm_gbs * 1e3) + 2.0 * chip.launch_us;
            fill_common(p, chip, out);
            return TG_OK;
        }
        *why = "";
    }
    int path = opts ? opts->path : TG_PATH_AUTO;
    if (path == TG_PATH_AUTO && tile_forced)
        path = TG_PATH_MFMA;  // a forced macro tile means the macro-tile kernel
    if (path != TG_PATH_MFMA && path != TG_PATH_AUTO && opts && opts->k_groups > 1) {
        *why = "K groups exist on the macro-tile path only";
        return TG_ERR_UNSUPPORTED;
    }
    if (path == TG_PATH_AUTO) {
        if (p.M == 1 || p.N == 1)
            path = TG_PATH_GEMV;
        else if (kSkinnyEnabled && skinny_fits(p) && out->arith_intensity < ridge)
            path = TG_PATH_SKINNY;
        else
            path = TG_PATH_MFMA;
    }
    int rc;
    switch (path) {
    case TG_PATH_MFMA:
        rc = plan_mfma(p, chip, occupancy, opts, occ, occ_ctx, model, out, why);
        break;
    case TG_PATH_GEMV:
        rc = plan_gemv(p, chip, opts, out, why);
        break;
    case TG_PATH_SKINNY:
        rc = plan_skinny(p, chip, opts, out, why);
        break;
    default:
        *why = "unknown forced path";
        rc = TG_ERR_ARG;
    }
    if (rc == TG_OK)
        fill_common(p, chip, out);
    return rc;
}

}  // namespace tg
