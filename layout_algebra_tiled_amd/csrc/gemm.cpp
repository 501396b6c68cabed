// GEMM entry points: operand validation, planning and launch.
//
// The host API shape (validate, size the workspace, run, all with status
// codes) follows "CUTLASS, in depth", "A complete Hopper GEMM with the
// builder API"; the alignment and architecture refusals follow "CUTLASS and
// CuTe layouts", "Pitfalls". Operands are tensors (pointer + layout) and are
// classified by their stride-1 mode ("Layouts as Algebra: CUTLASS & CuTe",
// "One notation, and no more transposes"). The block tile grid is the
// tile-index mode of zipped_divide(D, tile) ("CUTLASS and CuTe layouts", "A
// layout is a shape and a stride").

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <cstring>

#include <mutex>

#include "gemm_kernels.hpp"
#include "layout_host.hpp"
#include "lt.h"
#include "tiled_config.hpp"

// Scratch of the allocation-free entry point (lt_gemm_run_noalloc): the
// split-K partials and arrival counters live here instead of in a caller's
// workspace. Each GPU the library runs on holds its own copy until the
// process ends. In host code this name is only a stand-in for the symbol:
// kernels get the device address looked up below, never the name itself.
static __device__ __align__(256) unsigned char scratch[LT_NOALLOC_SCRATCH_BYTES];

namespace lt {

lt_status ensure_device();   // device.hip

namespace {

// One rank-2 operand reduced to (extent, stride) per mode.
struct Mat {
    const void* ptr = nullptr;
    int dtype = 0;
    int64_t e0 = 0, e1 = 0;   // extents
    int64_t s0 = 0, s1 = 0;   // strides
    int64_t footprint = 0;    // cosize in elements
};

// A mode must coalesce to one leaf (or have extent 1).
lt_status mode_single(const Tree& m, int64_t* ext, int64_t* stride) {
    int64_t n;
    lt_status st = tree_size(m, &n);
    if (st != LT_OK) return st;
    if (n == 0) {   // an empty mode: its strides are never used
        *ext = 0;
        *stride = 0;
        return LT_OK;
    }
    Tree c = coalesce(m);
    if (c.s.size() != 1) return LT_ERR_UNSUPPORTED;
    *ext = c.s[0];
    *stride = c.s[0] == 1 ? 0 : c.d[0];
    return LT_OK;
}

lt_status read_mat(const lt_tensor* t, bool need_ptr, Mat* out) {
    if (!t) return LT_ERR_INVALID_ARGUMENT;
    if (t->dtype != LT_F16 && t->dtype != LT_BF16) return LT_ERR_UNSUPPORTED;
    Tree tr;
    lt_status st = from_pod(&t->layout, &tr);
    if (st != LT_OK) return st;
    if (tr.rank() != 2) return LT_ERR_INVALID_ARGUMENT;
    std::vector<Tree> ms = tr.modes();
    Mat m;
    st = mode_single(ms[0], &m.e0, &m.s0);
    if (st != LT_OK) return st;
    st = mode_single(ms[1], &m.e1, &m.s1);
    if (st != LT_OK) return st;
    st = tree_cosize(tr, &m.footprint);
    if (st != LT_OK) return st;
    m.ptr = t->ptr;
    m.dtype = t->dtype;
    if (need_ptr && !m.ptr && m.e0 * m.e1 > 0) return LT_ERR_INVALID_ARGUMENT;
    *out = m;
    return LT_OK;
}

// Stride-1 mode of an operand: 0 or 1, or -1 if neither. A mode of extent 1
// is contiguous trivially.
int unit_mode(const Mat& m) {
    if (m.e1 > 1 && m.s1 == 1) return 1;
    if (m.e0 > 1 && m.s0 == 1) return 0;
    if (m.e1 <= 1) return 1;
    if (m.e0 <= 1) return 0;
    return -1;
}

// Order of the data-parallel launch's 256x256 tiles. Rounds of 256
// workgroups run together, 32 on each XCD (workgroup w runs on XCD w mod 8,
// and each XCD takes its workgroups in order). Raster: XCD x takes the
// stretch of T/8 consecutive tiles from x*T/8 in groups of 8 tile rows
// walked down the rows before moving right ("CUTLASS, in depth", "Kernel
// schedules": L2-friendly tile order). Super-blocks: round k is the k-th
// 16x16 block of tiles (blocks in row order), XCD x taking its 8x4 part at
// rows 8 (x mod 2), columns 4 (x / 2); each XCD's L2 sees the same 8x4
// footprint either way, but the 256 tiles of a round touch 32 operand
// panels (16 of A, 16 of B) instead of up to 64 + 4 when the XCDs'
// stretches lie on different tile rows.
static void raster_tile(int64_t lin, int64_t tm, int64_t tn, int64_t* r, int64_t* c) {
    const int64_t gm0 = std::min<int64_t>(tm, 8), gsz = gm0 * tn, grp = lin / gsz, first = grp * gm0;
    const int64_t gm = std::min<int64_t>(tm - first, gm0), in = lin - grp * gsz;
    *r = first + in % gm;
    *c = in / gm;
}

// Panels (256 rows of A or 256 columns of B, K deep) a tile order fetches
// through a least-recently-used cache of `cap` whole panels: each round
// touches its A panels, then its B panels. A plain model of the part's
// last-level cache, which the planner uses only to compare the two orders.
static int64_t order_fetches(bool superblock, int64_t tm, int64_t tn, int64_t cap) {
    const int64_t T = tm * tn, per = T / 8;
    std::vector<int64_t> lru;   // panel ids, most recent last (A row r: r; B column c: tm + c)
    std::vector<char> mark(tm + tn);
    int64_t n = 0;
    for (int64_t k = 0; k < T / 256; ++k) {
        std::fill(mark.begin(), mark.end(), 0);
        for (int x = 0; x < 8; ++x)
            for (int j = 0; j < 32; ++j) {
                int64_t r, c;
                if (superblock) {
                    const int64_t sbn = tn / 16;
                    r = 16 * (k / sbn) + 8 * (x & 1) + (j & 7);
                    c = 16 * (k % sbn) + 4 * (x >> 1) + (j >> 3);
                } else {
                    raster_tile(x * per + 32 * k + j, tm, tn, &r, &c);
                }
                mark[r] = 1;
                mark[tm + c] = 1;
            }
        for (int64_t id = 0; id < tm + tn; ++id) {
            if (!mark[id]) continue;
            auto it = std::find(lru.begin(), lru.end(), id);
            if (it != lru.end())
                lru.erase(it);
            else
                ++n;
            lru.push_back(id);
            if ((int64_t)lru.size() > cap) lru.erase(lru.begin());
        }
    }
    return n;
}

// Super-blocks pay when a round's 32 panels fit the model's 192 MiB (of the
// part's 256 MB last-level cache), so the next round along a super-row
// finds A again, and the model fetches at most 85 % of the raster's panels.
// Measured (bf16, back to back, the two orders interleaved): 16384^2 x 8192
// 3177 vs 3307 us, 12288^3 2605 vs 2806, 16384 x 8192 x 8192 1596 vs 1728,
// 16384^2 x 12288 4645 vs 5082 (all chosen); 8192^3 789 vs 791, 8192 x
// 28672 x 8192 2745 vs 2664 (raster kept: all of A stays cached), 16384^3
// 6639 vs 6470 and 12288^2 x 16384 3950 vs 3894 (raster kept: a round's
// panels exceed the cache).
static bool superblock_pays(int64_t tm, int64_t tn, int64_t K) {
    const int64_t panel = 256 * K * 2, budget = int64_t(192) << 20;
    if (32 * panel > budget) return false;
    const int64_t cap = budget / panel;
    return 100 * order_fetches(true, tm, tn, cap) <= 85 * order_fetches(false, tm, tn, cap);
}

// 128-bit access of 16-bit elements: 16-byte aligned base and the non-unit
// stride a multiple of 8 elements ("CUTLASS and CuTe layouts", "Pitfalls";
// "CUTLASS, in depth", "Failure modes").
bool aligned(const Mat& m, int unit) {
    if (reinterpret_cast<uintptr_t>(m.ptr) % 16 != 0) return false;
    int64_t other = unit == 1 ? m.s0 : m.s1;
    int64_t other_ext = unit == 1 ? m.e0 : m.e1;
    return other_ext <= 1 || other % 8 == 0;
}

bool overlaps(const Mat& x, const Mat& y) {
    if (!x.ptr || !y.ptr || x.footprint == 0 || y.footprint == 0) return false;
    auto a0 = reinterpret_cast<uintptr_t>(x.ptr), a1 = a0 + 2 * x.footprint;
    auto b0 = reinterpret_cast<uintptr_t>(y.ptr), b1 = b0 + 2 * y.footprint;
    return a0 < b1 && b0 < a1;
}

struct Plan {
    lt_gemm_plan_info info;
    bool empty = false;          // M == 0 or N == 0
    bool transposed = false;     // solved as D^T = B^T A^T
    Mat A, B, C, D;              // after the transposition, if any
    int64_t M = 0, N = 0, K = 0;
    bool a_k = false, b_k = false;
    // tiled kernel: whole tiles, then a split-K remainder
    int64_t dp_tiles = 0, sk_tiles = 0;
    int sk_splits = 1;
    int64_t sk_counter_bytes = 0;   // workspace: counters first, then partials
    int tile_m = 256, tile_n = 256; // tiled kernel: block tile tile_m x tile_n
    int persist_grid = 0;           // > 0: persistent launch of this many workgroups
    bool superblock = false;        // the data-parallel launch walks 16x16-tile super-blocks
    bool krev = false;              // its odd rounds walk K downward
};

// Compute units of a gfx950 part (MI355X): the unit of wave quantisation.
constexpr int64_t kCUs = 256;

void transpose(Mat* m) {
    std::swap(m->e0, m->e1);
    std::swap(m->s0, m->s1);
}

lt_status make_plan(const lt_tensor* tA, const lt_tensor* tB, const lt_tensor* tC, const lt_tensor* tD,
                    int beta_nonzero, const lt_gemm_options* opt, Plan* plan) {
    Plan p;
    std::memset(&p.info, 0, sizeof(p.info));
    lt_status st;
    if ((st = read_mat(tA, true, &p.A)) != LT_OK) return st;
    if ((st = read_mat(tB, true, &p.B)) != LT_OK) return st;
    if ((st = read_mat(tD, true, &p.D)) != LT_OK) return st;
    if (beta_nonzero) {
        if (!tC) return LT_ERR_INVALID_ARGUMENT;
        if ((st = read_mat(tC, true, &p.C)) != LT_OK) return st;
    }
    if (p.A.dtype != p.B.dtype) return LT_ERR_UNSUPPORTED;
    if (beta_nonzero && p.C.dtype != p.D.dtype) return LT_ERR_UNSUPPORTED;
    if (p.D.dtype != p.A.dtype) return LT_ERR_UNSUPPORTED;
    // shapes: A (M,K), B (K,N), C/D (M,N)
    p.M = p.A.e0;
    p.K = p.A.e1;
    p.N = p.B.e1;
    if (p.B.e0 != p.K || p.D.e0 != p.M || p.D.e1 != p.N) return LT_ERR_INVALID_ARGUMENT;
    if (beta_nonzero && (p.C.e0 != p.M || p.C.e1 != p.N)) return LT_ERR_INVALID_ARGUMENT;
    if (p.M > INT32_MAX || p.N > INT32_MAX || p.K > INT32_MAX) return LT_ERR_OUT_OF_RANGE;

    // stride-1 modes and alignment
    const int ua = unit_mode(p.A), ub = unit_mode(p.B), ud = unit_mode(p.D);
    const int uc = beta_nonzero ? unit_mode(p.C) : 1;
    if (ua < 0 || ub < 0 || ud < 0 || uc < 0) return LT_ERR_UNSUPPORTED;
    if (!aligned(p.A, ua) || !aligned(p.B, ub) || !aligned(p.D, ud) || (beta_nonzero && !aligned(p.C, uc)))
        return LT_ERR_MISALIGNED_OPERAND;
    // D may be C exactly, never a partial overlap; never A or B.
    if (overlaps(p.D, p.A) || overlaps(p.D, p.B)) return LT_ERR_INVALID_ARGUMENT;
    if (beta_nonzero && overlaps(p.D, p.C) &&
        !(p.D.ptr == p.C.ptr && p.D.s0 == p.C.s0 && p.D.s1 == p.C.s1))
        return LT_ERR_INVALID_ARGUMENT;

    if (p.M == 0 || p.N == 0) {
        p.empty = true;
        *plan = p;
        return LT_OK;
    }

    // An M-major D is solved as D^T = B^T A^T: a transpose is a stride swap,
    // so the kernels only ever see an N-major output.
    if (ud == 0 && p.D.e1 != 1) {
        p.transposed = true;
        Mat a = p.A, b = p.B;
        p.A = b;
        transpose(&p.A);
        p.B = a;
        transpose(&p.B);
        transpose(&p.D);
        if (beta_nonzero) transpose(&p.C);
        std::swap(p.M, p.N);
    }
    p.a_k = p.A.e1 == 1 || p.A.s1 == 1;   // K-major A
    p.b_k = p.B.e0 == 1 || p.B.s0 == 1;   // K-major B
    const bool d_n = p.D.e1 == 1 || p.D.s1 == 1;
    const bool c_n = !beta_nonzero || p.C.e1 == 1 || p.C.s1 == 1;

    int kernel = opt ? opt->kernel : LT_KERNEL_AUTO;
    const TiledShape ts = tiled_shape(p.a_k, p.b_k, 256, 256);
    // M-major A and N-major B stream through the same kernel (transposed
    // fragment reads); any stride-1 mode of A and B works.
    // The tiled kernel addresses a K slice as a uniform base plus a per-lane
    // 32-bit byte offset: the largest such offset must stay below 4 GiB.
    auto offsets_fit = [&](bool kmaj, int64_t ld, int64_t rows) {
        const int64_t top = kmaj ? (rows - 1) * ld + ts.bk : (int64_t)(ts.bk - 1) * ld + rows;
        return top * 2 < (int64_t(1) << 32);
    };
    // Ragged M, N, K run on the tiled kernel too (edge tiles clamp their copy
    // rows and predicate their stores, a partial K slice is zero-filled), as
    // long as every copy moves whole 16-byte chunks: K a multiple of 8 for a
    // K-major operand, the M (N) extent a multiple of 8 for an M-major A
    // (N-major B).
    const bool chunks_ok = (p.a_k ? p.K % 8 == 0 : p.M % 8 == 0) && (p.b_k ? p.K % 8 == 0 : p.N % 8 == 0);
    const bool tiled_ok = p.K > 0 && d_n && c_n && chunks_ok && offsets_fit(p.a_k, p.a_k ? p.A.s0 : p.A.s1, p.M) &&
                          offsets_fit(p.b_k, p.b_k ? p.B.s1 : p.B.s0, p.N);
    // Automatic choice: the 256x256 kernel when the problem holds at least
    // one tile's worth of outputs and padding it to whole tiles adds at most
    // half again; the 16x16 kernel otherwise.
    const int64_t tm_ = (p.M + ts.bm - 1) / ts.bm, tn_ = (p.N + ts.bn - 1) / ts.bn;
    const bool tiled_pays = p.M * p.N >= (int64_t)ts.bm * ts.bn &&
                            2 * tm_ * ts.bm * tn_ * ts.bn <= 3 * p.M * p.N;
    int split = (opt && opt->split_k > 0) ? opt->split_k : 0;
    // The skinny kernel addresses 32 rows of A and 32 columns of B as a
    // uniform base plus a 32-bit per-lane byte offset.
    const bool skinny_offsets_fit = (31 * (p.A.e0 == 1 ? 0 : p.A.s0) + 256) * 2 < (int64_t(1) << 32) &&
                                    (31 * p.B.s1 + 256) * 2 < (int64_t(1) << 32);
    auto skinny_ok_for = [&](int s) {
        if (!(p.M <= 32 && p.a_k && p.b_k && d_n && c_n && p.N % kSkinnyBN == 0 && s >= 1 && skinny_offsets_fit))
            return false;
        const int64_t per = (int64_t)s * kSkinnyKQuantum;
        return p.K > 0 && p.K % per == 0;
    };
    if (kernel == LT_KERNEL_AUTO) {
        if (p.M <= 32 && skinny_ok_for(1)) {
            kernel = LT_KERNEL_SKINNY;
        } else if (tiled_ok && tiled_pays) {
            kernel = LT_KERNEL_TILED;
        } else {
            kernel = LT_KERNEL_WAVE16;
        }
    }
    lt_gemm_plan_info& in = p.info;
    in.kernel = kernel;
    in.a_kmajor = p.a_k;
    in.b_kmajor = p.b_k;
    in.d_nmajor = 1;
    in.split_k = 1;
    switch (kernel) {
        case LT_KERNEL_WAVE16: {
            if (opt && ((opt->tile_m && opt->tile_m != 16) || (opt->tile_n && opt->tile_n != 16)))
                return LT_ERR_UNSUPPORTED;
            in.tile_m = in.tile_n = 16;
            in.tile_k = 32;
            in.wave_m = in.wave_n = 16;
            in.waves = 4;
            in.stages = 0;
            const int64_t tiles = ((p.M + 15) / 16) * ((p.N + 15) / 16);
            in.grid = (tiles + 3) / 4;
            in.tiles = tiles;
            in.lds_bytes = 0;
            in.mfma_per_wave_kstep = 1;   // one 16x16x32 per 32-deep K step
            in.mfma_m = in.mfma_n = 16;
            in.mfma_k = 32;
            break;
        }
        case LT_KERNEL_TILED: {
            if (!tiled_ok) return d_n && c_n ? LT_ERR_NOT_DIVISIBLE : LT_ERR_UNSUPPORTED;
            const int want_n = opt ? opt->tile_n : 0;
            const int want_m = opt ? opt->tile_m : 0;
            if (want_m != 0 && want_m != 256 && want_m != 128) return LT_ERR_UNSUPPORTED;
            if (want_n != 0 && want_n != 256 && want_n != 128) return LT_ERR_UNSUPPORTED;
            if (want_m == 128 && want_n == 256) return LT_ERR_UNSUPPORTED;   // no 128x256 tile
            // 256x128 and 128x128 tiles are never split
            if ((want_n == 128 || want_m == 128) && split > 1) return LT_ERR_UNSUPPORTED;
            // Block tile and wave quantisation ("CUTLASS, in depth", "Worked
            // example: tile choice and wave quantisation"): ntiles whole
            // tiles on kCUs compute units leave the last round part empty.
            // Costs in K-slice times of a 256x128 tile (a 256x256 slice
            // counts two):
            //   256x256, data-parallel: ceil(n256/kCUs) * KT * 2;
            //   256x256 with the last round's rem tiles split into S K
            //     segments (S = kCUs/rem, at most 8, at least 4 slices
            //     each): whole rounds, ceil(KT/S), and 12 slices for each of
            //     the S-1 fp32 partials the last segment reads back through
            //     the coherent path (measured: 58 us for 4 partials, 125 us
            //     for 7), plus 24 when all 256x128 tiles fit one round (a
            //     partial costs about the same time, 9-10 us, but slices run
            //     faster on a part-empty chip: 2048x2048x8192 measured 87-90
            //     us in 128 whole 256x128 tiles against 91-92 us split 4
            //     ways), all times 2; taken when it saves 3 %;
            //   256x128: ceil(n128/kCUs) * KT * 23/20 (a 256x128 tile reads
            //     a sixth more LDS bytes per flop and has half the work to
            //     hide its prologue and epilogue behind).
            // split_k = 1 turns the split off; split_k > 1 forces S (on all
            // 256x256 tiles when they fill no whole round, else on the last
            // round's).
            const int64_t KTt = (p.K + ts.bk - 1) / ts.bk;
            const int64_t n256 = tm_ * tn_;
            const int64_t n128 = tm_ * ((p.N + 127) / 128);
            int64_t rem = n256 % kCUs;
            int64_t S = 1;
            int64_t c256 = (n256 + kCUs - 1) / kCUs * KTt * 2;
            if (split == 0) {
                if (rem != 0) {
                    S = std::min<int64_t>({kCUs / rem, 8, KTt / 4});
                    if (S >= 2) {
                        const int64_t t_split =
                            (n256 / kCUs * KTt + (KTt + S - 1) / S + 12 * (S - 1) + (n128 <= kCUs ? 24 : 0)) * 2;
                        if (100 * t_split < 97 * c256)
                            c256 = t_split;
                        else
                            S = 1;
                    }
                }
            } else if (split > 1) {
                S = std::min<int64_t>(split, KTt);
                if (rem == 0) rem = std::min<int64_t>(n256, kCUs);
            }
            if (S < 2) {
                S = 1;
                rem = 0;
            }
            const int64_t c128x20 = (n128 + kCUs - 1) / kCUs * KTt * 23;
            // 128x128: a quarter of a 256x256 tile's work per slice at a
            // lower rate (more LDS bytes per MFMA, shorter K steps to hide
            // the reads behind): 16 in the units in which a 256x128 slice
            // costs 23 (measured 14.5-16.2: bf16 1024^3 10.6 us against 16.8
            // for 256x128, 2048^3 20.7 against 29.4, 2048^2 x 8192 63.0
            // against 91.2; the larger tiles win from 3072^3: 72.9 against
            // 65.7 for 256x256); only for a fully automatic tile choice, and
            // against a split of 256x256 tiles only when they fill at least
            // half the CUs (1024^2 x 16384: 64 128x128 tiles 92.4 us, 16
            // tiles split 8 ways 83.7; 1536^2 x 12288: 144 tiles 77.1, the
            // split 96.1; 2048^2 x 16384: 256 tiles 117.3, the split 135.7)
            const int64_t n64 = ((p.M + 127) / 128) * ((p.N + 127) / 128);
            const int64_t c64x20 = (n64 + kCUs - 1) / kCUs * KTt * 16;
            int tile_m = 256, tile_n = 256;
            if (want_n == 128 || (want_n == 0 && split <= 1 && c128x20 < c256 * 20)) tile_n = 128;
            if (want_m == 128 || (want_m == 0 && want_n == 0 && split <= 1 && (S < 2 || 2 * n64 >= kCUs) &&
                                  c64x20 < std::min(c128x20, c256 * 20))) {
                tile_m = 128;
                tile_n = 128;
            }
            if (tile_n == 128) {
                S = 1;
                rem = 0;
            }
            const TiledShape tsc = tiled_shape(p.a_k, p.b_k, tile_m, tile_n);
            in.tile_m = tsc.bm;
            in.tile_n = tsc.bn;
            in.tile_k = tsc.bk;
            in.wave_m = tsc.wave_m;
            in.wave_n = tsc.wave_n;
            in.waves = tsc.waves;
            in.stages = tsc.stages;
            in.lds_bytes = tsc.lds_bytes;
            if (in.lds_bytes > 160 * 1024) return LT_ERR_LDS_OVERFLOW;
            const int64_t ntiles = tile_m == 128 ? n64 : tile_n == 128 ? n128 : n256;
            // Persistent launch of 256x128 tiles ("CUTLASS, in depth",
            // "Kernel schedules"): one workgroup per compute unit walks its
            // tiles and copies the next tile's first slices while the
            // current one finishes. Whole tiles only, K a multiple of the
            // slice depth, at least 4 slices per tile, and for 256x256 tiles
            // beta = 0 and no split remainder; chosen when the tiles take
            // more than one round of the compute units, for 256x256 tiles up
            // to 64 slices. Measured against one workgroup per tile (kernel
            // traces, interleaved): fp16 6144x4096x2048 256x128, beta = -1
            // 106.3 vs 111.5 us, beta = 0 101.7-107.3 vs 109.3 us; bf16
            // 256x256 8192^2 x 2048 214.5 vs 223.0 us, 6144x8192x4096 306.3
            // vs 311.6 us, 8192^2 x 4096 421.1 vs 425.5 us; at 8192^3 (128
            // slices, the part at its power cap) 752.0 vs 748.6 us with
            // events around each launch, so longer K stays one workgroup per
            // tile.
            const int want_p = opt ? opt->persistent : 0;
            if (want_p < 0 || want_p > 2) return LT_ERR_INVALID_ARGUMENT;
            // (256x256 tiles: beta = 0 and no split remainder only)
            // (with C, a copy of C rows reaches 16 rows of C through a 32-bit
            // byte offset)
            const bool c_rows_fit = !beta_nonzero || p.C.s0 * 2 * 16 < (int64_t(1) << 32);
            const bool persist_ok = tile_m == 256 && (tile_n == 128 || (!beta_nonzero && rem == 0)) &&
                                    p.M % tsc.bm == 0 &&
                                    p.N % tsc.bn == 0 && p.K % tsc.bk == 0 && KTt >= 4 && c_rows_fit;
            if (want_p == 2 && !persist_ok) return LT_ERR_UNSUPPORTED;
            const bool persist =
                persist_ok && (want_p == 2 || (want_p == 0 && ntiles > kCUs && (tile_n == 128 || KTt <= 64)));
            p.persist_grid = persist ? (int)std::min<int64_t>(ntiles, kCUs) : 0;
            in.persistent = persist ? 1 : 0;
            // tile order of the data-parallel launch (whole, unsplit 256x256
            // tiles in 16x16-tile super-blocks, or the raster)
            const int want_o = opt ? opt->tile_order : 0;
            if (want_o < 0 || want_o > 3) return LT_ERR_INVALID_ARGUMENT;
            const bool sb_ok = !persist && tile_m == 256 && tile_n == 256 && rem == 0 && tm_ % 16 == 0 &&
                               tn_ % 16 == 0;
            if (want_o == 2 && !sb_ok) return LT_ERR_UNSUPPORTED;
            p.superblock = sb_ok && (want_o == 2 || (want_o == 0 && superblock_pays(tm_, tn_, p.K)));
            // K-reversed raster: when a round's panels exceed the cache
            // model's 192 MiB (K above 12288), odd rounds walk K downward
            // and start on what the round before touched last. Measured
            // (bf16, back to back): 16384^3 6197 vs 6531 us, 12288^2 x 16384
            // 3739 vs 3885; neutral where the panels fit (8192^3 812 vs
            // 802-809, 12288^3 in super-blocks 2637 vs 2617)
            const bool kr_ok = !persist && tile_m == 256 && tile_n == 256 && rem == 0 && p.K % tsc.bk == 0 &&
                               n256 > kCUs;
            if (want_o == 3 && !kr_ok) return LT_ERR_UNSUPPORTED;
            p.krev = kr_ok && !p.superblock &&
                     (want_o == 3 || (want_o == 0 && 32 * 256 * p.K * 2 > (int64_t(192) << 20)));
            in.tile_order = persist ? 0 : p.superblock ? 2 : p.krev ? 3 : 1;
            p.tile_m = tile_m;
            p.tile_n = tile_n;
            p.dp_tiles = ntiles - rem;
            p.sk_tiles = rem;
            p.sk_splits = static_cast<int>(S);
            p.sk_counter_bytes = (rem * 4 + 255) / 256 * 256;
            in.split_k = p.sk_splits;
            in.grid = persist ? p.persist_grid : p.dp_tiles + rem * S;
            in.tiles = ntiles;
            in.sk_tiles = rem;
            in.sk_workgroups = static_cast<int32_t>(rem * S);
            in.workspace_bytes = rem > 0 ? p.sk_counter_bytes + rem * S * (int64_t)ts.bm * ts.bn * 4 : 0;
            // LDS per workgroup of the first launch (the persistent or the
            // data-parallel one; the split launch when every tile is split):
            // the ring plus the staged store's region, by the kernel's rule
            in.lds_bytes = launch_lds_bytes((int)tsc.lds_bytes,
                                            staged_d_launch(persist, !persist && p.dp_tiles > 0, p.a_k, p.b_k),
                                            persist && beta_nonzero);
            if (in.lds_bytes > 160 * 1024) return LT_ERR_LDS_OVERFLOW;
            // (wave_m/mf) * (wave_n/mf) * (bk/mfma_k): the analogue of counting mma
            // per warp per K slice ("CUTLASS and CuTe layouts", "The arch tag
            // is not one instruction")
            in.mfma_per_wave_kstep = tsc.mfma_per_wave_slice;
            in.mfma_m = in.mfma_n = tsc.mfma_mn;
            in.mfma_k = tsc.mfma_k;
            break;
        }
        case LT_KERNEL_SKINNY: {
            if (split == 0) {
                // enough workgroups to cover the 256 CUs, if K allows
                split = 1;
                const int64_t wgs = p.N / kSkinnyBN;
                while (wgs * split < 256 && skinny_ok_for(split * 2)) split *= 2;
            }
            if (!skinny_ok_for(split)) return LT_ERR_NOT_DIVISIBLE;
            in.tile_m = 32;
            in.tile_n = kSkinnyBN;
            in.tile_k = static_cast<int32_t>(p.K / split);
            in.wave_m = 32;
            in.wave_n = kSkinnyBN / kSkinnyWaves;   // the two waves split the columns
            in.waves = kSkinnyWaves;
            in.split_k = split;
            in.grid = (p.N / kSkinnyBN) * split;
            in.tiles = p.N / kSkinnyBN;
            in.lds_bytes = lt::SkinnyCfg::LDS;
            in.stages = lt::SkinnyCfg::R;
            in.workspace_bytes = split > 1 ? (int64_t)split * 32 * p.N * 4 : 0;
            in.mfma_per_wave_kstep = 4;   // two 16x16x32 (the two 16-row halves of A) per 32 of a 64-deep K block
            in.mfma_m = in.mfma_n = 16;
            in.mfma_k = 32;
            break;
        }
        default:
            return LT_ERR_INVALID_ARGUMENT;
    }
    *plan = p;
    return LT_OK;
}

// The last plan made on this thread, keyed by the bytes of its arguments: a
// workspace query followed by the run of the same problem (or a loop of runs)
// plans once. The plan depends on nothing but these arguments.
struct PlanKey {
    lt_tensor t[4];
    lt_gemm_options opt;
    int32_t has_c, has_opt, bnz;
};

lt_status plan_cached(const lt_tensor* tA, const lt_tensor* tB, const lt_tensor* tC, const lt_tensor* tD,
                      int beta_nonzero, const lt_gemm_options* opt, Plan* plan) {
    thread_local PlanKey last_key;
    thread_local Plan last_plan;
    thread_local bool have_last = false;
    if (!tA || !tB || !tD) return LT_ERR_INVALID_ARGUMENT;
    PlanKey k;
    std::memset(&k, 0, sizeof(k));
    std::memcpy(&k.t[0], tA, sizeof(lt_tensor));
    std::memcpy(&k.t[1], tB, sizeof(lt_tensor));
    if (tC && beta_nonzero) std::memcpy(&k.t[2], tC, sizeof(lt_tensor));
    std::memcpy(&k.t[3], tD, sizeof(lt_tensor));
    if (opt) std::memcpy(&k.opt, opt, sizeof(lt_gemm_options));
    k.has_c = tC && beta_nonzero ? 1 : 0;
    k.has_opt = opt ? 1 : 0;
    k.bnz = beta_nonzero ? 1 : 0;
    if (have_last && std::memcmp(&k, &last_key, sizeof(k)) == 0) {
        *plan = last_plan;
        return LT_OK;
    }
    const lt_status st = make_plan(tA, tB, tC, tD, beta_nonzero, opt, plan);
    if (st == LT_OK) {
        last_key = k;
        last_plan = *plan;
        have_last = true;
    }
    return st;
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

lt_status scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LT_ERR_HIP;
    if (dev < 0 || dev >= 64) return LT_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LT_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LT_OK;
}

}  // namespace
}  // namespace lt

extern "C" {

lt_status lt_gemm_plan(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                       int32_t beta_nonzero, const lt_gemm_options* opt, lt_gemm_plan_info* info) {
    lt::Plan p;
    lt_status st = lt::make_plan(A, B, C, D, beta_nonzero, opt, &p);
    if (st != LT_OK) return st;
    if (info) *info = p.info;
    return LT_OK;
}

lt_status lt_gemm_can_implement(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                                int32_t beta_nonzero, const lt_gemm_options* opt) {
    lt::Plan p;
    return lt::make_plan(A, B, C, D, beta_nonzero, opt, &p);
}

lt_status lt_gemm_workspace_size(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                                 int32_t beta_nonzero, const lt_gemm_options* opt, size_t* bytes) {
    if (!bytes) return LT_ERR_INVALID_ARGUMENT;
    lt::Plan p;
    lt_status st = lt::plan_cached(A, B, C, D, beta_nonzero, opt, &p);
    if (st != LT_OK) return st;
    *bytes = static_cast<size_t>(p.info.workspace_bytes);
    return LT_OK;
}

lt_status lt_gemm_run(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D, float alpha,
                      float beta, const lt_gemm_options* opt, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return lt_gemm_run_ex(A, B, C, D, alpha, beta, opt, nullptr, workspace, workspace_bytes, stream);
}

lt_status lt_gemm_run_ex(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                         float alpha, float beta, const lt_gemm_options* opt, const lt_epilogue* epi,
                         void* workspace, size_t workspace_bytes, void* stream) {
    lt::Plan p;
    const int bnz = beta != 0.0f;
    if (epi && (epi->activation < LT_ACT_NONE || epi->activation > LT_ACT_GELU || epi->bias_stride < 0))
        return LT_ERR_INVALID_ARGUMENT;
    lt_status st = lt::plan_cached(A, B, C, D, bnz, opt, &p);
    if (st != LT_OK) return st;
    if ((size_t)p.info.workspace_bytes > workspace_bytes || (p.info.workspace_bytes > 0 && !workspace) ||
        (p.info.workspace_bytes > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        return LT_ERR_WORKSPACE;
    lt::EpiArgs ea;
    if (epi && (epi->bias || epi->activation != LT_ACT_NONE || epi->amax)) {
        ea.fused = 1;
        ea.bias = static_cast<const uint16_t*>(epi->bias);
        ea.bias_stride = epi->bias_stride == 0 ? 1 : epi->bias_stride;
        // a transposed plan solves D^T: D's rows are its columns
        ea.bias_on_rows = (epi->bias_per_row != 0) != p.transposed ? 1 : 0;
        ea.act = epi->activation;
        ea.amax = epi->amax;
    }
    if (p.empty) {
        if (!ea.amax) return LT_OK;
        st = lt::ensure_device();
        if (st != LT_OK) return st;
        return lt::launch_zero_f32(ea.amax, stream) == 0 ? LT_OK : LT_ERR_HIP;   // max over no outputs
    }
    st = lt::ensure_device();
    if (st != LT_OK) return st;
    const int dt = p.A.dtype;
    const uint16_t* cptr = bnz ? static_cast<const uint16_t*>(p.C.ptr) : nullptr;
    int err = 0;
    if (ea.amax && (err = lt::launch_zero_f32(ea.amax, stream)) != 0) return LT_ERR_HIP;
    switch (p.info.kernel) {
        case LT_KERNEL_WAVE16: {
            lt::Wave16Args a;
            a.A = static_cast<const uint16_t*>(p.A.ptr);
            a.B = static_cast<const uint16_t*>(p.B.ptr);
            a.C = cptr;
            a.D = static_cast<uint16_t*>(const_cast<void*>(p.D.ptr));
            a.sam = p.A.s0;
            a.sak = p.A.e1 == 1 ? 1 : p.A.s1;
            a.sbk = p.B.e0 == 1 ? 1 : p.B.s0;
            a.sbn = p.B.s1;
            a.scm = bnz ? p.C.s0 : 0;
            a.scn = bnz ? (p.C.e1 == 1 ? 1 : p.C.s1) : 0;
            a.sdm = p.D.s0;
            a.sdn = p.D.e1 == 1 ? 1 : p.D.s1;
            a.M = (int)p.M;
            a.N = (int)p.N;
            a.K = (int)p.K;
            a.alpha = alpha;
            a.beta = beta;
            a.tiles_m = (int)((p.M + 15) / 16);
            a.tiles_n = (int)((p.N + 15) / 16);
            a.epi = ea;
            err = lt::launch_wave16(dt, a, stream);
            break;
        }
        case LT_KERNEL_TILED: {
            lt::TiledArgs a;
            a.A = static_cast<const uint16_t*>(p.A.ptr);
            a.B = static_cast<const uint16_t*>(p.B.ptr);
            a.C = cptr;
            a.D = static_cast<uint16_t*>(const_cast<void*>(p.D.ptr));
            // the non-unit stride of each operand (K-major A: row stride;
            // M-major A: K stride; likewise for B)
            a.lda = p.a_k ? p.A.s0 : p.A.s1;
            a.ldb = p.b_k ? p.B.s1 : p.B.s0;
            a.ldc = bnz ? p.C.s0 : 0;
            a.ldd = p.D.s0;
            a.M = (int)p.M;
            a.N = (int)p.N;
            a.K = (int)p.K;
            a.alpha = alpha;
            a.beta = beta;
            // The tile grid: mode 1 of zipped_divide(D', (256,256)), where D'
            // is D's layout with M and N rounded up to whole tiles (the
            // outputs past (M, N) are predicated off in the epilogue).
            const lt::TiledShape ts = lt::tiled_shape(p.a_k, p.b_k, p.tile_m, p.tile_n);
            const int64_t mp = (p.M + ts.bm - 1) / ts.bm * ts.bm, np = (p.N + ts.bn - 1) / ts.bn * ts.bn;
            lt::Tree dl = lt::Tree::tuple({lt::Tree::leaf(mp, p.D.s0), lt::Tree::leaf(np, 1)});
            const int64_t tiler[2] = {ts.bm, ts.bn};
            lt::Tree zd;
            st = lt::divide_shape(dl, 2, tiler, true, &zd);
            if (st != LT_OK) return st;
            lt::Tree grid = zd.mode(1);
            a.tiles_m = (int)grid.s[0];
            a.tiles_n = (int)grid.s[1];
            const int64_t kt = (p.K + ts.bk - 1) / ts.bk, kbase = p.K - kt * ts.bk;
            a.A0 = static_cast<const char*>(p.A.ptr) + kbase * (p.a_k ? 2 : 2 * a.lda);
            a.B0 = static_cast<const char*>(p.B.ptr) + kbase * (p.b_k ? 2 : 2 * a.ldb);
            a.group_m = std::min(a.tiles_m, 8);
            a.dp_tiles = (int)p.dp_tiles;
            a.sk_splits = p.sk_splits;
            // (a persistent grid is the tile count or 256: a multiple of 8
            // whenever the tile count is)
            a.xcd_remap = p.dp_tiles % 8 == 0 ? 1 : 0;
            a.superblock = p.superblock ? 1 : 0;
            a.krev = p.krev ? 1 : 0;
            a.counters = nullptr;
            a.partials = nullptr;
            if (p.sk_tiles > 0) {
                a.counters = static_cast<int*>(workspace);
                a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.sk_counter_bytes);
                if ((err = lt::launch_zero_i32(a.counters, (int)p.sk_tiles, stream)) != 0) return LT_ERR_HIP;
            }
            a.epi = ea;
            // the fused epilogue runs in the one-workgroup-per-tile launch
            err = lt::launch_tiled(dt, p.a_k, p.b_k, p.tile_m, p.tile_n, ea.fused ? 0 : p.persist_grid, a, stream);
            break;
        }
        case LT_KERNEL_SKINNY: {
            lt::SkinnyArgs a;
            a.A = static_cast<const uint16_t*>(p.A.ptr);
            a.B = static_cast<const uint16_t*>(p.B.ptr);
            a.C = cptr;
            a.D = static_cast<uint16_t*>(const_cast<void*>(p.D.ptr));
            a.ws = static_cast<float*>(workspace);
            a.lda = p.A.e0 == 1 ? 0 : p.A.s0;
            a.ldb = p.B.s1;
            a.ldc = bnz ? p.C.s0 : 0;
            a.ldd = p.D.s0;
            a.M = (int)p.M;
            a.N = (int)p.N;
            a.K = (int)p.K;
            a.alpha = alpha;
            a.beta = beta;
            a.split_k = p.info.split_k;
            a.k_per_wg = (int)(p.K / a.split_k);
            a.epi = ea;
            err = lt::launch_skinny(dt, a, stream);
            break;
        }
        default:
            return LT_ERR_INVALID_ARGUMENT;
    }
    return err == 0 ? LT_OK : LT_ERR_HIP;
}

lt_status lt_gemm_run_noalloc(const lt_tensor* A, const lt_tensor* B, const lt_tensor* C, const lt_tensor* D,
                              float alpha, float beta, const lt_gemm_options* opt, const lt_epilogue* epi,
                              void* stream) {
    lt::Plan p;
    lt_status st = lt::plan_cached(A, B, C, D, beta != 0.0f, opt, &p);
    if (st != LT_OK) return st;
    if (p.info.workspace_bytes > (int64_t)LT_NOALLOC_SCRATCH_BYTES) return LT_ERR_WORKSPACE;
    if (p.info.workspace_bytes == 0 || p.empty)
        return lt_gemm_run_ex(A, B, C, D, alpha, beta, opt, epi, nullptr, 0, stream);
    st = lt::ensure_device();   // the architecture gate comes before the device is touched
    if (st != LT_OK) return st;
    void* ws = nullptr;
    st = lt::scratch_address(&ws);
    if (st != LT_OK) return st;
    return lt_gemm_run_ex(A, B, C, D, alpha, beta, opt, epi, ws, LT_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
