// Launch interface between the host planner (gemm.cpp) and the HIP kernels
// (gemm_kernels.hip). Internal; not part of the public ABI.
#pragma once

#include <cstdint>

namespace lt {

// Fused epilogue ("CUTLASS, in depth", "Epilogue fusion"): after
// alpha*acc + beta*C, add a bias vector and apply an activation while the
// accumulators are in registers, and reduce max |D| for output scaling.
struct EpiArgs {
    int fused = 0;                 // 0: plain alpha/beta epilogue (the rest unused)
    const uint16_t* bias = nullptr;  // D's dtype; nullptr: no bias
    int64_t bias_stride = 1;       // elements between consecutive bias values
    int bias_on_rows = 0;          // 1: bias[m] for row m; 0: bias[n] for column n
    int act = 0;                   // lt_activation
    float* amax = nullptr;         // max |stored D| (as float bits, atomic max); nullptr: none
};

// Generic wave-per-16x16-tile kernel: any strides, ragged M/N/K.
struct Wave16Args {
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* C;
    uint16_t* D;
    int64_t sam, sak;   // A(m,k) at m*sam + k*sak
    int64_t sbk, sbn;   // B(k,n) at k*sbk + n*sbn
    int64_t scm, scn;   // C(m,n)
    int64_t sdm, sdn;   // D(m,n)
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;   // tile grid: mode 1 of zipped_divide(D, (16,16)), colex
    EpiArgs epi;
};

// 256x256 block-tiled kernel. A is K-major or M-major, B is K-major or
// N-major, D and C are N-major. Any M, N, K >= 1, with copies in whole 16-byte
// chunks: K a multiple of 8 for a K-major operand, M (N) a multiple of 8 for
// an M-major A (N-major B). tiles_m/tiles_n = ceil(M/256)/ceil(N/256).
struct TiledArgs {
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* C;
    uint16_t* D;
    int64_t lda, ldb, ldc, ldd;   // the non-unit stride of each operand
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;
    int group_m;                  // tile rows per raster group
    int xcd_remap;                // 1: spread consecutive tiles over one XCD
    int superblock;               // 1: the data-parallel launch walks 16x16-tile super-blocks
    int krev;                     // 1: its odd rounds of 256 workgroups walk K downward
    // A and B moved to the start of K slice 0, k = kbase = K - ceil(K/BK)*BK
    // (<= 0): a pointer offset only, never dereferenced below k = 0
    const void* A0;
    const void* B0;
    EpiArgs epi;
    // Data-parallel tiles plus a split-K remainder: the first dp_tiles
    // tiles (raster order) are computed whole, one workgroup each; each of
    // the remaining tiles is split into sk_splits K segments, one workgroup
    // each (a second launch), whose fp32 partials meet in `partials`
    // ([tile][split][256*256]); the segment that finishes last (counted in
    // `counters`, one int per split tile, zero on entry and left zero) adds
    // the others and stores.
    int dp_tiles;
    int sk_splits;
    float* partials;
    int* counters;
};

// Skinny kernel: M <= 32, K-major A and B, N-major D; B streamed once.
struct SkinnyArgs {
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* C;
    uint16_t* D;
    float* ws;                    // split_k > 1: fp32 partials [split_k][32][N]
    int64_t lda, ldb, ldc, ldd;
    int M, N, K;
    float alpha, beta;
    int split_k;
    int k_per_wg;                 // K elements per workgroup (a multiple of 128)
    EpiArgs epi;
};

constexpr int kSkinnyWaves = 2;     // waves per workgroup (16 of its columns each)
constexpr int kSkinnyBN = 32;       // columns of N per workgroup
// The two waves of a skinny workgroup take 16 of its 32 columns each and
// share one LDS ring. A slot of the ring holds 256 deep of the 32 A rows and
// the 32 B columns (512 contiguous bytes of each row or column); each wave
// copies its 16 B columns and 16 of the A rows. The ring depth keeps the
// slots in flight within the 6-bit vmcnt and the ring within 160 KiB of LDS.
struct SkinnyCfg {
    static constexpr int SK = 256;                 // K per slot
    static constexpr int CB = 2 * SK;              // bytes of one row or column per slot
    static constexpr int HALF = 32 * CB;           // bytes of the A (or B) half of a slot
    static constexpr int SLOT = 2 * HALF;          // bytes of one slot
    static constexpr int NW = SLOT / 2048;         // 16-byte-per-lane copies per wave per slot
    static constexpr int KSTEPS = SK / 32;         // 16x16x32 MFMA steps per slot
    static constexpr int R_VM = 1 + 63 / NW;
    static constexpr int R_LDS = 160 * 1024 / SLOT;
    static constexpr int R = R_VM < R_LDS ? R_VM : R_LDS;   // ring slots: R - 1 slots in flight
    static constexpr int LDS = R * SLOT;           // bytes per workgroup
    static_assert(R >= 3, "the ring issues a slot after the barrier that frees it");
};
// The K range of a workgroup must be a whole number of 256-deep slots
constexpr int kSkinnyKQuantum = 256;

// Compile-time shape of the tiled kernel the planner launches.
struct TiledShape {
    int bm, bn, bk;          // block tile and K slice
    int wave_m, wave_n;      // tile of one wave
    int waves;               // waves per workgroup
    int stages;              // LDS ring depth
    int lds_bytes;           // per workgroup
    int mfma_per_wave_slice; // MFMAs per wave per K slice
    int mfma_mn, mfma_k;     // MFMA instruction: mfma_mn x mfma_mn outputs, K depth
};
// The block shape of the data-parallel launch of the tiled kernel for a
// block tile tile_m x tile_n (256x256, 256x128 or 128x128).
TiledShape tiled_shape(bool a_kmajor, bool b_kmajor, int tile_m, int tile_n);

// Each returns 0 on success or the hipError_t of the launch.
int launch_wave16(int dtype, const Wave16Args& a, void* stream);
int launch_tiled(int dtype, bool a_kmajor, bool b_kmajor, int tile_m, int tile_n, int persist_grid,
                 const TiledArgs& a, void* stream);
// The variants of the tiled kernel, launch_tiled_<dtype><A K-major>_<B
// K-major>; each is compiled in a translation unit of its own
// (gemm_tiled.hip built with LT_TILED_DT / LT_TILED_AK / LT_TILED_BK).
int launch_tiled_11_1(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_11_0(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_10_1(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_10_0(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_21_1(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_21_0(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_20_1(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_tiled_20_0(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream);
int launch_skinny(int dtype, const SkinnyArgs& a, void* stream);
// *p = 0.0f on the stream (a one-thread kernel: no memset node in a captured graph)
int launch_zero_f32(float* p, void* stream);
// p[0..n) = 0 on the stream (a fill kernel, for the same reason)
int launch_zero_i32(int* p, int n, void* stream);

}  // namespace lt
