// GEMM kernels for gfx950 (CDNA4): D = alpha * A*B + beta * C, fp16/bf16
// operands, fp32 accumulation on the matrix cores.
//
// The block tile, the copy partition of a tile over threads, the LDS tile
// layout (row-major chunks composed with an XOR swizzle) and the MFMA
// fragments are the compile-time layouts of device_layout.hpp; global
// operands are addressed through their runtime Shape:Stride strides. The
// structure follows the tiled GEMM of "Layouts as Algebra: CUTLASS & CuTe",
// "The kernel, in three lines" (block tile by local_tile, thread share by
// local_partition, a K-tile loop of copy / barrier / MMA) and "CUTLASS, in
// depth", "The problem CUTLASS solves" (tiles staged through on-chip memory),
// redesigned for CDNA4: 64-lane waves, 32x32x16 MFMA, direct global-to-LDS
// loads instead of cp.async/TMA, and a double-buffered LDS ring.

#include <hip/hip_runtime.h>

#include "device_layout.hpp"
#include "gemm_kernels.hpp"
#include "lt.h"

namespace lt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

#define LDS_AS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// dtype traits
// ---------------------------------------------------------------------------

template <int DT>
struct Tr;

template <>
struct Tr<LT_F16> {
    using V8 = f16x8;
    static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return static_cast<float>(__builtin_bit_cast(_Float16, x));
    }
    static __device__ __forceinline__ uint16_t from_f32(float x) {   // round to nearest even
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    }
};

template <>
struct Tr<LT_BF16> {
    using V8 = bf16x8;
    static __device__ __forceinline__ f32x16 mfma32(V8 a, V8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
    }
    static __device__ __forceinline__ uint16_t from_f32(float x) {   // round to nearest even
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    }
};

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return static_cast<uint32_t>(Tr<DT>::from_f32(a)) | (static_cast<uint32_t>(Tr<DT>::from_f32(b)) << 16);
}

// Epilogue of four consecutive N outputs of one row: alpha*acc + beta*c,
// rounded to the output format and stored as one 8-byte write.
template <int DT>
__device__ __forceinline__ void store4(uint16_t* D, const uint16_t* C, int64_t dof, int64_t cof, float a0,
                                       float a1, float a2, float a3, float alpha, float beta) {
    float v0 = alpha * a0, v1 = alpha * a1, v2 = alpha * a2, v3 = alpha * a3;
    if (beta != 0.0f) {
        u32x2 c = *reinterpret_cast<const u32x2*>(C + cof);
        v0 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.x & 0xffff));
        v1 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.x >> 16));
        v2 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.y & 0xffff));
        v3 += beta * Tr<DT>::to_f32(static_cast<uint16_t>(c.y >> 16));
    }
    u32x2 o;
    o.x = pack2<DT>(v0, v1);
    o.y = pack2<DT>(v2, v3);
    *reinterpret_cast<u32x2*>(D + dof) = o;
}

// ---------------------------------------------------------------------------
// WAVE16: one wave per 16x16 output tile, any operand strides, ragged edges.
// The tile grid is mode 1 of zipped_divide(D, (16,16)) ("CUTLASS and CuTe
// layouts", "A layout is a shape and a stride"): tile index t unravels
// colexicographically to (tm, tn). Fragments come straight from global memory
// through each operand's layout; out-of-range elements read as zero.
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ typename Tr<DT>::V8 load_frag8(const uint16_t* P, int row, int k, int64_t s_row,
                                                           int64_t s_k, int nrows, int K) {
    typename Tr<DT>::V8 v;
    if (row < nrows && s_k == 1 && k + 8 <= K) {
        u32x4 raw = *reinterpret_cast<const u32x4*>(P + row * s_row + k);
        return __builtin_bit_cast(typename Tr<DT>::V8, raw);
    }
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (row < nrows && k + i < K) ? P[row * s_row + (int64_t)(k + i) * s_k] : 0;
    u32x4 raw;
    raw.x = e[0] | (uint32_t(e[1]) << 16);
    raw.y = e[2] | (uint32_t(e[3]) << 16);
    raw.z = e[4] | (uint32_t(e[5]) << 16);
    raw.w = e[6] | (uint32_t(e[7]) << 16);
    v = __builtin_bit_cast(typename Tr<DT>::V8, raw);
    return v;
}

template <int DT>
__global__ __launch_bounds__(256) void gemm_wave16(Wave16Args p) {
    const int lane = threadIdx.x & 63;
    const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= p.tiles_m * p.tiles_n) return;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int m0 = tm * 16, n0 = tn * 16;
    // 16x16x32 MFMA operand fragment: lane -> (row = lane % 16, kchunk = lane / 16)
    const int r = lane & 15, h = lane >> 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.K; k0 += 32) {
        const int k = k0 + 8 * h;
        auto a = load_frag8<DT>(p.A, m0 + r, k, p.sam, p.sak, p.M, p.K);
        auto b = load_frag8<DT>(p.B, n0 + r, k, p.sbn, p.sbk, p.N, p.K);
        // operand roles swapped (B as the row operand) so each lane ends with
        // four consecutive N outputs of one M row
        acc = Tr<DT>::mfma16(b, a, acc);
    }
    const int m = m0 + r;
    const int n = n0 + 4 * h;
    if (m >= p.M) return;
    if (p.sdn == 1 && (p.beta == 0.0f || p.scn == 1) && n + 4 <= p.N) {
        store4<DT>(p.D, p.C, m * p.sdm + n, m * p.scm + n, acc[0], acc[1], acc[2], acc[3], p.alpha, p.beta);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (n + i >= p.N) break;
        float v = p.alpha * acc[i];
        if (p.beta != 0.0f) v += p.beta * Tr<DT>::to_f32(p.C[m * p.scm + (int64_t)(n + i) * p.scn]);
        p.D[m * p.sdm + (int64_t)(n + i) * p.sdn] = Tr<DT>::from_f32(v);
    }
}

// ---------------------------------------------------------------------------
// TILED: 256x256 block tile, K step 64, four waves of 128x128, LDS double
// buffer filled by direct global-to-LDS 16-byte loads.
// ---------------------------------------------------------------------------

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kStageBytes = 2 * kBM * kBK * 2;     // A tile + B tile
constexpr int kOperandBytes = kBM * kBK * 2;       // 32 KiB

// Bijection from workgroup id to output tile: consecutive ids land on
// different XCDs (round-robin dispatch), so ids are first regrouped so that
// each XCD walks a contiguous range of the raster; the raster runs down
// group_m tile rows before moving one tile column right, so tiles in flight
// together share A rows and B columns in L2 ("CUTLASS, in depth", "Kernel
// schedules": rasterised, L2-friendly tile order).
__device__ __forceinline__ void tile_of(int wg, const TiledArgs& p, int* tm, int* tn) {
    const int ntiles = p.tiles_m * p.tiles_n;
    int lin = wg;
    if (p.xcd_remap) lin = (wg & 7) * (ntiles >> 3) + (wg >> 3);
    const int gsz = p.group_m * p.tiles_n;
    const int grp = lin / gsz;
    const int first = grp * p.group_m;
    const int gm = min(p.tiles_m - first, p.group_m);
    const int in = lin - grp * gsz;
    *tm = first + in % gm;
    *tn = in / gm;
}

template <int DT>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kk(TiledArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    using V8 = typename Tr<DT>::V8;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, p, &tm, &tn);
    const int m0 = tm * kBM, n0 = tn * kBN;

    // Copy partition (kCopyTV): wave w fills stored chunks [512w, 512w+512)
    // of each operand tile, 64 per instruction, lane -> stored chunk. The
    // stored chunk s = lane + 64 j + 512 w sits at row s/8 and swizzled column
    // s%8; the logical K chunk there is (s%8) ^ (row & 7).
    const int crow = lane >> 3;                                  // row within the 8-row block
    const int kchunk = (lane & 7) ^ (crow & 7);                  // logical chunk fetched
    const int row0 = wave * 64 + crow;
    const uint16_t* gA = p.A + (int64_t)(m0 + row0) * p.lda + kchunk * 8;
    const uint16_t* gB = p.B + (int64_t)(n0 + row0) * p.ldb + kchunk * 8;
    const int64_t a_step = 8 * p.lda, b_step = 8 * p.ldb;        // next instruction: 8 rows on

    auto issue = [&](int stage, int k0) {
        char* sa = smem + stage * kStageBytes + wave * 8192;
        char* sb = sa + kOperandBytes;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __builtin_amdgcn_global_load_lds(gA + j * a_step + k0, (LDS_AS void*)(sa + j * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gB + j * b_step + k0, (LDS_AS void*)(sb + j * 1024), 16, 0, 0);
        }
    };

    // Fragment partition (kFragLane): lane reads row lane%32 of each 32-row
    // block and logical K chunk 2s + lane/32 for K step s, at its swizzled
    // position (row & 7 == lane & 7 for every block).
    const int wm = wave >> 1, wn = wave & 1;
    const int frow = lane & 31, fh = lane >> 5;
    int foff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) foff[s] = dev::tile_chunk(frow, 2 * s + fh) * 16;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int KT = p.K / kBK;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();

    for (int t = 0; t < KT; ++t) {
        const int cur = t & 1;
        if (t + 1 < KT) issue(cur ^ 1, (t + 1) * kBK);
        const char* sa = smem + cur * kStageBytes + wm * 128 * 128;
        const char* sb = smem + cur * kStageBytes + kOperandBytes + wn * 128 * 128;
        // Fragments of K step s+1 are read while the 16 MFMAs of step s run.
        V8 af[2][4], bf[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[0][i] = *(const LDS_AS V8*)(sa + i * 4096 + foff[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[0][j] = *(const LDS_AS V8*)(sb + j * 4096 + foff[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = s & 1;
            if (s + 1 < 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i) af[c ^ 1][i] = *(const LDS_AS V8*)(sa + i * 4096 + foff[s + 1]);
#pragma unroll
                for (int j = 0; j < 4; ++j) bf[c ^ 1][j] = *(const LDS_AS V8*)(sb + j * 4096 + foff[s + 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = Tr<DT>::mfma32(bf[c][j], af[c][i], acc[i][j]);
        }
        // Issue order for the scheduler: the next tile's copies first, the
        // first step's fragments, then each step's 16 MFMAs with the next
        // step's 8 fragment reads threaded between them.
        __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);   // global-to-LDS copies
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // fragments of step 0
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's loads of tile t+1 landed
        __syncthreads();                      // everyone's landed; everyone done reading stage cur
    }

    // Epilogue: block (i, j), register group g holds row m = lane%32 and
    // columns 8g + 4*(lane/32) + 0..3 of the 32x32 block.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 128 + i * 32 + frow;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * 128 + j * 32 + 8 * g + 4 * fh;
                store4<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, acc[i][j][4 * g],
                           acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3], p.alpha, p.beta);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// SKINNY: M <= 32. B (K-major) is streamed once from HBM straight into MFMA
// fragments; each workgroup owns 32 columns of N and splits its K range over
// eight waves; partial sums meet in LDS. With split_k > 1 the K range is
// further split over workgroups and fp32 partials go to a workspace that a
// second kernel reduces ("CUTLASS, in depth", "Worked example: tile choice
// and wave quantisation": narrow N tile and split-K for decode-like shapes).
//
// K order inside a 64-wide K block: lane half h holds K values
// 32h + 8s .. 32h + 8s + 7 for MFMA step s, the same for the A and the B
// fragment, so each lane streams 64 contiguous bytes of its B column.
// ---------------------------------------------------------------------------

constexpr int kSkU = 4;   // K blocks of 64 in flight per batch

template <int DT>
__global__ __launch_bounds__(512, 1) void gemm_skinny(SkinnyArgs p) {
    __shared__ float red[kSkinnyWaves - 1][16][64];
    using V8 = typename Tr<DT>::V8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = blockIdx.x, sk = blockIdx.y;
    const int n0 = nb * kSkinnyBN;
    const int frow = lane & 31, fh = lane >> 5;
    const int kbeg = (sk * kSkinnyWaves + wave) * p.k_per_wave;
    const uint16_t* gB = p.B + (int64_t)(n0 + frow) * p.ldb + kbeg + 32 * fh;
    const bool arow = frow < p.M;
    const uint16_t* gA = p.A + (int64_t)(arow ? frow : 0) * p.lda + kbeg + 32 * fh;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

    const int nkb = p.k_per_wave / 64;
    int kb = 0;
    for (; kb + kSkU <= nkb; kb += kSkU) {
        u32x4 bv[kSkU][4], av[kSkU][4];
#pragma unroll
        for (int u = 0; u < kSkU; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                bv[u][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(gB + (kb + u) * 64 + 8 * s));
#pragma unroll
        for (int u = 0; u < kSkU; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                av[u][s] = arow ? *reinterpret_cast<const u32x4*>(gA + (kb + u) * 64 + 8 * s) : zero;
#pragma unroll
        for (int u = 0; u < kSkU; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = Tr<DT>::mfma32(__builtin_bit_cast(V8, bv[u][s]), __builtin_bit_cast(V8, av[u][s]), acc);
    }
    for (; kb < nkb; ++kb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 b = *reinterpret_cast<const u32x4*>(gB + kb * 64 + 8 * s);
            u32x4 a = arow ? *reinterpret_cast<const u32x4*>(gA + kb * 64 + 8 * s) : zero;
            acc = Tr<DT>::mfma32(__builtin_bit_cast(V8, b), __builtin_bit_cast(V8, a), acc);
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[v];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kSkinnyWaves - 1; ++w)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] += red[w][v][lane];

    // lane holds m = lane % 32 and n = n0 + 8g + 4*(lane/32) + 0..3
    const int m = frow;
    if (m >= p.M) return;
    if (p.split_k == 1) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = n0 + 8 * g + 4 * fh;
            store4<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, acc[4 * g], acc[4 * g + 1],
                       acc[4 * g + 2], acc[4 * g + 3], p.alpha, p.beta);
        }
    } else {
        float* w = p.ws + ((int64_t)sk * 32 + m) * p.N;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n = n0 + 8 * g + 4 * fh;
            *reinterpret_cast<f32x4*>(w + n) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        }
    }
}

// Sum of the split_k fp32 partials, then the epilogue: one thread per four
// consecutive outputs of a row.
template <int DT>
__global__ __launch_bounds__(256) void skinny_reduce(SkinnyArgs p) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // quad index
    const int64_t quads_per_row = p.N / 4;
    if (q >= (int64_t)p.M * quads_per_row) return;
    const int m = (int)(q / quads_per_row);
    const int n = (int)(q % quads_per_row) * 4;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < p.split_k; ++k) s += *reinterpret_cast<const f32x4*>(p.ws + ((int64_t)k * 32 + m) * p.N + n);
    store4<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, s[0], s[1], s[2], s[3], p.alpha, p.beta);
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int launch_wave16(int dtype, const Wave16Args& a, void* stream) {
    const int tiles = a.tiles_m * a.tiles_n;
    dim3 grid((tiles + 3) / 4), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == LT_F16)
        hipLaunchKernelGGL(gemm_wave16<LT_F16>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(gemm_wave16<LT_BF16>, grid, block, 0, s, a);
    return static_cast<int>(hipGetLastError());
}

int launch_tiled(int dtype, bool a_kmajor, bool b_kmajor, const TiledArgs& a, void* stream) {
    if (!a_kmajor || !b_kmajor) return static_cast<int>(hipErrorInvalidValue);
    static bool attr_set[2] = {false, false};
    auto kf16 = gemm_tiled_kk<LT_F16>;
    auto kbf16 = gemm_tiled_kk<LT_BF16>;
    const int which = dtype == LT_F16 ? 0 : 1;
    if (!attr_set[which]) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(which == 0 ? kf16 : kbf16),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kTiledLdsBytes);
        if (e != hipSuccess) return static_cast<int>(e);
        attr_set[which] = true;
    }
    dim3 grid(a.tiles_m * a.tiles_n), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (which == 0)
        hipLaunchKernelGGL(kf16, grid, block, kTiledLdsBytes, s, a);
    else
        hipLaunchKernelGGL(kbf16, grid, block, kTiledLdsBytes, s, a);
    return static_cast<int>(hipGetLastError());
}

int launch_skinny(int dtype, const SkinnyArgs& a, void* stream) {
    dim3 grid(a.N / kSkinnyBN, a.split_k), block(64 * kSkinnyWaves);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == LT_F16)
        hipLaunchKernelGGL(gemm_skinny<LT_F16>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(gemm_skinny<LT_BF16>, grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.split_k == 1) return static_cast<int>(e);
    const int64_t quads = (int64_t)a.M * (a.N / 4);
    dim3 rgrid((unsigned)((quads + 255) / 256)), rblock(256);
    if (dtype == LT_F16)
        hipLaunchKernelGGL(skinny_reduce<LT_F16>, rgrid, rblock, 0, s, a);
    else
        hipLaunchKernelGGL(skinny_reduce<LT_BF16>, rgrid, rblock, 0, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace lt
