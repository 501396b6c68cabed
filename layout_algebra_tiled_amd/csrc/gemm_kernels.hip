// GEMM kernels for gfx950 (CDNA4) other than the block-tiled one
// (gemm_tiled.hip): the wave-per-16x16-tile kernel for any layout and ragged
// shapes, and the skinny (M <= 32) kernel. D = alpha * A*B + beta * C,
// fp16/bf16 operands, fp32 accumulation on the matrix cores; global operands
// are addressed through their runtime Shape:Stride strides.

#include <hip/hip_runtime.h>

#include "device_layout.hpp"
#include "gemm_kernels.hpp"
#include "kernel_common.hpp"
#include "tiled_config.hpp"

namespace lt {
namespace {

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
    if (p.epi.fused) {
        float amax = 0.0f;
        if (m < p.M) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (n + i >= p.N) break;
                const float v = fused_value<DT>(acc[i], p.alpha, p.beta, p.C, m * p.scm + (int64_t)(n + i) * p.scn,
                                                p.epi, m, n + i);
                const uint16_t o = Tr<DT>::from_f32(v);
                p.D[m * p.sdm + (int64_t)(n + i) * p.sdn] = o;
                amax = fmaxf(amax, fabsf(Tr<DT>::to_f32(o)));
            }
        }
        if (p.epi.amax) amax_commit(p.epi.amax, amax);   // every lane of the wave takes part
        return;
    }
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
// SKINNY: M <= 32, K-major A and B. The job is to stream B (K x N) from HBM
// exactly once at full bandwidth ("CUTLASS, in depth", "Worked example: tile
// choice and wave quantisation": narrow N tile plus split-K for decode-like
// shapes, or treat the product as memory-bound). Each workgroup owns 32
// columns of N; its four waves split the workgroup's K range. Every wave owns
// a private ring of kSkinnyStages LDS slots; a slot holds a 64-deep K slice of
// the 32 A rows and of the 32 B columns (4 KiB each), filled by direct
// global-to-LDS loads in which 8 lanes cover one row's 128 contiguous bytes,
// so every load instruction reads 8 whole cache lines. One explicit vmcnt
// wait per slot and no barriers; the four waves' partial sums meet in LDS at
// the end. With split_k > 1 the K range is split over workgroups too and fp32
// partials go to a workspace that skinny_reduce sums.
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(64 * kSkinnyWaves, 1) void gemm_skinny(SkinnyArgs p) {
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    using V8 = typename Tr<DT>::V8;
    constexpr int R = kSkinnyStages;
    constexpr int HALF = 32 * 64 * 2;                 // 32 rows x 64 K x 16 bit
    constexpr int SLOT = 2 * HALF;                    // A rows, then B columns
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * kSkinnyBN, sk = blockIdx.y;
    const int kbeg = (sk * kSkinnyWaves + wave) * p.k_per_wave;
    const int nst = p.k_per_wave / 64;                // slots to stream
    char* ring = smem + wave * R * SLOT;

    // Copy: instruction j fills rows 8j .. 8j+7 of each half-slot, 8 lanes
    // per row; both halves use the K-major tile layout (128-byte rows of 8
    // chunks, chunk ^ ((row >> 1) & 7)), so each lane fetches the logical
    // chunk stored at its position. Rows of A past M repeat row M-1 (their
    // outputs are never stored).
    const uint16_t* ga[4];
    const uint16_t* gb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int lchunk = dev::KTile<64>::at(row, lane & 7) - 8 * row;
        ga[j] = p.A + (int64_t)min(row, p.M - 1) * p.lda + kbeg + 8 * lchunk;
        gb[j] = p.B + (int64_t)(n0 + row) * p.ldb + kbeg + 8 * lchunk;
    }
    // Fragment offsets inside a half-slot: row lane%32, K chunk 2s + lane/32
    const int frow = lane & 31, fh = lane >> 5;
    int foff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) foff[s] = 16 * dev::KTile<64>::at(frow, 2 * s + fh);

    // Each wave starts its walk over its K range at a slot picked by a small
    // hash of (workgroup, wave) and wraps around. B's columns are 2^k bytes
    // apart for power-of-two K, so without the rotation every wave of the GPU
    // streams addresses with the same low bits at the same time and piles
    // onto a few DRAM channels (measured: 36.6 us unrotated vs 31.0 us on the
    // 32x8192x8192 workload). The K sum is order-free.
    const int rot = (blockIdx.x * 13 + wave * 7 + (blockIdx.x >> 3)) % nst;
    auto issue = [&](int slot, int st) {
        char* dst = ring + slot * SLOT;
        int sr = st + rot;
        sr = sr >= nst ? sr - nst : sr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const void* a = ga[j] + sr * 64;
            const void* b = gb[j] + sr * 64;
            __builtin_amdgcn_global_load_lds(a, (LDS_AS void*)(dst + j * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(b, (LDS_AS void*)(dst + HALF + j * 1024), 16, 0, 0);
        }
    };

    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

    for (int r = 0; r < R - 1 && r < nst; ++r) issue(r, r);
    int slot = 0;
    for (int t = 0; t < nst; ++t) {
        if (t + R - 1 < nst) {
            issue(slot == 0 ? R - 1 : slot - 1, t + R - 1);
            // slot t landed: 8 loads per slot, R-1 newer slots may fly
            __builtin_amdgcn_s_waitcnt(((8 * (R - 1)) & 15) | (0x7 << 4) | (0xf << 8) | (((8 * (R - 1)) >> 4) << 14));
        } else {
            __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
        }
        const char* sl = ring + slot * SLOT;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            V8 a = *(const LDS_AS V8*)(sl + foff[s]);
            V8 b = *(const LDS_AS V8*)(sl + HALF + foff[s]);
            // B as the row operand: each lane ends with four consecutive N
            acc = Tr<DT>::mfma32(b, a, acc);
        }
        slot = slot + 1 == R ? 0 : slot + 1;
    }

    // Partial sums of the four waves meet in LDS (each wave's own ring).
    __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
    float* red = reinterpret_cast<float*>(ring);
    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) red[v * 64 + lane] = acc[v];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) {
        const float* o = reinterpret_cast<const float*>(smem + w * R * SLOT);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] += o[v * 64 + lane];
    }

    // lane holds m = lane % 32 and n = n0 + 8g + 4*(lane/32) + 0..3
    const int m = frow;
    if (p.split_k == 1 && p.epi.fused) {
        float amax = 0.0f;
        if (m < p.M) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 8 * g + 4 * fh;
                const float v[4] = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
                store4_fused<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, v, 4, p.alpha, p.beta,
                                 p.epi, m, n, &amax);
            }
        }
        if (p.epi.amax) amax_commit(p.epi.amax, amax);
        return;
    }
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
    const bool in = q < (int64_t)p.M * quads_per_row;
    if (!in && !(p.epi.fused && p.epi.amax)) return;
    const int m = in ? (int)(q / quads_per_row) : 0;
    const int n = in ? (int)(q % quads_per_row) * 4 : 0;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if (in)
        for (int k = 0; k < p.split_k; ++k)
            s += *reinterpret_cast<const f32x4*>(p.ws + ((int64_t)k * 32 + m) * p.N + n);
    if (p.epi.fused) {
        float amax = 0.0f;
        const float v[4] = {s[0], s[1], s[2], s[3]};
        if (in)
            store4_fused<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, v, 4, p.alpha, p.beta, p.epi,
                             m, n, &amax);
        if (p.epi.amax) amax_commit(p.epi.amax, amax);   // every lane of the wave takes part
        return;
    }
    store4<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, s[0], s[1], s[2], s[3], p.alpha, p.beta);
}

__global__ void zero_f32(float* p) { *p = 0.0f; }

__global__ void zero_i32(int* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
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

int launch_zero_f32(float* p, void* stream) {
    hipLaunchKernelGGL(zero_f32, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), p);
    return static_cast<int>(hipGetLastError());
}

int launch_zero_i32(int* p, int n, void* stream) {
    hipLaunchKernelGGL(zero_i32, dim3((n + 255) / 256 < 64 ? (n + 255) / 256 : 64), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p, n);
    return static_cast<int>(hipGetLastError());
}

template <class Cf>
TiledShape shape_of() {
    return TiledShape{Cf::BM, Cf::BN, Cf::BK, Cf::TWM, Cf::TWN, Cf::NW, Cf::S, Cf::LDS, Cf::FM * Cf::FN * Cf::KS,
                      Cf::MF, Cf::MFMA::KSTEP};
}

template <bool AK, bool BKM>
TiledShape shape_for(int tile_n) {
    return tile_n == 128 ? shape_of<Dp128<AK, BKM>>() : shape_of<Dp256<AK, BKM>>();
}

TiledShape tiled_shape(bool a_kmajor, bool b_kmajor, int tile_n) {
    if (a_kmajor && b_kmajor) return shape_for<true, true>(tile_n);
    if (a_kmajor) return shape_for<true, false>(tile_n);
    if (b_kmajor) return shape_for<false, true>(tile_n);
    return shape_for<false, false>(tile_n);
}

int launch_tiled(int dtype, bool a_kmajor, bool b_kmajor, int tile_n, const TiledArgs& a, void* stream) {
    static_assert(LT_F16 == 1 && LT_BF16 == 2, "variant names carry the dtype code");
    if (dtype == LT_F16) {
        if (a_kmajor) return b_kmajor ? launch_tiled_11_1(a, tile_n, stream) : launch_tiled_11_0(a, tile_n, stream);
        return b_kmajor ? launch_tiled_10_1(a, tile_n, stream) : launch_tiled_10_0(a, tile_n, stream);
    }
    if (a_kmajor) return b_kmajor ? launch_tiled_21_1(a, tile_n, stream) : launch_tiled_21_0(a, tile_n, stream);
    return b_kmajor ? launch_tiled_20_1(a, tile_n, stream) : launch_tiled_20_0(a, tile_n, stream);
}

int launch_skinny(int dtype, const SkinnyArgs& a, void* stream) {
    dim3 grid(a.N / kSkinnyBN, a.split_k), block(64 * kSkinnyWaves);
    hipStream_t s = static_cast<hipStream_t>(stream);
    static std::atomic<uint64_t> attr[2];
    const int which = dtype == LT_F16 ? 0 : 1;
    const void* k = which == 0 ? reinterpret_cast<const void*>(&gemm_skinny<LT_F16>)
                               : reinterpret_cast<const void*>(&gemm_skinny<LT_BF16>);
    if (const int e = set_lds_limit_once(k, kSkinnyLdsBytes, attr[which])) return e;
    if (dtype == LT_F16)
        hipLaunchKernelGGL(gemm_skinny<LT_F16>, grid, block, kSkinnyLdsBytes, s, a);
    else
        hipLaunchKernelGGL(gemm_skinny<LT_BF16>, grid, block, kSkinnyLdsBytes, s, a);
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
