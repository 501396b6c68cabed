// GEMM kernels for gfx950 (CDNA4) other than the block-tiled one
// (gemm_tiled.hip): the wave-per-16x16-tile kernel for any layout and ragged
// shapes, and the skinny (M <= 32) kernel. D = alpha * A*B + beta * C,
// fp16/bf16 operands, fp32 accumulation on the matrix cores; global operands
// are addressed through their runtime Shape:Stride strides.

#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"
#include "kernel_common.hpp"

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
