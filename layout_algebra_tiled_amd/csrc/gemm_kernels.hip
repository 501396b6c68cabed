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
// columns of N and its two waves 16 of them each, with all 32 rows of A (two
// 16x16x32 MFMAs per 32 of K share the wave's B fragment), so A, read by
// every workgroup and served by L2, crosses to a CU once per 32 columns. The
// pair streams its K range through a ring of SkinnyCfg::R slots in LDS, each
// SkinnyCfg::SK (256) deep of the 32 A rows and 32 B columns, filled by
// direct global-to-LDS copies in which 32 lanes cover the 512 contiguous
// bytes of one row or column (the longer the run per column, the closer the
// stream gets to the HBM peak: 32 columns 16 KiB apart are open at once per
// workgroup; 256-byte runs measured 25.4 us, 512-byte runs 23.9 us on the
// 32x8192x8192 workload). Each
// wave copies its own 16 columns and 16 of the A rows; per slot it waits for
// its own copies, then a workgroup barrier makes the partner's visible and
// frees the slot read before. With split_k > 1 the K range is split over
// workgroups and fp32 partials go to a workspace that skinny_reduce sums.
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(64 * kSkinnyWaves, 1) void gemm_skinny(SkinnyArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)   // generic lambdas around the LDS-copy builtin: device pass only
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    using V8 = typename Tr<DT>::V8;
    using SC = SkinnyCfg;
    constexpr int R = SC::R, SK = SC::SK, CB = SC::CB, HALF = SC::HALF, SLOT = SC::SLOT, NW = SC::NW;
    constexpr int LPC = CB / 16;                      // lanes per row in a copy (32)
    constexpr int CPI = 64 / LPC;                     // rows per copy instruction (2)
    constexpr int NH = NW / 2;                        // copies per wave per half slot (8)
    static_assert(LPC >= 16 && NH * CPI == 16 && kSkinnyWaves == 2, "a wave copies 16 rows of each half");
    const int lane = threadIdx.x & 63;
    const int ch = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // column half
    const int n0 = blockIdx.x * kSkinnyBN, sk = blockIdx.y;
    const int kbeg = sk * p.k_per_wg;
    const int nst = p.k_per_wg / SK;                  // slots to stream
    char* ring = smem;

    // Both halves of a slot (A rows, then B columns) hold 32 rows of CB bytes
    // in 16-byte chunks; chunk q of row c is stored at position q ^ (c & 15),
    // so the 16 lanes of a fragment read that share q and take consecutive c
    // land on 16 distinct 16-byte bank groups.
    // Copy j of a half, lane L fills byte (NH ch + j)*1024 + 16L: row c =
    // 16 ch + CPI j + L/LPC, stored position L%LPC, i.e. logical chunk
    // (L%LPC) ^ (c & 15). Every address is a workgroup-uniform base plus a
    // 32-bit per-lane byte offset (32 rows of A or columns of B span far less
    // than 4 GiB). Rows of A past M repeat row M-1 (their outputs are never
    // stored).
    const int cl = lane / LPC, cs = lane % LPC;
    uint32_t aoff[NH], boff[NH];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
        const int c = 16 * ch + j * CPI + cl;
        aoff[j] = 2u * (uint32_t)(min(c, p.M - 1) * p.lda + 8 * (cs ^ (c & 15)));
        boff[j] = 2u * (uint32_t)(c * p.ldb + 8 * (cs ^ (c & 15)));
    }
    // 16x16x32 MFMA step s of a slot covers K 32s .. 32s+31: lane (r, g)
    // holds 8 of them, K 32s + 8g .. +7, of B column 16 ch + r (the row
    // operand) and of A row 16 mb + r for the two 16-row blocks mb of A.
    const int fr = lane & 15, fg = lane >> 4;
    int afo[SC::KSTEPS], bfo[SC::KSTEPS];
#pragma unroll
    for (int s = 0; s < SC::KSTEPS; ++s) {
        const int q = 4 * s + fg;
        afo[s] = fr * CB + 16 * (q ^ fr);                                      // row fr (+16 for mb = 1)
        bfo[s] = HALF + (16 * ch + fr) * CB + 16 * (q ^ ((16 * ch + fr) & 15));
    }

    // Each workgroup starts its walk over its K range at a slot picked by a
    // small hash of its index and wraps around. B's columns are 2^k bytes
    // apart for power-of-two K, so without the rotation every workgroup of
    // the GPU streams addresses with the same low bits at the same time and
    // piles onto a few DRAM channels. The hash matters: streaming this
    // kernel's B pattern alone (32 columns of 16 KiB per workgroup, 256
    // workgroups) takes 32.3 us with no rotation, 30.3 us with start slot
    // g % 64, 24.4 us with (13 g + g/8) % 64 and 23.0 us with the
    // (41 g + 7 (g/32)) % 64 used here. The K sum is order-free.
    const int rot = (blockIdx.x * 41 + (blockIdx.x >> 5) * 7) % nst;
    auto issue = [&](auto slot_c, int st) {
        constexpr int slot = decltype(slot_c)::value;
        char* dst = ring + slot * SLOT + ch * NH * 1024;
        int sr = st + rot;
        sr = sr >= nst ? sr - nst : sr;
        const int64_t k = kbeg + sr * SK;
        const char* ab = reinterpret_cast<const char*>(p.A + k);
        const char* bb = reinterpret_cast<const char*>(p.B + (int64_t)n0 * p.ldb + k);
#pragma unroll
        for (int j = 0; j < NH; ++j)
            __builtin_amdgcn_global_load_lds(ab + aoff[j], (LDS_AS void*)(dst + j * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < NH; ++j)
            __builtin_amdgcn_global_load_lds(bb + boff[j], (LDS_AS void*)(dst + HALF + j * 1024), 16, 0, 0);
    };
    f32x4 acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        const char* sl = ring + slot * SLOT;
        V8 a0[SC::KSTEPS], a1[SC::KSTEPS], b[SC::KSTEPS];
#pragma unroll
        for (int s = 0; s < SC::KSTEPS; ++s) {
            b[s] = *(const LDS_AS V8*)(sl + bfo[s]);
            a0[s] = *(const LDS_AS V8*)(sl + afo[s]);
            a1[s] = *(const LDS_AS V8*)(sl + afo[s] + 16 * CB);
        }
        // B as the row operand: each lane ends with four consecutive N
#pragma unroll
        for (int s = 0; s < SC::KSTEPS; ++s) {
            acc[0] = Tr<DT>::mfma16(b[s], a0[s], acc[0]);
            acc[1] = Tr<DT>::mfma16(b[s], a1[s], acc[1]);
        }
    };

    // Iteration t: wait for this wave's copies of slot t, barrier (the
    // partner's copies of slot t are in; both waves are done with slot t-1),
    // refill slot t-1's ring slot with slot t+R-1, compute slot t. R - 1
    // slots are in flight while slot t computes.
    // Steady state: every slot of a trip issues unconditionally.
    int t0 = 0;
    if (nst >= 2 * R - 1) {
        static_for<0, R - 1>([&](auto r) { issue(r, r.value); });
        for (; t0 + 2 * R - 1 <= nst; t0 += R) {
            static_for<0, R>([&](auto r) {
                LT_WAIT_VM(NW * (R - 2));
                __builtin_amdgcn_s_barrier();
                issue(ic<(r.value + R - 1) % R>{}, t0 + r.value + R - 1);
                compute(r);
            });
        }
    } else {
        static_for<0, R - 1>([&](auto r) {
            if (r.value < nst) issue(r, r.value);
        });
    }
    // The last slots (fewer than 2R - 1): the same steps; once nothing is
    // left to issue, each slot waits only for itself (min(R - 2, nst-1-t)
    // newer slots may still fly), so the last slots' MFMAs overlap the
    // arrival of the ones after them. nst and t0 are the same for both
    // waves, so both meet every barrier.
    static_for<0, 2 * R - 2>([&](auto i) {
        const int t = t0 + i.value;
        if (t < nst) {
            const int newer = min(R - 2, nst - 1 - t);
            static_for<0, R - 1>([&](auto c) {
                if (newer == c.value) LT_WAIT_VM(NW * c.value);
            });
            __builtin_amdgcn_s_barrier();
            if (t + R - 1 < nst) issue(ic<(i.value + R - 1) % R>{}, t + R - 1);
            compute(ic<i.value % R>{});
        }
    });

    // lane holds m = 16 mb + lane % 16 and n = n0 + 16 ch + 4 (lane / 16) + 0..3
    const int n = n0 + 16 * ch + 4 * fg;
    if (p.split_k == 1 && p.epi.fused) {
        float amax = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int m = 16 * mb + fr;
            if (m < p.M) {
                const float v[4] = {acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]};
                store4_fused<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, v, 4, p.alpha, p.beta,
                                 p.epi, m, n, &amax);
            }
        }
        if (p.epi.amax) amax_commit(p.epi.amax, amax);
        return;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = 16 * mb + fr;
        if (m >= p.M) continue;
        if (p.split_k == 1) {
            store4<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, acc[mb][0], acc[mb][1],
                       acc[mb][2], acc[mb][3], p.alpha, p.beta);
        } else {
            float* w = p.ws + ((int64_t)sk * 32 + m) * p.N;
            *reinterpret_cast<f32x4*>(w + n) = acc[mb];
        }
    }
#endif
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
TiledShape shape_for(int tile_m, int tile_n) {
    if (tile_m == 128) return shape_of<Dp128x128<AK, BKM>>();
    return tile_n == 128 ? shape_of<Dp128<AK, BKM>>() : shape_of<Dp256<AK, BKM>>();
}

TiledShape tiled_shape(bool a_kmajor, bool b_kmajor, int tile_m, int tile_n) {
    if (a_kmajor && b_kmajor) return shape_for<true, true>(tile_m, tile_n);
    if (a_kmajor) return shape_for<true, false>(tile_m, tile_n);
    if (b_kmajor) return shape_for<false, true>(tile_m, tile_n);
    return shape_for<false, false>(tile_m, tile_n);
}

int launch_tiled(int dtype, bool a_kmajor, bool b_kmajor, int tile_m, int tile_n, int persist_grid,
                 const TiledArgs& a, void* stream) {
    static_assert(LT_F16 == 1 && LT_BF16 == 2, "variant names carry the dtype code");
    const int pg = persist_grid, tm = tile_m, tn = tile_n;
    if (dtype == LT_F16) {
        if (a_kmajor) return b_kmajor ? launch_tiled_11_1(a, tm, tn, pg, stream) : launch_tiled_11_0(a, tm, tn, pg, stream);
        return b_kmajor ? launch_tiled_10_1(a, tm, tn, pg, stream) : launch_tiled_10_0(a, tm, tn, pg, stream);
    }
    if (a_kmajor) return b_kmajor ? launch_tiled_21_1(a, tm, tn, pg, stream) : launch_tiled_21_0(a, tm, tn, pg, stream);
    return b_kmajor ? launch_tiled_20_1(a, tm, tn, pg, stream) : launch_tiled_20_0(a, tm, tn, pg, stream);
}

template <int DT>
int launch_skinny_dt(const SkinnyArgs& a, hipStream_t s) {
    static std::atomic<uint64_t> attr;
    dim3 grid(a.N / kSkinnyBN, a.split_k), block(64 * kSkinnyWaves);
    constexpr int lds = SkinnyCfg::LDS;
    if (const int e = set_lds_limit_once(reinterpret_cast<const void*>(&gemm_skinny<DT>), lds, attr)) return e;
    hipLaunchKernelGGL(gemm_skinny<DT>, grid, block, lds, s, a);
    return 0;
}

int launch_skinny(int dtype, const SkinnyArgs& a, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int le = dtype == LT_F16 ? launch_skinny_dt<LT_F16>(a, s) : launch_skinny_dt<LT_BF16>(a, s);
    if (le) return le;
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
