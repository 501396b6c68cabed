// Block-tiled GEMM for gfx950: D = alpha * A*B + beta * C with a 256x256,
// 256x128 or 128x128 block tile, fp16/bf16 operands, fp32 accumulation in
// 16x16x32 MFMAs. M, N and K need not be multiples of the tile: edge tiles clamp their
// copy rows and store only the outputs inside (M, N); a partial K slice is
// zero-filled in LDS.
//
// Structure (the tiled GEMM of "Layouts as Algebra: CUTLASS & CuTe", "The
// kernel, in three lines", redesigned for CDNA4):
//   - local_tile: workgroup -> one block tile of D (XCD-aware raster order);
//   - the K loop streams BK-deep slices of the A and B tiles through an
//     S-stage LDS ring filled by direct global-to-LDS 16-byte loads
//     (global_load_lds_dwordx4; the copy's thread-value layout puts lane l's
//     16 bytes at stored chunk l, and the lane fetches the logical chunk the
//     swizzle stores there; the maps are in tiled_config.hpp);
//   - local_partition: each wave owns a TWM x TWN sub-tile and reads its MFMA
//     fragments from LDS one K step ahead of the MFMAs that use them
//     (ds_read_b128 for K-major operands, the transposing ds_read_b64_tr_b16
//     for M- or N-major operands);
//   - epilogue alpha*acc + beta*C, rounded once, 8-byte stores.
// One workgroup barrier per K slice: it publishes slice t+1 and frees slice
// t's stage, into which slice t+S is loaded at once.
//
// This file is compiled once per (dtype, A major-ness, B major-ness), chosen
// by LT_TILED_DT / LT_TILED_AK / LT_TILED_BK, each object holding that
// variant's kernels; the dispatch is in gemm_kernels.hip.

#include <type_traits>

#include "gemm_kernels.hpp"
#include "kernel_common.hpp"
#include "tiled_config.hpp"

namespace lt {
namespace {

// Linear tile index -> tile coordinates: raster down group_m tile rows
// before moving right, so tiles in flight together on one XCD share A rows
// and B columns in its L2 ("CUTLASS, in depth", "Kernel schedules":
// L2-friendly tile order).
__device__ __forceinline__ void tile_coords(int lin, const TiledArgs& p, int* tm, int* tn) {
    const int gsz = p.group_m * p.tiles_n;
    const int grp = lin / gsz;
    const int first = grp * p.group_m;
    const int gm = min(p.tiles_m - first, p.group_m);
    const int in = lin - grp * gsz;
    *tm = first + in % gm;
    *tn = in / gm;
}

// Launches of the tiled kernel: one workgroup per tile (the data-parallel
// launch), one per K segment of the split remainder's tiles, or one per
// compute unit walking a list of whole tiles (persistent; with C loaded for
// beta != 0, or without).
enum TiledMode : int { kDataParallel = 0, kSplit = 1, kPersistent = 2, kPersistentC = 3 };

// Workgroup -> (linear tile, K slices [kt0, kt1), split index or -1). In
// the data-parallel launch consecutive workgroup ids go to different XCDs
// (round-robin dispatch), so the ids are regrouped for each XCD to walk a
// contiguous stretch of the raster. In the split launch workgroup r takes K
// segment r % sk_splits of remainder tile r / sk_splits.
template <bool SPLIT>
__device__ __forceinline__ void work_of(int wg, const TiledArgs& p, int KT, int* lin, int* kt0, int* kt1,
                                        int* seg) {
    if constexpr (!SPLIT) {
        *lin = p.xcd_remap ? (wg & 7) * (p.dp_tiles >> 3) + (wg >> 3) : wg;
        *kt0 = 0;
        *kt1 = KT;
        *seg = -1;
        return;
    }
    const int r = wg, S = p.sk_splits;
    const int s = r % S;
    *lin = p.dp_tiles + r / S;
    *kt0 = s * KT / S;
    *kt1 = (s + 1) * KT / S;
    *seg = s;
}

// f(i, j) for every accumulator block, i < FM, j < FN, with i and j as
// compile-time constants: unrolled whatever the block count, so the
// accumulator array never needs a memory home.
template <int FM, int FN, class F>
__host__ __device__ __forceinline__ void for_blocks(F&& f) {
    static_for<0, FM * FN>([&](auto ij) { f(ic<decltype(ij)::value / FN>{}, ic<decltype(ij)::value % FN>{}); });
}

// Issue slots of the one-wave-per-SIMD schedule, over the NQ MFMAs of a K
// step: copy c of NC follows MFMA (2c+1)*NQ/(2*NC) (spread over the whole
// step), fragment read r of NR follows MFMA r*(3/4)*NQ/NR (spread over the
// first three quarters, so the last read has a quarter of the step to land).
// -1: nothing after MFMA q.
constexpr int copy_after(int q, int nc, int nq) {
    for (int c = 0; c < nc; ++c)
        if ((2 * c + 1) * nq / (2 * nc) == q) return c;
    return -1;
}
constexpr int read_after(int q, int nr, int nq) {
    for (int r = 0; r < nr; ++r)
        if (r * nq * 3 / 4 / nr == q) return r;
    return -1;
}

// One MFMA operand fragment (8 16-bit values per lane). From a K-major LDS
// tile it is one 16-byte read; from an M/N-major tile, two transposing
// 8-byte reads (ds_read_b64_tr_b16 through the compiler's builtin, so the
// compiler tracks them: it waits for each before its first use, and any copy
// of the registers it makes comes after that wait).
template <class V8, bool KMAJ>
struct Frag;
template <class V8>
struct Frag<V8, true> {
    V8 v;
    __device__ __forceinline__ V8 get() const { return v; }
};
template <class V8>
struct Frag<V8, false> {
    i16x4 lo, hi;
    __device__ __forceinline__ V8 get() const {
        return __builtin_bit_cast(V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// The two transposing reads of an M/N-major fragment: K rows 4q..4q+3 of
// the lane's group come from `p0` (q = 0) and four K rows further (q = 1).
template <class V8, int KROW_BYTES>
__device__ __forceinline__ Frag<V8, false> read_tr(const LDS_AS char* p0) {
    Frag<V8, false> f;
    LDS_AS char* p = const_cast<LDS_AS char*>(p0);   // (the builtin takes a non-const pointer; it only reads)
    f.lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
    f.hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p + 4 * KROW_BYTES));
    return f;
}

// Direct global-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l reads gbase + voff + IMM and writes LDS at lds + IMM + 16*l. gbase
// and lds are wave-uniform (SGPRs), voff a per-lane 32-bit byte offset, so
// no address arithmetic runs per copy. Inline asm: the compiler does not
// see these as writes to LDS, so it never waits for copies in flight before
// an LDS read of other bytes; the kernel orders copies and reads itself
// (vmcnt waits, then the workgroup barrier). M0 carries the LDS base and is
// written here before every copy; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is a reserved register; see above
template <int IMM>
__device__ __forceinline__ void copy16(uint32_t lds, const char* gbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3"
                 :
                 : "s"(lds), "v"(voff), "s"(gbase), "i"(IMM)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Which launches stage D through LDS, and how much LDS they hold: the rule
// in tiled_config.hpp, which the planner reports from.
template <class Cf, int MODE>
constexpr bool staged_d() {
    return Cf::EXPLICIT && staged_d_launch(MODE == kPersistent || MODE == kPersistentC, MODE == kDataParallel,
                                           Cf::AK, Cf::BKM);
}
template <class Cf, int MODE>
constexpr int staged_d_bytes() {
    return staged_d<Cf, MODE>() ? staged_d_region(Cf::LDS) : 0;
}

}  // namespace

// The kernel's body is compiled in the device pass only: the host pass needs
// just the launch stub (and with the body in view it silently emits no stub
// for a kernel whose generic lambdas call the direct-to-LDS builtin).
template <int DT, class Cf, int MODE>
__global__ __launch_bounds__(Cf::NT, 1) void gemm_tiled(TiledArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr bool SPLIT = MODE == kSplit;
    constexpr bool PERS = MODE == kPersistent || MODE == kPersistentC;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    using V8 = typename Tr<DT>::V8;
    constexpr int BK = Cf::BK, S = Cf::S, KS = Cf::KS, FM = Cf::FM, FN = Cf::FN;
    using OA = Operand<Cf, Cf::AK, Cf::BM>;
    using OB = Operand<Cf, Cf::BKM, Cf::BN>;
    using FA = Frag<V8, Cf::AK>;
    using FB = Frag<V8, Cf::BKM>;
    // (the wave index is uniform: read it into an SGPR so that LDS bases
    // derived from it are scalars)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // K slices: KT = ceil(K / BK). When BK does not divide K, the K range is
    // shifted to start at kbase = K - KT*BK < 0, so that only slice 0 is
    // partial: its first -kbase K positions are zero-filled in LDS, and every
    // later slice is a full, unpredicated copy.
    const int KT = (p.K + BK - 1) / BK;
    const int kbase = p.K - KT * BK;
    int lin, kt0, kt1, seg;
    // Persistent launch: this workgroup's tiles are first + j*step, j <
    // ntl. With the XCD regrouping, XCD x owns the stretch of dp_tiles/8
    // tiles from x*dp_tiles/8 and its workgroups take them in turn, so the
    // tiles in flight on one XCD are consecutive in the raster, as in the
    // data-parallel launch.
    int first = 0, step = 0, ntl = 1;
    if constexpr (PERS) {
        if (p.xcd_remap) {
            const int x = blockIdx.x & 7, l = blockIdx.x >> 3, wpx = gridDim.x >> 3, tpx = p.dp_tiles >> 3;
            first = x * tpx + l;
            step = wpx;
            ntl = (tpx - l + wpx - 1) / wpx;
        } else {
            first = blockIdx.x;
            step = gridDim.x;
            ntl = (p.dp_tiles - (int)blockIdx.x + step - 1) / step;
        }
        if (ntl <= 0) return;   // (the planner launches at most one workgroup per tile)
        lin = first;
        kt0 = 0;
        kt1 = KT;
        seg = -1;
    } else {
        work_of<SPLIT>(blockIdx.x, p, KT, &lin, &kt0, &kt1, &seg);
    }
    const int NS = kt1 - kt0;   // K slices this workgroup runs (>= 1)
    int tm, tn;
    tile_coords(lin, p, &tm, &tn);
    if constexpr (!PERS && !SPLIT) {
        // super-blocks (the planner sets this only for whole, unsplit tiles
        // in multiples of 16 each way): the j-th workgroup of XCD x takes
        // tile (8 (x mod 2) + j mod 8, 4 (x / 2) + (j mod 32) / 8) of 16x16
        // block j / 32, blocks in row order
        if (p.superblock) {
            const int x = blockIdx.x & 7, j = blockIdx.x >> 3, sb = j >> 5, r = j & 31, sbn = p.tiles_n >> 4;
            tm = 16 * (sb / sbn) + 8 * (x & 1) + (r & 7);
            tn = 16 * (sb % sbn) + 4 * (x >> 1) + (r >> 3);
        }
    }
    int m0 = tm * Cf::BM, n0 = tn * Cf::BN;   // (the persistent launch moves them tile by tile)

    // ---- copy: S-stage ring, stage s at s*STAGE (A slice, then B slice).
    // Up to four copy instructions of one operand write LDS through the same
    // base (M0) and reach their own 1 KiB through the instruction offset,
    // which the hardware adds to both the global and the LDS address; the
    // global source is a uniform slice base plus a per-lane 32-bit offset,
    // minus that same instruction offset.
    // (the persistent launch runs whole tiles only: its offsets are taken
    // from the tile's first row, which a scalar tile base adds)
    uint32_t aoffg[OA::OPI], boffg[OB::OPI];
#pragma unroll
    for (int i = 0; i < OA::OPI; ++i)
        aoffg[i] = PERS ? OA::offset(p.lda, 0, Cf::BM, wave, lane, i) : OA::offset(p.lda, m0, p.M, wave, lane, i);
#pragma unroll
    for (int i = 0; i < OB::OPI; ++i)
        boffg[i] = PERS ? OB::offset(p.ldb, 0, Cf::BN, wave, lane, i) : OB::offset(p.ldb, n0, p.N, wave, lane, i);
    const int64_t a_ks = OA::kslice_bytes(p.lda);
    const int64_t b_ks = OB::kslice_bytes(p.ldb);
    // slice 0 sources: the operands' bases moved by kbase (the host does
    // that, so the slice address stays a kernel argument plus a multiple of
    // the slice stride); lanes whose chunk lies below K = 0 never load
    // (the persistent launch: the current tile's first rows)
    const char* a_k0 = reinterpret_cast<const char*>(p.A0) + (PERS ? OA::tile_bytes(p.lda, m0) : 0);
    const char* b_k0 = reinterpret_cast<const char*>(p.B0) + (PERS ? OB::tile_bytes(p.ldb, n0) : 0);
    auto a_lds = [&](int stage) { return smem + stage * Cf::STAGE + wave * OA::OPI * 1024; };
    auto b_lds = [&](int stage) { return smem + stage * Cf::STAGE + Cf::A_BYTES + wave * OB::OPI * 1024; };
    auto lds_u32 = [](const char* p) {
        return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const LDS_AS char*)p));
    };

    // Copy instruction c (< IPW) of the slice whose A and B sources start
    // at ga and gb into `stage`: A's OPI, then B's. (groups of four: the
    // instruction offset is at most 4095 bytes)
    auto issue_one = [&](int stage, const char* ga, const char* gb, auto cc) {
        constexpr int c = decltype(cc)::value;
        if constexpr (c < OA::OPI) {
            constexpr int i = c, g = i / 4, o = (i % 4) * 1024;
            copy16<o>(lds_u32(a_lds(stage) + g * 4096), ga - o, aoffg[i]);
        } else {
            constexpr int i = c - OA::OPI, g = i / 4, o = (i % 4) * 1024;
            copy16<o>(lds_u32(b_lds(stage) + g * 4096), gb - o, boffg[i]);
        }
    };
    auto issue_at = [&](int stage, const char* ga, const char* gb) {
        static_for<0, Cf::IPW>([&](auto cc) { issue_one(stage, ga, gb, cc); });
    };
    // slice kt of this workgroup's K range
    // (the planner's K-reversed raster: the workgroups of odd rounds, 256
    // at a time, walk their K slices downward, so a round starts on the
    // slices the round before touched last, still in the last-level cache
    // for the tile rows the two share; whole slices only)
    const int krev = (!PERS && !SPLIT && p.krev && kbase == 0) ? (blockIdx.x >> 8) & 1 : 0;
    auto kslice = [&](int kt) { return kt0 + (krev ? NS - 1 - kt : kt); };
    auto src_a = [&](int kt) { return a_k0 + kslice(kt) * a_ks; };
    auto src_b = [&](int kt) { return b_k0 + kslice(kt) * b_ks; };
    auto issue = [&](int stage, int kt) { issue_at(stage, src_a(kt), src_b(kt)); };

    // Slice 0 when it is partial: a lane whose chunk lies below K = 0 writes
    // zeros where the copy would have put it (the copy's lane-linear LDS
    // position) instead of loading.
    auto issue_first_partial = [&]() {
        static_for<0, OA::OPI>([&](auto ic_) {
            constexpr int i = decltype(ic_)::value, g = i / 4, o = (i % 4) * 1024;
            char* d = a_lds(0) + g * 4096;
            if (kbase + OA::kpos(wave, lane, i) >= 0)
                copy16<o>(lds_u32(d), a_k0 - o, aoffg[i]);
            else
                *(LDS_AS u32x4*)(d + o + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        });
        static_for<0, OB::OPI>([&](auto ic_) {
            constexpr int i = decltype(ic_)::value, g = i / 4, o = (i % 4) * 1024;
            char* d = b_lds(0) + g * 4096;
            if (kbase + OB::kpos(wave, lane, i) >= 0)
                copy16<o>(lds_u32(d), b_k0 - o, boffg[i]);
            else
                *(LDS_AS u32x4*)(d + o + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        });
    };

    // ---- fragments: wave (wm, wn) owns rows wm*TWM.. of A and wn*TWN.. of B
    const int wm = wave % Cf::NWM, wn = wave / Cf::NWM;
    const int arow0 = wm * Cf::TWM, brow0 = wn * Cf::TWN;
    // per-lane LDS byte offsets; the K step s and the block add immediates
    using Mf = typename Cf::MFMA;
    int aoff[Cf::AK ? KS : FM], boff[Cf::BKM ? KS : FN];
    if constexpr (Cf::AK) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            aoff[s] = 16 * dev::KTile<BK>::at(arow0 + Mf::frag_row(lane), Mf::CHUNKS * s + Mf::frag_chunk(lane));
    } else {
#pragma unroll
        for (int b = 0; b < FM; ++b)
            aoff[b] = 16 * OA::MT::at(Mf::tr_krow(lane, 0), (arow0 + Cf::MF * b + Mf::tr_col(lane)) >> 3) +
                      2 * (Mf::tr_col(lane) & 7);
    }
    if constexpr (Cf::BKM) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            boff[s] = 16 * dev::KTile<BK>::at(brow0 + Mf::frag_row(lane), Mf::CHUNKS * s + Mf::frag_chunk(lane));
    } else {
#pragma unroll
        for (int b = 0; b < FN; ++b)
            boff[b] = 16 * OB::MT::at(Mf::tr_krow(lane, 0), (brow0 + Cf::MF * b + Mf::tr_col(lane)) >> 3) +
                      2 * (Mf::tr_col(lane) & 7);
    }

    // Fragment b of K step s of the slice in `stage`. K-major: row block b
    // is MF rows of BK*2 bytes further. M/N-major: K rows KSTEP*s + 4q (+
    // the lane's own rows, folded into off[b]); the row swizzle depends only
    // on krow & 3 and bit 3 of krow, which KSTEP*s + 4q keeps.
    auto read_a = [&](int stage, int s, int b) -> FA {
        const char* base = smem + stage * Cf::STAGE;
        if constexpr (Cf::AK)
            return FA{*(const LDS_AS V8*)(base + aoff[s] + b * Cf::MF * BK * 2)};
        else
            return read_tr<V8, OA::KROW_BYTES>(
                (const LDS_AS char*)(base + aoff[b] + Mf::KSTEP * s * OA::KROW_BYTES));
    };
    auto read_b = [&](int stage, int s, int b) -> FB {
        const char* base = smem + stage * Cf::STAGE + Cf::A_BYTES;
        if constexpr (Cf::BKM)
            return FB{*(const LDS_AS V8*)(base + boff[s] + b * Cf::MF * BK * 2)};
        else
            return read_tr<V8, OB::KROW_BYTES>(
                (const LDS_AS char*)(base + boff[b] + Mf::KSTEP * s * OB::KROW_BYTES));
    };

    FA af[2][FM];
    FB bfr[2][FN];
    auto read_step = [&](int stage, int s, int buf) {
#pragma unroll
        for (int b = 0; b < FM; ++b) af[buf][b] = read_a(stage, s, b);
#pragma unroll
        for (int b = 0; b < FN; ++b) bfr[buf][b] = read_b(stage, s, b);
    };
    // fragment r of K step s: A block r (r < FM), else B block r - FM
    auto read_one = [&](int stage, int s, int buf, auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (r < FM)
            af[buf][r] = read_a(stage, s, r);
        else
            bfr[buf][r - FM] = read_b(stage, s, r - FM);
    };

    using Acc = f32x4;
    static_assert(Cf::MF == 16, "the tiled kernel issues 16x16x32 MFMAs");
    Acc acc[FM][FN];
    for_blocks<FM, FN>([&](auto i, auto j) {
#pragma unroll
        for (int v = 0; v < Mf::NACC; ++v) acc[i][j][v] = 0.0f;
    });

    // ---- C prefetch (256x128 tiles, 3 stages, beta != 0, plain epilogue,
    // a whole tile, at least 3 slices): the 64 KiB C tile is copied into LDS
    // while the last slices run, into the two stages that no longer receive
    // slices: rows 0..191 (48 KiB) into slice NS-3's stage after that
    // slice's barrier, rows 192..255 into slice NS-2's stage after its
    // barrier. Chunk q (8 elements) of C row r sits at position q ^ (r mod
    // 16) of its 256-byte row, so the epilogue's 16 lanes that read one
    // column group of 16 consecutive rows hit 16 distinct bank groups. Copy k
    // (0..15) of wave w fills 1 KiB: rows 16k + 4w .. 16k + 4w + 3, lane l
    // row 16k + 4w + l/16, stored position l%16.
    constexpr bool CPF_CFG = !SPLIT && Cf::EXPLICIT && S == 3 && Cf::BN == 128 && Cf::BM == 256;
    constexpr int CROW = Cf::BN * 2;                  // bytes of one C row
    constexpr int CX_ROWS = Cf::STAGE / CROW;         // rows that fit one stage (192)
    static_assert(!CPF_CFG || (CX_ROWS == 192 && Cf::NW == 4), "C prefetch layout");
    const bool cpf = CPF_CFG && p.beta != 0.0f && !p.epi.fused && m0 + Cf::BM <= p.M && n0 + Cf::BN <= p.N &&
                     NS >= S && (int64_t)p.ldc * 2 * Cf::BM < (int64_t(1) << 32);
    // copy k of the C tile at (mt, nt) into the 48 KiB (k < 12) or 16 KiB
    // (k >= 12: rows 192..255) region at `base`
    auto issue_c_of = [&](const char* base, auto kc, int mt, int nt) {
        constexpr int k = decltype(kc)::value;
        constexpr int slot = k < 12 ? k : k - 12;
        const uint32_t cvoff =
            2u * (uint32_t)((wave * 4 + lane / 16) * p.ldc + 8 * ((lane % 16) ^ ((wave * 4 + lane / 16) & 15)));
        const char* c_tile = reinterpret_cast<const char*>(p.C + (int64_t)(mt + 16 * k) * p.ldc + nt);
        copy16<0>(lds_u32(base + (slot * 4 + wave) * 1024), c_tile, cvoff);
    };
    auto issue_c = [&](const char* base, auto kc) { issue_c_of(base, kc, m0, n0); };

    // ---- prologue: slices 0 .. S-1
    if (kbase < 0 && kt0 == 0)
        issue_first_partial();
    else
        issue(0, 0);
#pragma unroll
    for (int s = 1; s < S; ++s)
        if (s < NS) issue(s, s);
    if (NS >= S)
        LT_WAIT_VM(Cf::IPW * (S - 1));
    else
        LT_WAIT_VM(0);
    __syncthreads();
    read_step(0, 0, 0);

    // One K slice: KS MFMA steps on the fragments already in registers, the
    // next step's fragments read one step ahead. In the last step the
    // barrier publishes slice t+1 (and frees slice t's stage, refilled with
    // slice t+S at once), and slice t+1's first fragments are read while the
    // last step's MFMAs run. Three branch-free variants: with a refill, with
    // a next slice but no refill, and the final slice.
    constexpr int NMF = FM * FN, NRD = (Cf::AK ? FM : 2 * FM) + (Cf::BKM ? FN : 2 * FN);
    int stage = 0;
    auto slice_s = [&](auto has_next, auto refill, int t, auto par) {
        static_for<0, KS>([&](auto sc) {
            constexpr int s = decltype(sc)::value, cur = (decltype(par)::value + s) & 1, nxt = cur ^ 1;
            if constexpr (s + 1 < KS) {
                read_step(stage, s + 1, nxt);
            } else if constexpr (decltype(has_next)::value) {
                if constexpr (decltype(refill)::value)
                    LT_WAIT_VM(Cf::IPW * (S - 2));   // slice t+1 landed (S-2 newer slices may fly)
                else
                    LT_WAIT_VM(0);
                __syncthreads();   // slice t+1 visible to all; slice t's stage free
                if constexpr (decltype(refill)::value) issue(stage, t + S);
                read_step(stage + 1 == S ? 0 : stage + 1, 0, nxt);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = Tr<DT>::mfma16(bfr[cur][j].get(), af[cur][i].get(), acc[i][j]);
            // Issue order for this step: groups of two MFMAs, then two of the
            // slice copies (last step only), then two fragment reads for the
            // next step, until the reads are out; the remaining MFMAs cover
            // the reads' latency.
            if (s + 1 < KS || decltype(has_next)::value) {
                constexpr int MPG = 2, VPG = 2, RPG = 2;
                constexpr int GROUPS = (NRD + RPG - 1) / RPG;
                const bool copies = s + 1 == KS && decltype(refill)::value;
#pragma unroll
                for (int q = 0; q < GROUPS; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, MPG, 0);
                    if (copies && VPG * q < Cf::IPW) __builtin_amdgcn_sched_group_barrier(0x020, VPG, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, RPG, 0);
                }
                if (copies && VPG * GROUPS < Cf::IPW)
                    __builtin_amdgcn_sched_group_barrier(0x020, Cf::IPW - VPG * GROUPS, 0);
                if (NMF > MPG * GROUPS) __builtin_amdgcn_sched_group_barrier(0x008, NMF - MPG * GROUPS, 0);
            }
        });
        stage = stage + 1 == S ? 0 : stage + 1;
    };
    // The one-wave-per-SIMD schedule. Per K step: the MFMAs in block order,
    // the next step's fragment reads spread over the first three quarters of
    // them (one every few MFMAs, so the LDS sees a steady stream and the last
    // read has a quarter of the step to land), and in the last step, after
    // the barrier, the slice copies spread over all of them. The accumulators
    // are asm operands bound to AGPRs ("a"), which keeps all of them there.
    auto mfma_one = [&](int cur, auto qc) {
        constexpr int q = decltype(qc)::value, i = q / FN, j = q % FN;
        auto& c = acc[i][j];
        const V8 x = bfr[cur][j].get(), y = af[cur][i].get();
        if constexpr (DT == LT_BF16)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
        else
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    };
    // the same with a zero accumulator input: the first K step of a tile
    // in the persistent launch starts each block at zero this way
    auto mfma_first = [&](int cur, auto qc) {
        constexpr int q = decltype(qc)::value, i = q / FN, j = q % FN;
        auto& c = acc[i][j];
        const V8 x = bfr[cur][j].get(), y = af[cur][i].get();
        if constexpr (DT == LT_BF16)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(x), "v"(y));
        else
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(c) : "v"(x), "v"(y));
    };
    // cpc: 0, or 1 / 2 for the slice that also copies the first 12 / last 4
    // copies of the C tile (into its own stage, after its barrier). ga, gb:
    // the sources of the slice a refill copies. first: the slice starts a
    // tile of the persistent launch (its first K step zeroes the
    // accumulators). waitc: the vmcnt the barrier waits for, or -1 for the
    // count the variant implies.
    auto slice_x = [&](auto has_next, auto refill, const char* ga, const char* gb, auto par, auto cpc, auto first,
                       auto waitc) {
        constexpr int CP = decltype(cpc)::value;
        constexpr int WAITC = decltype(waitc)::value;
        static_for<0, KS>([&](auto sc) {
            constexpr int s = decltype(sc)::value, cur = (decltype(par)::value + s) & 1, nxt = cur ^ 1;
            constexpr bool last = s + 1 == KS;
            constexpr bool reads = !last || decltype(has_next)::value;
            constexpr bool copies = last && decltype(refill)::value;
            constexpr int NCP = !last ? 0 : CP == 1 ? 12 : CP == 2 ? 4 : 0;
            constexpr int NR = reads ? FM + FN : 0, NC = copies ? Cf::IPW : NCP, NQ = FM * FN;
            static_assert(Cf::IPW <= NQ && 4 * (FM + FN) <= 3 * NQ, "one copy and one read per MFMA at most");
            static_assert(CP == 0 || (!decltype(refill)::value && decltype(has_next)::value), "C copies");
            int rstage = stage, rs = s + 1;
            if constexpr (last && decltype(has_next)::value) {
                if constexpr (WAITC >= 0)
                    LT_WAIT_VM(WAITC);
                else if constexpr (decltype(refill)::value)
                    LT_WAIT_VM(Cf::IPW * (S - 2));   // slice t+1 landed (S-2 newer slices may fly)
                else if constexpr (CP == 2)
                    LT_WAIT_VM(12);                  // slice t+1 landed; the first 12 C copies may fly
                else
                    LT_WAIT_VM(0);
                __syncthreads();   // slice t+1 visible to all; slice t's stage free
                rstage = stage + 1 == S ? 0 : stage + 1;
                rs = 0;
            }
            static_for<0, NQ>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                if constexpr (decltype(first)::value && s == 0)
                    mfma_first(cur, qc);
                else
                    mfma_one(cur, qc);
                constexpr int c = copy_after(q, NC, NQ);
                if constexpr (c >= 0) {
                    if constexpr (copies)
                        issue_one(stage, ga, gb, ic<c>{});
                    else
                        issue_c(smem + stage * Cf::STAGE, ic<CP == 1 ? c : 12 + c>{});
                }
                constexpr int r = read_after(q, NR, NQ);
                if constexpr (r >= 0) read_one(rstage, rs, nxt, ic<r>{});
            });
        });
        stage = stage + 1 == S ? 0 : stage + 1;
    };
    const std::true_type yes{};
    const std::false_type no{};
    // slice t (local index); with one K step per slice its fragment buffer
    // is t's parity, a compile-time index in each of two copies of the body
    auto slice = [&](auto has_next, auto refill, int t, auto cpc) {
        auto go = [&](auto par) {
            if constexpr (Cf::EXPLICIT)
                slice_x(has_next, refill, src_a(t + S), src_b(t + S), par, cpc, no, ic<-1>{});
            else
                slice_s(has_next, refill, t, par);
        };
        if constexpr (KS % 2 == 0) {
            go(ic<0>{});
        } else {
            if (t & 1)
                go(ic<1>{});
            else
                go(ic<0>{});
        }
    };
    // the zeroed accumulators are written by VALU moves: wait states before
    // the first inline-asm MFMA reads them (the compiler does not see it as one)
    if constexpr (Cf::EXPLICIT) asm volatile("s_nop 7" ::: "memory");
    // ---- epilogue: block (i, j), registers 4g..4g+3 hold row m = lane % MF
    // and four consecutive columns of the MF x MF block. A tile on a ragged
    // edge stores only the outputs inside (M, N). With beta != 0 every C load
    // of the wave is issued before the first is waited on (one memory round
    // trip per tile, not one per block); the fragment registers are free by
    // now and hold them.
    constexpr int NG = Mf::NACC / 4;   // groups of four outputs per block
    // ---- staged store (K-major data-parallel and persistent launches:
    // whole tiles with beta = 0, edge tiles, and tiles whose C values are
    // already in registers). In the accumulators' layout the 16 lanes of a
    // quarter-wave store 8 bytes to each of 16
    // rows, so one store instruction reaches 64 cache lines. Staged through
    // LDS, the 16 lanes store 256 contiguous bytes of one row (two rows of
    // 128 with 64-column wave tiles): 8 lines per instruction, and half the
    // instructions. Each wave owns DSW bytes beside the ring and runs
    // passes of RPP rows of its wave tile: it writes them in the
    // accumulators' layout (8 bytes per lane), reads them back 16 bytes per
    // lane along the rows and stores them. The region is the wave's own and
    // LDS executes one wave's instructions in order, so no barrier is
    // needed. The rows are swizzled in 8-byte units (dev::StagedRows) so
    // that the writes (16 rows, one column group) and the reads (one or two
    // rows) each reach every bank once; a read whose two halves the swizzle
    // swapped swaps them back in registers.
    constexpr bool STAGED_D = staged_d<Cf, MODE>();
    constexpr int DSW = staged_d_bytes<Cf, MODE>() / Cf::NW;   // bytes per wave
    constexpr int RB = Cf::TWN * 2;                             // bytes of one wave-tile row
    constexpr int CPR = RB / 16;                                // its 16-byte chunks
    constexpr int RPP = STAGED_D ? DSW / RB : Cf::MF;           // rows per pass
    constexpr int BPP = RPP / Cf::MF;                           // accumulator block rows per pass
    static_assert(!STAGED_D || (NG == 1 && BPP >= 1 && FM % BPP == 0 && (CPR == 16 || CPR == 8) &&
                                (RPP * RB) % 1024 == 0 && Cf::LDS + Cf::NW * DSW <= 160 * 1024),
                  "staged store layout");
    using SR = dev::StagedRows<CPR>;
    // 8 accumulator values (16 bytes) of row r, chunk q, from a staged region
    auto read_row16 = [&](const char* region, int r, int q) {
        const u32x4 x = *(const LDS_AS u32x4*)(region + SR::slot(r, q));
        return SR::swapped(r) ? u32x4{x.z, x.w, x.x, x.y} : x;
    };
    // cval(i, j): the C values of block (i, j) for epi4 (zero when beta = 0).
    // A tile on a ragged edge (edge = true) stores the rows below M only, and
    // of a 16-byte chunk that N cuts, its first elements one at a time (D's
    // rows start 16-byte aligned, so every chunk left of N is whole).
    auto store_staged = [&](auto&& cval, auto edge) {
        constexpr bool EDGE = decltype(edge)::value;
        char* region = smem + Cf::LDS + wave * DSW;
        static_for<0, FM / BPP>([&](auto pc) {
            constexpr int ps = decltype(pc)::value;
            for_blocks<BPP, FN>([&](auto bi, auto j) {
                constexpr int i = ps * BPP + decltype(bi)::value;
                const int r = decltype(bi)::value * Cf::MF + Mf::out_col(lane);
                const int cb = 2 * (j * Cf::MF + Mf::out_row(lane, 0));   // byte of the wave-tile row
                const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                *(LDS_AS u32x2*)(region + SR::unit(r, cb >> 3)) = epi4<DT>(v, p.alpha, p.beta, cval(i, j));
            });
            // all the pass's reads, then its stores (each store waits only
            // for its own read)
            constexpr int NRD16 = RPP * RB / 1024;
            u32x4 w[NRD16];
            static_for<0, NRD16>([&](auto kc) {
                const int lin16 = decltype(kc)::value * 64 + lane;   // 16-byte unit of the pass
                w[decltype(kc)::value] = read_row16(region, lin16 / CPR, lin16 % CPR);
            });
            static_for<0, NRD16>([&](auto kc) {
                const int lin16 = decltype(kc)::value * 64 + lane;
                const int r = lin16 / CPR, q = lin16 % CPR;
                const int m = m0 + arow0 + ps * RPP + r, n = n0 + brow0 + 8 * q;
                uint16_t* dst = p.D + (int64_t)m * p.ldd + n;
                const u32x4 x = w[decltype(kc)::value];
                if constexpr (EDGE) {
                    if (m < p.M) {
                        if (n + 8 <= p.N) {
                            *reinterpret_cast<u32x4*>(dst) = x;
                        } else if (n < p.N) {
                            const uint32_t u[4] = {x.x, x.y, x.z, x.w};
                            for (int e = 0; e < p.N - n; ++e) dst[e] = uint16_t(u[e >> 1] >> (16 * (e & 1)));
                        }
                    }
                } else {
                    *reinterpret_cast<u32x4*>(dst) = x;
                }
            });
            // one pass at a time: the next pass's conversions are not hoisted
            // above this one's stores (they would hold more registers)
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // ---- staged store with C (a whole 256x256 tile of the data-parallel
    // launch, beta != 0). After a barrier the ring is free, a quarter per
    // wave, which holds the wave's C tile (dev::StagedC): the wave copies
    // it in row-coalesced 16-byte copies (each lane fetching the chunk that
    // the map stores at its position) and reads it in the accumulators'
    // layout. It then writes D into the same rows in the layout of the
    // store without C (a block row's D goes in only after all of its C has
    // been read: the two layouts place a row's units differently) and reads
    // D back along the rows for the stores. A wave reads all of its C before
    // it stores any D and no other wave reads those elements, so D may be
    // C.
    constexpr bool STAGED_C = STAGED_D && MODE == kDataParallel && Cf::BN == 256;
    constexpr int CWB = Cf::TWM * RB;   // bytes of a wave's C tile
    static_assert(!STAGED_C || (Cf::NW * CWB <= Cf::LDS && CWB % 8192 == 0), "the C tiles fit the ring");
    auto store_staged_c = [&]() {
        static_assert(!STAGED_C || CPR == 16, "256-byte rows");
        char* region = smem + wave * CWB;
        const char* cbase = reinterpret_cast<const char*>(p.C + (int64_t)(m0 + arow0) * p.ldc + n0 + brow0);
        __syncthreads();   // every wave is done with the ring
        static_for<0, CWB / 1024>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const int lin16 = 64 * k + lane, r = lin16 / CPR;
            copy16<0>(lds_u32(region + 1024 * k), cbase,
                      2u * (uint32_t)(r * p.ldc + 8 * dev::StagedC::chunk_at(r, lin16 % CPR)));
        });
        LT_WAIT_VM(0);   // the wave's own C copies have landed
        // C read and D written in the accumulators' layout, a block row at a time
        static_for<0, FM>([&](auto ic_) {
            constexpr int i = decltype(ic_)::value;
            u32x2 cvr[FN];
            static_for<0, FN>([&](auto jc) {
                const int r = i * Cf::MF + Mf::out_col(lane), cb = 2 * (jc * Cf::MF + Mf::out_row(lane, 0));
                cvr[jc] = *(const LDS_AS u32x2*)(region + dev::StagedC::at(r, cb >> 4) + (cb & 15));
            });
            static_for<0, FN>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const int r = i * Cf::MF + Mf::out_col(lane), cb = 2 * (j * Cf::MF + Mf::out_row(lane, 0));
                const float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
                *(LDS_AS u32x2*)(region + SR::unit(r, cb >> 3)) = epi4<DT>(v, p.alpha, p.beta, cvr[j]);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        // D along the rows: eight reads, then their stores
        static_for<0, CWB / 8192>([&](auto bc) {
            u32x4 w[8];
            static_for<0, 8>([&](auto kc) {
                const int lin16 = 64 * (8 * bc + kc) + lane;
                w[kc] = read_row16(region, lin16 / CPR, lin16 % CPR);
            });
            static_for<0, 8>([&](auto kc) {
                const int lin16 = 64 * (8 * bc + kc) + lane, r = lin16 / CPR, q = lin16 % CPR;
                *reinterpret_cast<u32x4*>(p.D + (int64_t)(m0 + arow0 + r) * p.ldd + n0 + brow0 + 8 * q) = w[kc];
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    auto epilogue = [&](auto edge) {
        constexpr bool EDGE = decltype(edge)::value;
        const bool use_c = p.beta != 0.0f;
        if constexpr (STAGED_D) {
            if (!use_c) {
                store_staged([](int, int) { return u32x2{0u, 0u}; }, edge);
                return;
            }
        }
        u32x2 cv[FM][FN][NG];
        auto load_c = [&](auto guarded) {
            for_blocks<FM, FN>([&](auto i, auto j) {
                const int m = m0 + arow0 + i * Cf::MF + Mf::out_col(lane);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int n = n0 + brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g);
                    const u32x2* src = reinterpret_cast<const u32x2*>(p.C + (int64_t)m * p.ldc + n);
                    if constexpr (decltype(guarded)::value) {
                        cv[i][j][g] = (m < p.M && n + 4 <= p.N) ? *src : u32x2{0u, 0u};
                        // the staged store takes C from here, also of the
                        // group that N cuts (the direct store reads that
                        // group's C itself)
                        if constexpr (STAGED_D) {
                            if (m < p.M && n < p.N && n + 4 > p.N) {
                                const uint16_t* c = p.C + (int64_t)m * p.ldc + n;
                                uint32_t h[4] = {0u, 0u, 0u, 0u};
                                for (int e = 0; e < p.N - n; ++e) h[e] = c[e];
                                cv[i][j][g] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
                            }
                        }
                    } else
                        cv[i][j][g] = *src;
                }
            });
        };
        if (!use_c) {
            for_blocks<FM, FN>([&](auto i, auto j) {
#pragma unroll
                for (int g = 0; g < NG; ++g) cv[i][j][g] = u32x2{0u, 0u};
            });
        } else if (CPF_CFG && !EDGE && cpf) {
            // the C tile is in LDS: rows < 192 in slice NS-3's stage, the
            // rest in slice NS-2's
            LT_WAIT_VM(0);
            __syncthreads();   // every wave's C copies landed
            const int sx = (NS - 3) % S, sy = (NS - 2) % S;
            for_blocks<FM, FN>([&](auto i, auto j) {
                const int r = arow0 + i * Cf::MF + Mf::out_col(lane);
                const char* row = smem + (r < CX_ROWS ? sx * Cf::STAGE + r * CROW : sy * Cf::STAGE + (r - CX_ROWS) * CROW);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int c = brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g);
                    cv[i][j][g] = *(const LDS_AS u32x2*)(row + 16 * ((c >> 3) ^ (r & 15)) + 2 * (c & 7));
                }
            });
            if constexpr (STAGED_D) {   // D through the region beside the stages
                store_staged([&](int i, int j) { return cv[i][j][0]; }, std::false_type{});
                return;
            }
        } else {
            load_c(std::integral_constant<bool, EDGE>{});   // a whole tile loads with no branch per block
            if constexpr (STAGED_D) {
                store_staged([&](int i, int j) { return cv[i][j][0]; }, edge);
                return;
            }
        }
        for_blocks<FM, FN>([&](auto i, auto j) {
            const int m = m0 + arow0 + i * Cf::MF + Mf::out_col(lane);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int n = n0 + brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g);
                const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                    acc[i][j][4 * g + 3]};
                if constexpr (EDGE) {
                    if (m < p.M && n < p.N) {
                        if (n + 4 <= p.N)
                            store4_c<DT>(p.D, (int64_t)m * p.ldd + n, v, p.alpha, p.beta, cv[i][j][g]);
                        else
                            store_n<DT>(p.D, p.C, (int64_t)m * p.ldd + n, (int64_t)m * p.ldc + n, v, p.N - n,
                                        p.alpha, p.beta);
                    }
                } else {
                    store4_c<DT>(p.D, (int64_t)m * p.ldd + n, v, p.alpha, p.beta, cv[i][j][g]);
                }
            }
        });
    };
    // The fused epilogue (bias, activation, max |D|), for any tile. Its C
    // values and bias entries are gathered before any is used, as above: a
    // row bias is one value per block row i, a column bias four per (j, g),
    // the same for every i.
    auto epilogue_fused = [&]() {
        const EpiArgs& e = p.epi;
        const bool use_c = p.beta != 0.0f;
        float brow[FM];
        uint16_t bcol[FN][NG][4];   // kept in the operand format until used: fewer registers
#pragma unroll
        for (int i = 0; i < FM; ++i) brow[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) bcol[j][g][q] = 0;
        if (e.bias && e.bias_on_rows) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m0 + arow0 + i * Cf::MF + Mf::out_col(lane);
                brow[i] = m < p.M ? Tr<DT>::to_f32(e.bias[(int64_t)m * e.bias_stride]) : 0.0f;
            }
        } else if (e.bias) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < NG; ++g)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n0 + brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g) + q;
                        bcol[j][g][q] = n < p.N ? e.bias[(int64_t)n * e.bias_stride] : uint16_t{0};
                    }
        }
        u32x2 cv[FM][FN][NG];
        for_blocks<FM, FN>([&](auto i, auto j) {
            const int m = m0 + arow0 + i * Cf::MF + Mf::out_col(lane);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int n = n0 + brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g);
                cv[i][j][g] = use_c && m < p.M && n + 4 <= p.N
                                  ? *reinterpret_cast<const u32x2*>(p.C + (int64_t)m * p.ldc + n)
                                  : u32x2{0u, 0u};
            }
        });
        float amax = 0.0f;
        for_blocks<FM, FN>([&](auto i, auto j) {
            const int m = m0 + arow0 + i * Cf::MF + Mf::out_col(lane);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int n = n0 + brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g);
                if (m >= p.M || n >= p.N) continue;
                const int cnt = min(4, p.N - n);
                const uint16_t c16[4] = {static_cast<uint16_t>(cv[i][j][g].x & 0xffff),
                                         static_cast<uint16_t>(cv[i][j][g].x >> 16),
                                         static_cast<uint16_t>(cv[i][j][g].y & 0xffff),
                                         static_cast<uint16_t>(cv[i][j][g].y >> 16)};
                uint16_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v = p.alpha * acc[i][j][4 * g + q];
                    if (use_c)   // a partial group (cnt < 4) reads its C elements here
                        v += p.beta * Tr<DT>::to_f32(cnt == 4 ? c16[q]
                                                              : (q < cnt ? p.C[(int64_t)m * p.ldc + n + q]
                                                                         : uint16_t{0}));
                    v += e.bias_on_rows ? brow[i] : Tr<DT>::to_f32(bcol[j][g][q]);
                    o[q] = Tr<DT>::from_f32(activate(v, e.act));
                    if (q < cnt) amax = fmaxf(amax, fabsf(Tr<DT>::to_f32(o[q])));
                }
                if (cnt == 4) {
                    u32x2 w;
                    w.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                    w.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                    *reinterpret_cast<u32x2*>(p.D + (int64_t)m * p.ldd + n) = w;
                } else {
                    for (int q = 0; q < cnt; ++q) p.D[(int64_t)m * p.ldd + n + q] = o[q];
                }
            }
        });
        if (e.amax) amax_commit(e.amax, amax);
    };
    // ---- persistent launch (whole tiles, K a multiple of BK, NS >= 4): the
    // K loop runs over the concatenation of this workgroup's tiles' slices,
    // so the next tile's first slices are copied while the current tile's
    // last slices run, and one more right after the current tile's
    // epilogue, into the stage that the last slices leave to C or to that
    // copy. ("CUTLASS, in depth", "Kernel schedules": a persistent kernel
    // walks tiles from a tile scheduler and overlaps one tile's epilogue
    // with the next tile's main loop.)
    if constexpr (PERS) {
        constexpr bool WITH_C = MODE == kPersistentC;
        static_assert(Cf::EXPLICIT && KS % 2 == 0 && (S == 3 || (S == 2 && !WITH_C)),
                      "the persistent launch runs the explicit schedule: 3 stages, or 2 without C");
        // With C (256x128 tiles, 3 stages): the C tile goes through LDS in
        // row-coalesced 16-byte copies, rows 0..191 (48 KiB, one stage) in
        // the refill slot of the tile's slice NS-2, rows 192..255 (16 KiB) in
        // the space beside the three stages at the tile's start; the next
        // tile's slice 1, whose slot that was, follows the epilogue.
        static_assert(!WITH_C || (CPF_CFG && CX_ROWS == 192), "C staging layout");
        const char* c_spare = smem + S * Cf::STAGE;
        auto issue_c_spare = [&](int mt, int nt) {
            static_for<12, 16>([&](auto kc) { issue_c_of(c_spare, kc, mt, nt); });
        };
        u32x2 cv[FM][FN][NG];
        // C of this tile, from LDS into the accumulators' layout: rows
        // below 192 from the stage at st_c, the others from the spare
        // region (16-byte chunk q of row r stored at q ^ (r mod 16))
        auto read_c_lds = [&](int st_c) {
            for_blocks<FM, FN>([&](auto i, auto j) {
                const int r = arow0 + i * Cf::MF + Mf::out_col(lane);
                const char* crow = r < CX_ROWS ? smem + st_c * Cf::STAGE + r * CROW : c_spare + (r - CX_ROWS) * CROW;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int c = brow0 + j * Cf::MF + Mf::out_row(lane, 4 * g);
                    cv[i][j][g] = *(const LDS_AS u32x2*)(crow + 16 * ((c >> 3) ^ (r & 15)) + 2 * (c & 7));
                }
            });
        };
        if constexpr (WITH_C) issue_c_spare(m0, n0);   // the first tile's C rows 192..255
        // Every tile runs the same slice sequence, so no control flow
        // joins while MFMA results are in flight (at a join the compiler
        // may copy accumulators): the last tile takes itself as its "next"
        // tile, whose first slices (and C rows 192..255) are then copied
        // again into LDS nobody reads, and waited for before the workgroup
        // ends.
        int m0n = m0, n0n = n0;
        const char* na = a_k0;
        const char* nb = b_k0;
        for (int j = 0;; ++j) {
            const bool more = j + 1 < ntl;
            if (more) {
                int tmj, tnj;
                tile_coords(first + (j + 1) * step, p, &tmj, &tnj);
                m0n = tmj * Cf::BM;
                n0n = tnj * Cf::BN;
                na = reinterpret_cast<const char*>(p.A0) + OA::tile_bytes(p.lda, m0n);
                nb = reinterpret_cast<const char*>(p.B0) + OB::tile_bytes(p.ldb, n0n);
            }
            // slice t refills slice t+S of the sequence: this tile's, else
            // the next tile's slice t+S-NS
            auto ref_a = [&](int t) { return t + S < NS ? a_k0 + (t + S) * a_ks : na + (t + S - NS) * a_ks; };
            auto ref_b = [&](int t) { return t + S < NS ? b_k0 + (t + S) * b_ks : nb + (t + S - NS) * b_ks; };
            if constexpr (!WITH_C) {
                slice_x(yes, yes, ref_a(0), ref_b(0), ic<0>{}, ic<0>{}, yes, ic<-1>{});
                for (int t = 1; t + 1 < NS; ++t)
                    slice_x(yes, yes, ref_a(t), ref_b(t), ic<0>{}, ic<0>{}, no, ic<-1>{});
                // the tile's last slice: the barrier waits for the next
                // tile's slice 0 while its slices 1 .. S-2 may fly
                const int st_last = stage;
                slice_x(yes, no, a_k0, b_k0, ic<0>{}, ic<0>{}, no, ic<Cf::IPW * (S - 2)>{});
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // MFMA results before VALU reads
                store_staged([](int, int) { return u32x2{0u, 0u}; }, std::false_type{});
                if (!more) break;
                issue_at(st_last, na + (S - 1) * a_ks, nb + (S - 1) * b_ks);   // the next tile's slice S-1
            } else {
                // vmcnt waits (loads complete in order; a wait counts the
                // loads issued after the one it waits for, and the epilogue's
                // stores can only lengthen it): slice 0 waits for slice 1,
                // after which only this tile's 4 C copies come (the first
                // tile: its slice 2 as well); slice 1 for slice 2, after
                // which 16 or 28 copies come (the next tile's slice 1, the C
                // copies and slice 3); slice NS-2 for slice NS-1 with the
                // next tile's slice 0 after it; slice NS-1 for the next
                // tile's slice 0 with this tile's C rows 0..191 after it; the
                // epilogue for those rows with the next tile's slice 2 after
                // them.
                slice_x(yes, yes, ref_a(0), ref_b(0), ic<0>{}, ic<0>{}, yes, ic<4>{});
                slice_x(yes, yes, ref_a(1), ref_b(1), ic<0>{}, ic<0>{}, no, ic<16>{});
                for (int t = 2; t + 2 < NS; ++t)
                    slice_x(yes, yes, ref_a(t), ref_b(t), ic<0>{}, ic<0>{}, no, ic<-1>{});
                // slice NS-2: its refill slot takes C rows 0..191
                const int st_c = stage;
                slice_x(yes, no, a_k0, b_k0, ic<0>{}, ic<1>{}, no, ic<Cf::IPW>{});
                // slice NS-1: refilled with the next tile's slice 2
                slice_x(yes, yes, na + 2 * a_ks, nb + 2 * b_ks, ic<0>{}, ic<0>{}, no, ic<Cf::IPW>{});
                asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // MFMA results before VALU reads
                LT_WAIT_VM(Cf::IPW);   // C rows 0..191 landed (the next tile's slice 2 may fly)
                __syncthreads();       // every wave's C copies visible
                read_c_lds(st_c);
                __syncthreads();       // every wave has its C values: the stage and the spare are free
                // the next tile's slice 1, this tile's D through the spare,
                // then (once every wave has read its rows back) the next
                // tile's C rows 192..255 into the spare (the last tile: its
                // own again, unused)
                issue_at(st_c, na + a_ks, nb + b_ks);
                store_staged([&](int i, int j) { return cv[i][j][0]; }, std::false_type{});
                __syncthreads();
                issue_c_spare(m0n, n0n);
                if (!more) break;
            }
            m0 = m0n;
            n0 = n0n;
            a_k0 = na;
            b_k0 = nb;
        }
        // no copy into LDS, nor a read of the unused fragments, outlives
        // the workgroup
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    int t = 0;
    for (; t + S < NS; ++t) slice(yes, yes, t, ic<0>{});   // refill slice t+S
    // The C-prefetch path runs its last slices and its epilogue on its own:
    // no control flow joins the two paths while MFMA results are in flight
    // (at a join the compiler may copy accumulators, and it cannot see the
    // inline-asm MFMAs' wait states).
    if constexpr (CPF_CFG) {
        if (cpf) {   // S == 3 and NS >= 3: slices NS-3 and NS-2 copy the C tile
            slice(yes, no, t, ic<1>{});
            ++t;
            slice(yes, no, t, ic<2>{});
            ++t;
            slice(no, no, t, ic<0>{});
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            epilogue(std::false_type{});   // a whole tile, beta != 0, plain epilogue
            return;
        }
    }
    for (; t + 1 < NS; ++t) slice(yes, no, t, ic<0>{});   // slices already in flight
    slice(no, no, t, ic<0>{});                            // the last slice
    // MFMA results before any VALU or memory instruction reads them (the
    // scheduling barrier keeps the epilogue's accumulator reads from being
    // hoisted into the last slice, where they would also hold registers
    // beside the accumulators)
    if constexpr (Cf::EXPLICIT) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // each accumulator block redefined here, in its AGPRs, by an empty
        // statement: a register the epilogues need moved or spilled is then
        // moved or spilled after the wait states, never between MFMAs
        for_blocks<FM, FN>([&](auto i, auto j) {
            auto& c = acc[i][j];
            asm volatile("" : "+a"(c));
        });
    }

    // ---- split-K segment: publish the fp32 partial; the segment that
    // arrives last adds the others' and goes on to the epilogue. No waiting:
    // the others simply end. The partials and the arrival count cross XCDs,
    // whose L2s are not coherent with each other: they are written and read
    // with agent-scope relaxed atomics (the coherent path, past this XCD's
    // L2), so no fence has to write back or invalidate a whole L2 while
    // other tiles are running. Order: every store of the partial completes
    // (vmcnt 0, then the barrier) before the count is incremented, and the
    // last segment issues its reads only after the increment returned.
    if constexpr (SPLIT) {
        const int skt = lin - p.dp_tiles, NSPL = p.sk_splits;
        // block (i, j) of split s2: register v of thread t at v*NT + t, so
        // that one store (load) instruction covers 256 contiguous bytes
        auto part = [&](int s2, int i, int j) {
            return p.partials + (((int64_t)skt * NSPL + s2) * (FM * FN) + (i * FN + j)) * (Cf::NT * Mf::NACC) +
                   threadIdx.x;
        };
        for_blocks<FM, FN>([&](auto i, auto j) {
            float* q = part(seg, i, j);
#pragma unroll
            for (int v = 0; v < Mf::NACC; ++v)
                __hip_atomic_store(q + v * Cf::NT, acc[i][j][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        });
        LT_WAIT_VM(0);
        __syncthreads();   // every store of the partial is complete; the LDS ring is free
        int* flag = reinterpret_cast<int*>(smem);
        if (threadIdx.x == 0)
            *flag = __hip_atomic_fetch_add(&p.counters[skt], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (*flag != NSPL - 1) return;
        for (int s2 = 0; s2 < NSPL; ++s2) {
            if (s2 == seg) continue;
            for_blocks<FM, FN>([&](auto i, auto j) {
                const float* q = part(s2, i, j);
#pragma unroll
                for (int v = 0; v < Mf::NACC; ++v)
                    acc[i][j][v] += __hip_atomic_load(q + v * Cf::NT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            });
        }
        if (threadIdx.x == 0) __hip_atomic_store(&p.counters[skt], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    const bool whole = m0 + Cf::BM <= p.M && n0 + Cf::BN <= p.N;
    if (p.epi.fused) {
        epilogue_fused();
    } else if constexpr (STAGED_C) {
        // whole tiles through LDS; the predicated path takes the rest (and
        // a C whose rows lie too far apart for the 32-bit copy offsets)
        if (whole && p.beta == 0.0f)
            store_staged([](int, int) { return u32x2{0u, 0u}; }, std::false_type{});
        else if (whole && (int64_t)p.ldc * 2 * Cf::TWM < (int64_t(1) << 32))
            store_staged_c();
        else
            epilogue(std::true_type{});
    } else if (!whole) {
        epilogue(std::true_type{});
    } else {
        epilogue(std::false_type{});
    }
#else
    (void)p;
#endif
}

namespace {

// LDS of a launch: the stages, then the staged store's region or (the
// persistent launch with C) the 16 KiB of C rows 192..255
template <class Cf, int MODE>
constexpr int launch_lds() {
    return launch_lds_bytes(Cf::LDS, staged_d<Cf, MODE>(), MODE == kPersistentC);
}
template <int DT, class Cf, int MODE>
int launch_mode(const TiledArgs& a, int grid, hipStream_t s) {
    constexpr int lds = launch_lds<Cf, MODE>();
    static_assert(lds <= 160 * 1024, "LDS per workgroup");
    static std::atomic<uint64_t> attr{0};
    if (const int e = set_lds_limit_once(reinterpret_cast<const void*>(&gemm_tiled<DT, Cf, MODE>), lds, attr))
        return e;
    hipLaunchKernelGGL((gemm_tiled<DT, Cf, MODE>), dim3(grid), dim3(Cf::NT), lds, s, a);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

// 128x128 tiles: one workgroup per tile. 256x128 tiles: one workgroup per
// tile, or (persist_grid > 0) a
// persistent launch of persist_grid workgroups walking the tiles; the
// planner never splits them. 256x256 tiles: the data-parallel tiles, then
// (same stream, so after them) the split remainder.
template <int DT, bool AK, bool BKM>
int launch_variant(const TiledArgs& a, int tile_m, int tile_n, int persist_grid, void* stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (tile_m == 128)   // 128x128 tiles: one workgroup per tile, never split or persistent
        return a.dp_tiles > 0 ? launch_mode<DT, Dp128x128<AK, BKM>, kDataParallel>(a, a.dp_tiles, s) : 0;
    if (tile_n == 128) {
        if (persist_grid > 0)
            return a.beta != 0.0f ? launch_mode<DT, Dp128<AK, BKM>, kPersistentC>(a, persist_grid, s)
                                  : launch_mode<DT, Dp128<AK, BKM>, kPersistent>(a, persist_grid, s);
        return a.dp_tiles > 0 ? launch_mode<DT, Dp128<AK, BKM>, kDataParallel>(a, a.dp_tiles, s) : 0;
    }
    if (persist_grid > 0)   // 256x256 tiles, beta = 0, no split remainder (the planner's rule)
        return a.beta == 0.0f ? launch_mode<DT, Dp256<AK, BKM>, kPersistent>(a, persist_grid, s)
                              : static_cast<int>(hipErrorInvalidValue);
    if (a.dp_tiles > 0) {
        const int e = launch_mode<DT, Dp256<AK, BKM>, kDataParallel>(a, a.dp_tiles, s);
        if (e != 0) return e;
    }
    const int split_wgs = (a.tiles_m * a.tiles_n - a.dp_tiles) * a.sk_splits;
    if (split_wgs > 0) return launch_mode<DT, Split256<AK, BKM>, kSplit>(a, split_wgs, s);
    return 0;
}

// This translation unit's variant as a plain function named by the variant
// (declared in gemm_kernels.hpp): launch_tiled_<dtype><A K-major>_<B K-major>.
#if defined(LT_TILED_DT) && defined(LT_TILED_AK) && defined(LT_TILED_BK)
#define LT_CAT(dt, ak, bk) launch_tiled_##dt##ak##_##bk
#define LT_NAME(dt, ak, bk) LT_CAT(dt, ak, bk)
int LT_NAME(LT_TILED_DT, LT_TILED_AK, LT_TILED_BK)(const TiledArgs& a, int tile_m, int tile_n, int persist_grid,
                                                    void* stream) {
    return launch_variant<LT_TILED_DT, LT_TILED_AK != 0, LT_TILED_BK != 0>(a, tile_m, tile_n, persist_grid, stream);
}
#endif

}  // namespace lt
