// Block-tile configurations of the tiled GEMM and the address maps of its
// global-to-LDS copy, for device code and for the host (the tests evaluate
// these maps on the CPU and compare them with the layout algebra).
//
// A block tile is BM x BN outputs, K sliced BK deep; each slice of A (BM x
// BK) and of B (BK x BN) is staged in LDS in an S-stage ring. NWM x NWN waves
// each own a (BM/NWM) x (BN/NWN) wave tile and issue MF x MF x KSTEP MFMAs.
#pragma once

#include <cstdint>

#include "device_layout.hpp"

namespace lt {

template <int BM_, int BN_, int NWM_, int NWN_, int BK_, int S_, int MF_, bool AK_, bool BK_MAJ_>
struct TCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
    static constexpr int NWM = NWM_, NWN = NWN_, NW = NWM * NWN, NT = 64 * NW;
    static constexpr int TWM = BM / NWM, TWN = BN / NWN;      // wave tile
    using MFMA = dev::Mfma<MF_>;                              // MF x MF outputs per instruction
    static constexpr int MF = MF_;
    static constexpr int FM = TWM / MF, FN = TWN / MF;        // MFMA blocks per wave
    static constexpr int KS = BK / MFMA::KSTEP;               // MFMA K steps per slice
    static constexpr bool AK = AK_, BKM = BK_MAJ_;            // K-major operands?
    // One wave per SIMD (4 waves): the accumulators are held in AGPRs by
    // MFMAs written as inline asm, in an issue order fixed here rather than
    // by the compiler's scheduler.
    static constexpr bool EXPLICIT = NW == 4 && MF_ == 16;
    static constexpr int A_BYTES = BM * BK * 2;               // one slice of A
    static constexpr int B_BYTES = BN * BK * 2;               // one slice of B
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = S * STAGE;
    static constexpr int OPA = A_BYTES / 1024 / NW;           // copy instructions per wave for A
    static constexpr int OPB = B_BYTES / 1024 / NW;           // ... for B
    static constexpr int IPW = OPA + OPB;                     // ... per slice
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "copy must split evenly over waves");
    // Fragments are double-buffered over K steps: with an even step count per
    // slice every slice starts on buffer 0; with one step per slice the
    // buffer alternates with the slice's parity.
    static_assert(KS == 1 || KS % 2 == 0, "one K step per slice, or an even count");
    static_assert(IPW * (S - 1) < 64, "vmcnt counts at most 63 outstanding loads");
    static_assert(BM <= 256 && BN <= 256 && (BM == 256 || BM == 128) && (BN == 256 || BN == 128), "tile");
};

LT_HD constexpr int imin(int a, int b) { return a < b ? a : b; }

// An operand in memory as a (rows, K) layout, A as M x K and B as N x K:
// (rows, K):(ld, 1) when K-major, (rows, K):(1, ld) when M/N-major. Element
// (row, k) sits at offset(row, k) elements from the operand's base.
template <bool KMAJ>
struct OperandLayout {
    int64_t ld;
    LT_HD constexpr int64_t offset(int64_t row, int64_t k) const { return KMAJ ? row * ld + k : row + k * ld; }
};

// One operand of the block tile: A (ROWS = BM rows of M) or B (ROWS = BN rows
// of N), K-major or M/N-major.
//   K-major:   LDS tile KTile<BK>: ROWS rows of BK elements, XOR-swizzled
//              16-byte chunks; element (row, k) at row*ld + k in memory.
//   M/N-major: LDS tile MNTileW<ROWS/8>: BK rows of K, ROWS elements each;
//              element (row, k) at k*ld + row in memory.
// The copy's thread-value layout is lane -> stored chunk: instruction i of
// wave w writes stored chunks 64*(w*OPI + i) + lane, and the lane fetches
// the logical chunk the swizzle stores there (each swizzle is an
// involution inside a row).
template <class Cf, bool KMAJ, int ROWS>
struct Operand {
    static constexpr int OPI = ROWS * Cf::BK * 2 / 1024 / Cf::NW;   // copy instructions per wave
    static constexpr int W = ROWS / 8;                               // chunks per K row (M/N-major)
    using KT = dev::KTile<Cf::BK>;
    using MT = dev::MNTileW<W>;

    // Stored chunk that copy instruction i of (wave, lane) writes.
    LT_HD static constexpr int stored_chunk(int wave, int lane, int i) {
        return dev::kCopyTV(lane + 64 * (wave * OPI + i));
    }
    // Logical (row, K chunk) of the tile whose 16 bytes that copy fetches:
    // K-major: row of M/N and 8-element K chunk; M/N-major: K row and
    // 8-element chunk of M/N.
    LT_HD static constexpr int src_row(int wave, int lane, int i) {
        const int q = stored_chunk(wave, lane, i);
        return KMAJ ? q / KT::C : q / W;
    }
    LT_HD static constexpr int src_chunk(int wave, int lane, int i) {
        const int q = stored_chunk(wave, lane, i);
        return KMAJ ? KT::at(q / KT::C, q % KT::C) - KT::C * (q / KT::C) : MT::at(q / W, q % W) - W * (q / W);
    }
    // Byte offset of that source relative to the operand's base, for the K
    // slice that starts at k = 0 (a later slice adds kslice_bytes): the
    // operand layout evaluated at the copied chunk's first element, whose
    // coordinate is the block tile's origin (row0, 0) plus the chunk's place
    // in the tile -- local_tile of the operand, then the copy's partition of
    // the tile ("Layouts as Algebra", "The kernel, in three lines"). Rows
    // past the operand's extent `rows` (a ragged edge tile) are clamped to
    // its last row (last 8-element chunk): valid memory whose products land
    // only in outputs that are not stored.
    LT_HD static constexpr uint32_t offset(int64_t ld, int row0, int rows, int wave, int lane, int i) {
        const int r = src_row(wave, lane, i), c = src_chunk(wave, lane, i);
        const OperandLayout<KMAJ> L{ld};
        if (KMAJ) return (uint32_t)(L.offset(imin(row0 + r, rows - 1), 8 * c) * 2);
        return (uint32_t)(L.offset(imin(row0 + 8 * c, rows - 8), r) * 2);
    }
    // Bytes from the operand's base to the origin (row0, 0) of a block tile:
    // for an interior tile, offset(ld, row0, rows, ...) = tile_bytes(ld,
    // row0) + offset(ld, 0, ROWS, ...).
    LT_HD static constexpr int64_t tile_bytes(int64_t ld, int row0) {
        return OperandLayout<KMAJ>{ld}.offset(row0, 0) * 2;
    }
    // K offset, within its slice, of what that copy fetches.
    LT_HD static constexpr int kpos(int wave, int lane, int i) {
        return KMAJ ? 8 * src_chunk(wave, lane, i) : src_row(wave, lane, i);
    }
    LT_HD static constexpr int64_t kslice_bytes(int64_t ld) { return OperandLayout<KMAJ>{ld}.offset(0, Cf::BK) * 2; }
    // Bytes between consecutive K rows of the M/N-major LDS tile.
    static constexpr int KROW_BYTES = W * 16;
};

// The staged D store of the plain epilogue (D, and C for a 256x256
// data-parallel tile, through LDS for 16-byte row stores) runs in the
// persistent launches and in the data-parallel launch with K-major A and B
// (with M-/N-major operands the fragment offsets leave the data-parallel
// kernel no registers for it), never in the split launch. Its region lies
// beside a ring of ring_lds bytes: 32 KiB when the ring leaves that much of
// the 160 KiB a workgroup may hold, else 16 KiB. The persistent launch with
// C shares those 16 KiB with the next tile's C rows 192..255. The planner
// reports the launch's LDS from the same rule.
LT_HD constexpr bool staged_d_launch(bool persistent, bool data_parallel, bool a_kmajor, bool b_kmajor) {
    return persistent || (data_parallel && a_kmajor && b_kmajor);
}
LT_HD constexpr int staged_d_region(int ring_lds) { return 160 * 1024 - ring_lds >= 32 * 1024 ? 32 * 1024 : 16 * 1024; }
// LDS of one workgroup: the ring, then the larger of the staged region and
// (persistent with C) the 16 KiB of C rows 192..255
LT_HD constexpr int launch_lds_bytes(int ring_lds, bool staged, bool persistent_c) {
    const int extra = staged ? staged_d_region(ring_lds) : 0;
    return ring_lds + (persistent_c && extra < 16 * 1024 ? 16 * 1024 : extra);
}

// The configurations the planner launches.
//   Dp256:   256x256 block tile, 4 waves of 128x128 (one per SIMD), 2 stages
//            of 64 KiB; every operand major-ness.
//   Dp128:   256x128 block tile, 4 waves of 128x64, 3 stages of 48 KiB: twice
//            the tiles, for shapes whose 256x256 tiles leave a round of the
//            CUs part empty.
//   Dp128x128: 128x128 block tile, 4 waves of 64x64, 4 stages of 32 KiB:
//            four times the tiles of 256x256, for problems whose larger
//            tiles would leave most of the CUs idle (data-parallel only).
//   Split256: the split-remainder launch, 8 waves (4 x 2) of 64x128: its
//            fix-up adds the other segments' fp32 partials in registers, and
//            with 256 accumulators per lane that step spills.
template <bool AK, bool BKM>
using Dp256 = TCfg<256, 256, 2, 2, 64, 2, 16, AK, BKM>;
template <bool AK, bool BKM>
using Dp128 = TCfg<256, 128, 2, 2, 64, 3, 16, AK, BKM>;
template <bool AK, bool BKM>
using Dp128x128 = TCfg<128, 128, 2, 2, 64, 4, 16, AK, BKM>;
template <bool AK, bool BKM>
using Split256 = TCfg<256, 256, 4, 2, 64, 2, 16, AK, BKM>;

}  // namespace lt
