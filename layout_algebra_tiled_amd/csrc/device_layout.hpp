// Compile-time layouts for device code.
//
// The kernels address every tile and fragment through small Shape:Stride
// layouts whose extents and strides are constants, so that evaluating them at
// a lane or loop index folds into shifts, masks and immediate offsets ("3.5
// CUTLASS II — CuTe 레이아웃·텐서", 3.5.10: prefer compile-time integers;
// "CUTLASS and CuTe layouts", "Two programs": a static layout costs nothing to
// pass). The same definitions compile for the host so tests can enumerate
// them and compare with the host layout algebra.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define LT_HD __host__ __device__ __forceinline__
#else
#define LT_HD inline
#endif

namespace lt::dev {

// A flat layout with N leaves; offset = sum of colex digits times strides.
template <int N>
struct Flat {
    int s[N];
    int d[N];

    LT_HD constexpr int size() const {
        int n = 1;
        for (int i = 0; i < N; ++i) n *= s[i];
        return n;
    }
    LT_HD constexpr int cosize() const {
        int top = 0;
        for (int i = 0; i < N; ++i) top += (s[i] - 1) * d[i];
        return top + 1;
    }
    // Evaluate at a 1-D index (first leaf fastest).
    LT_HD constexpr int operator()(int idx) const {
        int off = 0;
        for (int i = 0; i < N; ++i) {
            off += (idx % s[i]) * d[i];
            idx /= s[i];
        }
        return off;
    }
};

// XOR swizzle on an offset: bits [shift, shift+bits) are XORed into bits
// [base, base+bits). A bijection of [0, 2^(shift+bits)) onto itself; composed
// after a row-major tile layout it permutes the 16-byte chunks of each row by
// the row index, so that a column of chunks spreads over all LDS banks.
struct Xor {
    int bits, base, shift;
    LT_HD constexpr int operator()(int off) const {
        return off ^ (((off >> shift) & ((1 << bits) - 1)) << base);
    }
};

// ---------------------------------------------------------------------------
// Layouts of the 256x256x64 tiled kernel (K-major operands).
//
// One LDS operand tile holds 256 rows (M or N) by 64 K elements of 16 bits:
// 256 rows of 8 chunks of 16 bytes. In chunk units the unswizzled tile is the
// row-major layout (8,256):(1,8) over (chunk, row); the stored tile is that
// layout followed by Xor{3,0,3}: chunk' = chunk ^ (row & 7).
// ---------------------------------------------------------------------------

constexpr Flat<2> kTileChunks{{8, 256}, {1, 8}};   // (chunk, row) -> chunk index
constexpr Xor kTileSwizzle{3, 0, 3};

// Stored (swizzled) chunk index of logical (row, chunk).
LT_HD constexpr int tile_chunk(int row, int chunk) { return kTileSwizzle(kTileChunks(chunk + 8 * row)); }

// Direct-to-LDS copy: one instruction of one wave writes 64 consecutive
// stored chunks (1 KiB); the thread-value layout is lane -> stored chunk
// lane, so a lane fetches the logical chunk that the swizzle puts there. The
// swizzle is an involution on (row, chunk), so the logical chunk is the
// stored one XORed with the row again.
constexpr Flat<2> kCopyTV{{64, 32}, {1, 64}};       // (lane, instr) -> stored chunk

// MFMA 32x32x16 operand fragment: lane l holds row l%32 and the 8 K values of
// chunk l/32 of a 16-wide K step: (row, half) layout (32,2):(1,32) over the
// lane index, i.e. lane -> (row = l % 32, kchunk = l / 32).
constexpr Flat<2> kFragLane{{32, 2}, {1, 32}};

// Output of one 32x32 MFMA block, per lane and accumulator register v:
// column (the B-operand row) = lane % 32, row = 8*(v/4) + 4*(lane/32) + v%4.
LT_HD constexpr int acc_row(int lane, int v) { return 8 * (v / 4) + 4 * (lane / 32) + (v % 4); }
LT_HD constexpr int acc_col(int lane) { return lane % 32; }

}  // namespace lt::dev
