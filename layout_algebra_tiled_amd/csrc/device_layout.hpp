// Compile-time layouts for device code.
//
// The kernels address every tile and fragment through small Shape:Stride
// layouts whose extents and strides are constants, so that evaluating them at
// a lane or loop index folds into shifts, masks and immediate offsets ("3.5
// CUTLASS II — CuTe 레이아웃·텐서", 3.5.10: prefer compile-time integers;
// "CUTLASS and CuTe layouts", "Two programs": a static layout costs nothing to
// pass). The same definitions compile for the host, so tests can enumerate
// them and compare with the host layout algebra.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
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
// [base, base+bits). A bijection of every aligned block of 2^(shift+bits)
// offsets onto itself (an involution).
struct Xor {
    int bits, base, shift;
    LT_HD constexpr int operator()(int off) const {
        return off ^ (((off >> shift) & ((1 << bits) - 1)) << base);
    }
};

LT_HD constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// ---------------------------------------------------------------------------
// Operand tiles of the 256-row block-tiled kernel, in units of 16-byte chunks
// (eight 16-bit elements).
//
// K-major tile: 256 rows (M or N) by BK elements of K, row-major chunks
// (C, 256):(1, C) with C = BK/8 chunks per row, then an XOR swizzle that keys
// the chunk on the 256-byte window the row falls in: a column of 16
// consecutive rows read by 16 lanes then covers all 64 banks. With R = 16/C
// rows per 256 bytes: chunk' = chunk ^ ((row / R) % C).
//
// M/N-major tile: BK rows of K by 256 elements of M or N (32 chunks per row),
// chunk' = chunk ^ (4*(row & 3) + 2*((row >> 3) & 1)). A transposed read
// covers, per 32 lanes, either four K rows by 64 bytes (32x32x16 fragments)
// or eight K rows (two sets of four, 8 apart) by 32 bytes (16x16x32); with
// the XOR both land in 16 distinct 16-byte bank groups of a 256-byte window.
// ---------------------------------------------------------------------------

template <int BK>
struct KTile {
    static constexpr int C = BK / 8;                 // chunks per row
    static constexpr int R = 16 / C;                 // rows per 256-byte window
    static constexpr Flat<2> chunks{{C, 256}, {1, C}};
    static constexpr Xor swz{ilog2(C), 0, ilog2(C) + ilog2(R)};
    // stored chunk index of logical (row, chunk)
    LT_HD static constexpr int at(int row, int chunk) { return swz(chunks(chunk + C * row)); }
};

// W chunks (8*W elements of M or N) per K row: 32 for a 256-wide block tile,
// 16 for a 128-wide one. The XOR term is at most 14, so it stays inside a
// row of either width.
template <int W>
struct MNTileW {
    static_assert(W == 16 || W == 32, "K rows of 128 or 256 elements");
    static constexpr int C = W;
    static constexpr Flat<2> chunks{{W, 64}, {1, W}};
    LT_HD static constexpr int at(int krow, int chunk) {
        return chunks(chunk + W * krow) ^ (4 * (krow & 3) + 2 * ((krow >> 3) & 1));
    }
};
using MNTile = MNTileW<32>;

// ---------------------------------------------------------------------------
// The algebra at compile time, on the one-leaf layouts the thread-value maps
// are built from ("Layouts as Algebra", "Complement", "Composition", "Divide
// is tiling"; "3.5 CUTLASS II", 3.5.6-3.5.8):
//   complement(s:d, M)   = (d, M/(s*d)) : (1, s*d)   (d*s divides M),
//   compose(A, n:1)      = A restricted to its first n offsets (n a product
//                          of A's leading leaves, or a divisor of the first),
//   logical_product(A, B) = (A, compose(complement(A, size(A)*cosize(B)), B)).
// Unit leaves (extent 1) are dropped: they add nothing to an offset.
// ---------------------------------------------------------------------------

template <int N>
LT_HD constexpr bool operator==(const Flat<N>& a, const Flat<N>& b) {
    for (int i = 0; i < N; ++i)
        if (a.s[i] != b.s[i] || a.d[i] != b.d[i]) return false;
    return true;
}

LT_HD constexpr Flat<1> leaf(int s, int d) { return Flat<1>{{s}, {d}}; }

LT_HD constexpr Flat<2> complement(const Flat<1>& a, int M) {
    return Flat<2>{{a.d[0], M / (a.s[0] * a.d[0])}, {1, a.s[0] * a.d[0]}};
}

// A restricted to its first n offsets (B = n:1).
template <int N>
LT_HD constexpr Flat<N> compose(const Flat<N>& a, const Flat<1>& b) {
    Flat<N> r = a;
    int left = b.s[0];
    for (int i = 0; i < N; ++i) {
        const int take = left >= a.s[i] ? a.s[i] : left;
        r.s[i] = take < 1 ? 1 : take;
        left = take >= 1 ? left / r.s[i] : 1;
    }
    return r;
}

template <int N, int M>
LT_HD constexpr Flat<N + M> concat(const Flat<N>& a, const Flat<M>& b) {
    Flat<N + M> r{};
    for (int i = 0; i < N; ++i) r.s[i] = a.s[i], r.d[i] = a.d[i];
    for (int i = 0; i < M; ++i) r.s[N + i] = b.s[i], r.d[N + i] = b.d[i];
    return r;
}

// The leaves of extent > 1, in order, padded with unit leaves to NOUT.
template <int NOUT, int N>
LT_HD constexpr Flat<NOUT> drop_unit(const Flat<N>& a) {
    Flat<NOUT> r{};
    int k = 0;
    for (int i = 0; i < N; ++i)
        if (a.s[i] > 1 && k < NOUT) r.s[k] = a.s[i], r.d[k] = a.d[i], ++k;
    for (; k < NOUT; ++k) r.s[k] = 1, r.d[k] = 0;
    return r;
}

LT_HD constexpr Flat<3> logical_product(const Flat<1>& a, const Flat<1>& b) {
    const int m = a.s[0] * (b.cosize());
    return concat(a, compose(complement(a, m), b));
}

// Thread-value layouts of one mode ("Layouts as Algebra", "The threads are a
// layout too"): with T threads and V values per thread,
//   interleaved = logical_product(T:1, V:1) = (T,V):(1,T) -- on one step the
//                 threads take T consecutive offsets (a coalesced access);
//   blocked     = logical_product(V:1, T:1), modes swapped, = (T,V):(V,1) --
//                 each thread owns a run of V.
// Both are built here by the product above; the host library builds the
// same layouts through its own complement and composition
// (lt_make_tv_layout), and the tests compare the two.
LT_HD constexpr Flat<2> tv_interleaved(int T, int V) {
    return drop_unit<2>(logical_product(leaf(T, 1), leaf(V, 1)));
}
LT_HD constexpr Flat<2> tv_blocked(int T, int V) {
    const Flat<2> vt = drop_unit<2>(logical_product(leaf(V, 1), leaf(T, 1)));
    return Flat<2>{{vt.s[1], vt.s[0]}, {vt.d[1], vt.d[0]}};
}
static_assert(tv_interleaved(64, 1024) == Flat<2>{{64, 1024}, {1, 64}}, "interleaved closed form");
static_assert(tv_interleaved(16, 4) == Flat<2>{{16, 4}, {1, 16}}, "interleaved closed form");
static_assert(tv_blocked(64, 8) == Flat<2>{{64, 8}, {8, 1}}, "blocked closed form");

// Direct-to-LDS copy: one instruction of one wave writes 64 consecutive
// stored chunks (1 KiB); the thread-value layout is lane -> stored chunk, so a
// lane fetches the logical chunk that the swizzle puts there. Both swizzles
// are involutions on (row, chunk), so the logical chunk is the stored one
// swizzled again. 64 lanes interleaved over the copy instructions (values).
constexpr Flat<2> kCopyTV = tv_interleaved(64, 1 << 10);   // (lane, instr) -> stored chunk

// MFMA 32x32x16 operand fragment: lane l holds row l%32 and K values
// 8*(l/32) .. 8*(l/32)+7 of a 16-deep K step: (row, half) = (32,2):(1,32),
// the interleaved split of the 64 lanes over the 32 rows.
constexpr Flat<2> kFragLane = tv_interleaved(32, 2);

// Transposed LDS read (ds_read_b64_tr_b16), measured on gfx950: inside each
// group of 16 lanes, lane i receives as element e the (i % 4)-th 16-bit value
// of the 8-byte block addressed by lane 4e + i/4 of its group. To hand lane
// (group g, index i) the MFMA fragment values K = 8*(g/2) + 4q + e of row
// 16*(g%2) + i, lane j of group g points at K row 8*(g/2) + 4q + j/4 and
// columns 16*(g%2) + 4*(j%4) .. +3.
LT_HD constexpr int tr_krow(int lane, int q) { return 8 * (lane >> 5) + 4 * q + ((lane & 15) >> 2); }
LT_HD constexpr int tr_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }

// Output of one 32x32 MFMA block, per lane and accumulator register v:
// column (the B-operand row) = lane % 32, row = 8*(v/4) + 4*(lane/32) + v%4.
LT_HD constexpr int acc_row(int lane, int v) { return 8 * (v / 4) + 4 * (lane / 32) + (v % 4); }
LT_HD constexpr int acc_col(int lane) { return lane % 32; }

// The same maps for either MFMA shape the block-tiled kernel uses, MF x MF
// outputs per instruction: 32x32x16 (K step 16) or 16x16x32 (K step 32).
//   operand: lane l holds row l % MF and the 8 K values of chunk l / MF of
//            the K step ((MF, 64/MF):(1, MF));
//   transposed read: lane j of 16-lane group g points at K row
//            8*(l/MF) + 4q + (j/4), columns 16*((l/16) % (MF/16)) + 4*(j%4);
//   output:  register v of lane l is row 8*(v/4) + 4*(l/MF) + v%4 (the B
//            operand's row) and column l % MF; MF*MF/64 registers per lane.
template <int MF>
struct Mfma {
    static_assert(MF == 32 || MF == 16, "MFMA shape 32x32x16 or 16x16x32");
    static constexpr int KSTEP = 512 / MF;         // K per instruction
    static constexpr int CHUNKS = KSTEP / 8;       // 16-byte K chunks per step
    static constexpr int NACC = MF * MF / 64;      // accumulator registers per lane
    static constexpr Flat<2> frag = tv_interleaved(MF, 64 / MF);   // lane -> (row, K chunk)
    LT_HD static constexpr int frag_row(int lane) { return lane % MF; }
    LT_HD static constexpr int frag_chunk(int lane) { return lane / MF; }
    LT_HD static constexpr int tr_krow(int lane, int q) { return 8 * (lane / MF) + 4 * q + ((lane & 15) >> 2); }
    LT_HD static constexpr int tr_col(int lane) { return 16 * ((lane >> 4) % (MF / 16)) + 4 * (lane & 3); }
    LT_HD static constexpr int out_row(int lane, int v) { return 8 * (v / 4) + 4 * (lane / MF) + (v % 4); }
    LT_HD static constexpr int out_col(int lane) { return lane % MF; }
};

// Rows of the staged D store in LDS: rows of CPR 16-byte chunks (RB = 16 *
// CPR bytes), row after row. The accumulators write 8 bytes per lane, one
// 8-byte unit u (of 2*CPR) of each of 16 consecutive rows per quarter-wave;
// unit u of row r sits at unit u ^ g(r) of its row, with g(r) = r mod 16
// for 128-byte rows and 2 (r mod 16) + ((r / 8) mod 2) for 256-byte rows.
// Then the 16 rows' copies of a unit fall in 16 distinct 8-byte bank pairs
// of a 128-byte (32-bank) window, and a half-wave's 32 writes (two units
// each in 16 rows) in 32 distinct pairs of a 256-byte window, whichever of
// the two the LDS serves per cycle. A 16-byte read of chunk q finds units
// 2q and 2q+1 together in slot q ^ (g(r) / 2), in swapped order when g(r)
// is odd; the 16 (or 8) lanes reading one row (two 128-byte rows) reach
// distinct slots.
template <int CPR>
struct StagedRows {
    static_assert(CPR == 8 || CPR == 16, "rows of 128 or 256 bytes");
    LT_HD static constexpr int g(int r) { return CPR == 8 ? (r & 15) : 2 * (r & 15) + ((r >> 3) & 1); }
    // byte offset of 8-byte unit u of row r
    LT_HD static constexpr int unit(int r, int u) { return 8 * (2 * CPR * r + (u ^ g(r))); }
    // byte offset of the 16-byte slot holding chunk q of row r
    LT_HD static constexpr int slot(int r, int q) { return 16 * (CPR * r + (q ^ (g(r) >> 1))); }
    LT_HD static constexpr bool swapped(int r) { return (g(r) & 1) != 0; }
};

// The C tile of the staged store with C, 256-byte rows copied in whole
// 16-byte chunks by direct-to-LDS copies: chunk q of row r at slot q ^ (r
// mod 16). chunk_at inverts it: the chunk a copy writing slot pos of row r
// fetches. The accumulators' 8-byte reads of a half-wave (two units of 16
// rows) reach 32 distinct bank pairs of a 256-byte window.
struct StagedC {
    LT_HD static constexpr int at(int r, int q) { return 16 * (16 * r + (q ^ (r & 15))); }
    LT_HD static constexpr int chunk_at(int r, int pos) { return pos ^ (r & 15); }
};

}  // namespace lt::dev
