// Host build of the kernels' compile-time layouts: prints every map the
// tiled kernel evaluates so the tests can check it against the layout algebra.
#include <cstdio>
#include <initializer_list>

#include "device_layout.hpp"

using namespace lt::dev;

template <int BK>
void dump_ktile() {
    using T = KTile<BK>;
    std::printf("ktile %d %d\n", BK, T::C);
    for (int row = 0; row < 256; ++row)
        for (int c = 0; c < T::C; ++c) std::printf("%d ", T::at(row, c));
    std::printf("\n");
}

// Per MFMA shape: operand (row, chunk), transposed-read (krow q=0, krow q=1,
// col) and output (row, col) for every lane.
template <int MF>
void dump_mfma() {
    using M = Mfma<MF>;
    std::printf("mfrag %d %d %d\n", MF, M::KSTEP, M::NACC);
    for (int l = 0; l < 64; ++l) std::printf("%d %d %d ", M::frag_row(l), M::frag_chunk(l), M::frag(l));
    std::printf("\nmtr %d\n", MF);
    for (int l = 0; l < 64; ++l) std::printf("%d %d %d ", M::tr_krow(l, 0), M::tr_krow(l, 1), M::tr_col(l));
    std::printf("\nmout %d\n", MF);
    for (int l = 0; l < 64; ++l)
        for (int v = 0; v < M::NACC; ++v) std::printf("%d %d ", M::out_row(l, v), M::out_col(l));
    std::printf("\n");
}

int main() {
    dump_ktile<32>();
    dump_ktile<64>();
    std::printf("mntile 64 32\n");
    for (int k = 0; k < 64; ++k)
        for (int c = 0; c < 32; ++c) std::printf("%d ", MNTile::at(k, c));
    std::printf("\nmntile 64 16\n");
    for (int k = 0; k < 64; ++k)
        for (int c = 0; c < 16; ++c) std::printf("%d ", MNTileW<16>::at(k, c));
    std::printf("\ntr\n");
    for (int l = 0; l < 64; ++l) std::printf("%d %d %d ", tr_krow(l, 0), tr_krow(l, 1), tr_col(l));
    std::printf("\ncopy\n");
    for (int i = 0; i < 4; ++i)
        for (int l = 0; l < 64; ++l) std::printf("%d ", kCopyTV(l + 64 * i));
    std::printf("\nfrag\n");
    for (int l = 0; l < 64; ++l) std::printf("%d ", kFragLane(l));
    std::printf("\nacc\n");
    for (int l = 0; l < 64; ++l)
        for (int v = 0; v < 16; ++v) std::printf("%d %d ", acc_row(l, v), acc_col(l));
    std::printf("\n");
    dump_mfma<32>();
    dump_mfma<16>();
    // staged D rows (128 rows of either width): unit, slot, swapped; the C tile
    for (int cpr : {8, 16}) {
        std::printf("staged_unit %d 128\n", cpr);
        for (int r = 0; r < 128; ++r)
            for (int u = 0; u < 2 * cpr; ++u)
                std::printf("%d ", cpr == 8 ? StagedRows<8>::unit(r, u) : StagedRows<16>::unit(r, u));
        std::printf("\nstaged_slot %d 128\n", cpr);
        for (int r = 0; r < 128; ++r)
            for (int q = 0; q < cpr; ++q)
                std::printf("%d %d ", cpr == 8 ? StagedRows<8>::slot(r, q) : StagedRows<16>::slot(r, q),
                            (int)(cpr == 8 ? StagedRows<8>::swapped(r) : StagedRows<16>::swapped(r)));
        std::printf("\n");
    }
    std::printf("staged_c 16 128\n");
    for (int r = 0; r < 128; ++r)
        for (int q = 0; q < 16; ++q) std::printf("%d %d ", StagedC::at(r, q), StagedC::chunk_at(r, q));
    std::printf("\n");
    return 0;
}
