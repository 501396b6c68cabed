// Host build of the kernels' compile-time layouts: prints every map the
// tiled kernel evaluates so the tests can check it against the layout algebra.
#include <cstdio>

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

int main() {
    dump_ktile<32>();
    dump_ktile<64>();
    std::printf("mntile 64 32\n");
    for (int k = 0; k < 64; ++k)
        for (int c = 0; c < 32; ++c) std::printf("%d ", MNTile::at(k, c));
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
    return 0;
}
