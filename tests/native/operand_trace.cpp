// Host build of the tiled kernel's copy addressing (tiled_config.hpp): for
// each case read from stdin, "cfg op kmaj ld rows row0" (cfg 0 = 256x256 with
// 4 waves, 1 = 256x128, 2 = 256x256 with 8 waves; op a or b), prints
//   "case OPI NW BK KSLICE_BYTES"
// and then, for every wave, lane and copy instruction i of that operand, the
// stored LDS chunk the copy fills and the byte offset, from the operand's
// base at the start of K slice 0, of the 16 bytes it reads.
#include <cstdio>
#include <cstring>

#include "tiled_config.hpp"

using namespace lt;

template <class Cf, bool KMAJ, int ROWS>
void trace(long long ld, int rows, int row0) {
    using O = Operand<Cf, KMAJ, ROWS>;
    std::printf("case %d %d %d %lld\n", O::OPI, Cf::NW, Cf::BK, (long long)O::kslice_bytes(ld));
    for (int w = 0; w < Cf::NW; ++w)
        for (int l = 0; l < 64; ++l)
            for (int i = 0; i < O::OPI; ++i)
                std::printf("%d %u ", O::stored_chunk(w, l, i), O::offset(ld, row0, rows, w, l, i));
    std::printf("\n");
}

template <template <bool, bool> class Cfg, int BN>
void dispatch(char op, int kmaj, long long ld, int rows, int row0) {
    // A is the M side (BM = 256 rows) and B the N side (BN rows); the other
    // operand's major-ness does not change this one's map.
    if (op == 'a') {
        if (kmaj) trace<Cfg<true, true>, true, 256>(ld, rows, row0);
        else trace<Cfg<false, true>, false, 256>(ld, rows, row0);
    } else {
        if (kmaj) trace<Cfg<true, true>, true, BN>(ld, rows, row0);
        else trace<Cfg<true, false>, false, BN>(ld, rows, row0);
    }
}

int main() {
    int cfg, kmaj, rows, row0;
    char op[8];
    long long ld;
    while (std::scanf("%d %7s %d %lld %d %d", &cfg, op, &kmaj, &ld, &rows, &row0) == 6) {
        if (cfg == 0) dispatch<Dp256, 256>(op[0], kmaj, ld, rows, row0);
        else if (cfg == 1) dispatch<Dp128, 128>(op[0], kmaj, ld, rows, row0);
        else dispatch<Split256, 256>(op[0], kmaj, ld, rows, row0);
    }
    return 0;
}
