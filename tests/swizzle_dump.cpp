// Prints the LDS swizzle maps of the gemm_bt kernels, evaluated by the
// kernels' own header functions on the host, for the CPU tests:
//   swz CPR SWZ row -> physical chunk offset XORed into every logical chunk
//   kouter row -> the pair swizzle of a K-outer row
//   epi CPR row chunk -> physical chunk of the parked output tile
#include <cstdio>

#include "dma_kernel.hpp"
#include "trans_kernel.hpp"

using namespace gbt;

int main() {
    for (int row = 0; row < 256; ++row) {
        std::printf("swz 8 0 %d %d\n", row, swz_row<8, 0>(row));
        std::printf("swz 8 1 %d %d\n", row, swz_row<8, 1>(row));
        std::printf("swz 8 2 %d %d\n", row, swz_row<8, 2>(row));
        std::printf("swz 4 0 %d %d\n", row, swz_row<4, 0>(row));
        std::printf("swz 4 1 %d %d\n", row, swz_row<4, 1>(row));
        std::printf("swz 4 2 %d %d\n", row, swz_row<4, 2>(row));
        std::printf("swz 16 0 %d %d\n", row, swz_row<16, 0>(row));
        std::printf("swz 16 1 %d %d\n", row, swz_row<16, 1>(row));
        std::printf("swz 16 2 %d %d\n", row, swz_row<16, 2>(row));
    }
    for (int row = 0; row < 64; ++row) std::printf("kouter %d %d\n", row, kouter_swz(row));
    const int cprs[] = {8, 12, 16, 24, 32, 64};
    for (int cpr : cprs)
        for (int row = 0; row < 64; ++row)
            for (int c = 0; c < cpr; ++c) std::printf("epi %d %d %d %d\n", cpr, row, c, epi_chunk(c, row, cpr));
    return 0;
}
