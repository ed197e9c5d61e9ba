// Tile configuration 128x128k128 of the multi-stage int8 kernel: 128 x 128 output tile, waves of 64 x 64, 128 k-bytes per stage, 2 LDS stages (64 KiB: two workgroups per CU).
// Stage rows of 128 bytes make every A (and [N,K] B) segment a whole
// 128-byte cache line.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_128x128k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<128, 128, 64, 64, 2, 128>(a, bkm, epi, zp, s);
}
// Outputs of at most 256 tiles over a long K, split over K or not: three
// stages (96 KiB, one workgroup per CU, which such grids give anyway).
// Mid-sized M at K = N = 8192 (graph-timed, one box), split: M = 32 27.2 ->
// 24.5 us, M = 64 27.3 -> 25.1, M = 128 28.6 -> 27.0, M = 256 39.0 -> 32.8
// against two stages (four stages 26.2 / 26.2 / 26.8 / 32.4 us); unsplit,
// 129 to 256 tiles: M = 320 / 384 / 512 60.4 / 60.9 / 61.7 -> 43.4 / 46.0 /
// 48.5 us against the two-stage kernel.
hipError_t launch_dma_128x128k128_split(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_split<128, 128, 64, 64, 3, 128>(a, bkm, epi, zp, s);
}
}  // namespace qg
