// Tile configuration 64x128k128 of the multi-stage int8 kernel: 64 x 128
// output tile, waves of 32 x 64, 128 k-bytes per stage, 2 LDS stages (48 KiB).
// Small outputs get twice the workgroups of 128 x 128 tiles, each with half
// the multiplies between its first load and its last store.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_64x128k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<64, 128, 32, 64, 2, 128>(a, bkm, epi, zp, s);
}
// The same tile with three stages, split over K when a.splits > 1, for at
// most 64 rows over a long K: the 128x128 split tiles' workgroups with half
// their multiplies (rows 64 .. 127 of those tiles are empty).  A8W8 bf16 at
// N = K = 8192, graph-timed over 9 rotating weights: M = 17 / 32 / 64 23.8 /
// 24.5 / 25.0 -> 21.2 / 21.4 / 22.2 us (four stages 22.3 / 22.4 / 23.0).
hipError_t launch_dma_64x128k128_split(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_split<64, 128, 32, 64, 3, 128>(a, bkm, epi, zp, s);
}
}  // namespace qg
