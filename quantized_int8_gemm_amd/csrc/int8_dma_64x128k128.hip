// Tile configuration 64x128k128 of the multi-stage int8 kernel: 64 x 128
// output tile, waves of 32 x 64, 128 k-bytes per stage, 2 LDS stages (48 KiB).
// Small outputs get twice the workgroups of 128 x 128 tiles, each with half
// the multiplies between its first load and its last store.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_64x128k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<64, 128, 32, 64, 2, 128>(a, bkm, epi, zp, s);
}
}  // namespace qg
