// Tile configuration 256x128w8 of the multi-stage int8 kernel: 256 x 128 output
// tile, waves of 64 x 64, 4 LDS stages.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_256x128w8(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<256, 128, 64, 64, 4>(a, bkm, epi, zp, s);
}
}  // namespace qg
