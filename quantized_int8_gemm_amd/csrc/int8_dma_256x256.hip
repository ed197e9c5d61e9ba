// Tile configuration 256x256 of the multi-stage int8 kernel: 256 x 256 output
// tile, waves of 128 x 128, 4 LDS stages.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_256x256(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<256, 256, 128, 128, 4>(a, bkm, epi, zp, s);
}
}  // namespace qg
