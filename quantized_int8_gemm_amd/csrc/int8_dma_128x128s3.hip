// Tile configuration 128x128s3 of the multi-stage int8 kernel: 128 x 128 output
// tile, waves of 64 x 64, 3 LDS stages.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_128x128s3(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<128, 128, 64, 64, 3>(a, bkm, epi, zp, s);
}
}  // namespace qg
