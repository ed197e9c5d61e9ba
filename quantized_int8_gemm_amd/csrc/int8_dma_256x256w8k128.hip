// Tile configuration 256x256w8k128 of the multi-stage int8 kernel: 256 x 256 output tile, eight waves of 128 x 64, 128 k-bytes per stage, 2 LDS stages (128 KiB).
// Stage rows of 128 bytes make every A (and [N,K] B) segment a whole
// 128-byte cache line.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_256x256w8k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<256, 256, 128, 64, 2, 128>(a, bkm, epi, zp, s);
}
}  // namespace qg
