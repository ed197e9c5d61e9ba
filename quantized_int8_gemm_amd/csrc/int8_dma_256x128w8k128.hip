// Tile configuration 256x128w8k128 of the multi-stage int8 kernel: 256 x 128 output tile, eight waves of 64 x 64, 128 k-bytes per stage, 3 LDS stages (144 KiB).
// Stage rows of 128 bytes make every A (and [N,K] B) segment a whole
// 128-byte cache line.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_256x128w8k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<256, 128, 64, 64, 3, 128>(a, bkm, epi, zp, s);
}
}  // namespace qg
