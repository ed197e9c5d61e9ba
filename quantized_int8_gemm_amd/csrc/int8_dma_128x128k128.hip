// Tile configuration 128x128k128 of the multi-stage int8 kernel: 128 x 128 output tile, waves of 64 x 64, 128 k-bytes per stage, 2 LDS stages (64 KiB: two workgroups per CU).
// Stage rows of 128 bytes make every A (and [N,K] B) segment a whole
// 128-byte cache line.
#include "int8_dma_impl.h"

namespace qg {
hipError_t launch_dma_128x128k128(const Int8GemmArgs& a, bool bkm, int epi, int zp, hipStream_t s) {
    return dma::launch_shape<128, 128, 64, 64, 2, 128>(a, bkm, epi, zp, s);
}
}  // namespace qg
