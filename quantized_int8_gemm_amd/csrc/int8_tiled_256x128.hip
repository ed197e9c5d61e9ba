// Tile shape 256 x 128 (four waves of 128 x 64) of the tiled int8 kernel.
#include "int8_tiled_impl.h"

namespace qg {
hipError_t launch_tiled_256x128(const Int8GemmArgs& a, bool bkm, bool vec, int epi, int zp, hipStream_t s) {
    return tiled::launch_shape<256, 128, 128, 64, false>(a, bkm, vec, epi, zp, s);
}
}  // namespace qg
