// Instantiates the MFMA kernel for tile 0 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_0(MfmaTable &tab) { fill_tile<0>(tab); }
}  // namespace sgemm
