// Instantiates the MFMA kernel for tile 1 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_1(MfmaTable &tab) { fill_tile<1>(tab); }
}  // namespace sgemm
