// Instantiates the MFMA kernel for tile 2 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_2(MfmaTable &tab) { fill_tile<2>(tab); }
}  // namespace sgemm
