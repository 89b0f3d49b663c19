// Instantiates the MFMA kernel for tile 11 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_11(MfmaTable &tab) { fill_tile<11>(tab); }
}  // namespace sgemm
