// Instantiates the MFMA kernel for tile 5 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_5(MfmaTable &tab) { fill_tile<5>(tab); }
}  // namespace sgemm
