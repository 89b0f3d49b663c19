// Instantiates the MFMA kernel for tile 12 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_12(MfmaTable &tab) { fill_tile<12>(tab); }
}  // namespace sgemm
