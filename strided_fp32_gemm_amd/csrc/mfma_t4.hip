// Instantiates the MFMA kernel for tile 4 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_4(MfmaTable &tab) { fill_tile<4>(tab); }
}  // namespace sgemm
