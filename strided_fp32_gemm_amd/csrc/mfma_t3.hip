// Instantiates the MFMA kernel for tile 3 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_3(MfmaTable &tab) { fill_tile<3>(tab); }
}  // namespace sgemm
