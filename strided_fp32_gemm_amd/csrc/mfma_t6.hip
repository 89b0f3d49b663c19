// Instantiates the MFMA kernel for tile 6 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_6(MfmaTable &tab) { fill_tile<6>(tab); }
}  // namespace sgemm
