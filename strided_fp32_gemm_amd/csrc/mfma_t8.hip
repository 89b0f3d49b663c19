// Instantiates the MFMA kernel for tile 8 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_8(MfmaTable &tab) { fill_tile<8>(tab); }
}  // namespace sgemm
