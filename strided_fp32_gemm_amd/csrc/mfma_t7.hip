// Instantiates the MFMA kernel for tile 7 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_7(MfmaTable &tab) { fill_tile<7>(tab); }
}  // namespace sgemm
