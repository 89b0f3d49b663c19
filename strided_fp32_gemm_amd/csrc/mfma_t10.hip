// Instantiates the MFMA kernel for tile 10 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_10(MfmaTable &tab) { fill_tile<10>(tab); }
}  // namespace sgemm
