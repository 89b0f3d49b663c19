// Instantiates the MFMA kernel for tile 9 of kTiles (its launch-table row).
#include "mfma_kernel.hpp"

namespace sgemm {
void fill_tile_9(MfmaTable &tab) { fill_tile<9>(tab); }
}  // namespace sgemm
