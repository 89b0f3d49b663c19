// Instantiates the persistent short-k kernel for tile 0 of kPersistTiles.
#include "persist_kernel.hpp"

namespace sgemm {
void fill_persist_0(PersistTable &tab) { fill_persist<0>(tab); }
}  // namespace sgemm
