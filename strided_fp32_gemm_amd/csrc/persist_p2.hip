// Instantiates the persistent short-k kernel for tile 2 of kPersistTiles.
#include "persist_kernel.hpp"

namespace sgemm {
void fill_persist_2(PersistTable &tab) { fill_persist<2>(tab); }
}  // namespace sgemm
