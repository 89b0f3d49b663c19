// Instantiates the persistent short-k kernel for tile 1 of kPersistTiles.
#include "persist_kernel.hpp"

namespace sgemm {
void fill_persist_1(PersistTable &tab) { fill_persist<1>(tab); }
}  // namespace sgemm
