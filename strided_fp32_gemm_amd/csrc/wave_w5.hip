// Instantiates the direct wavefront kernel for tile 5 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_5(WaveTable &tab) { fill_wave<5>(tab); }
}  // namespace sgemm
