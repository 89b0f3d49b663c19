// Instantiates the direct wavefront kernel for tile 0 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_0(WaveTable &tab) { fill_wave<0>(tab); }
}  // namespace sgemm
