// Instantiates the direct wavefront kernel for tile 2 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_2(WaveTable &tab) { fill_wave<2>(tab); }
}  // namespace sgemm
