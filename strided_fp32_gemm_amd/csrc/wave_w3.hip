// Instantiates the direct wavefront kernel for tile 3 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_3(WaveTable &tab) { fill_wave<3>(tab); }
}  // namespace sgemm
