// Instantiates the direct wavefront kernel for tile 1 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_1(WaveTable &tab) { fill_wave<1>(tab); }
}  // namespace sgemm
