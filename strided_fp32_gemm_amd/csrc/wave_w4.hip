// Instantiates the direct wavefront kernel for tile 4 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_4(WaveTable &tab) { fill_wave<4>(tab); }
}  // namespace sgemm
