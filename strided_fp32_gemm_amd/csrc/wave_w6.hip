// Instantiates the direct wavefront kernel for tile 6 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_6(WaveTable &tab) { fill_wave<6>(tab); }
}  // namespace sgemm
