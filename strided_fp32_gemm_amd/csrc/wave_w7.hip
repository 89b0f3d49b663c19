// Instantiates the direct wavefront kernel for tile 7 of kWaveTiles.
#include "wave_kernel.hpp"

namespace sgemm {
void fill_wave_7(WaveTable &tab) { fill_wave<7>(tab); }
}  // namespace sgemm
