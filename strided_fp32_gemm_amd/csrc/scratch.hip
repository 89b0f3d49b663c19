// scratch.hip -- the allocation-free squared-distance entry point.
//
// sgemm_pairwise_sqdist needs batch*m + nY*n floats of device memory for the
// two norm vectors it adds in its epilogue, which the caller brings in as a
// workspace.  Callers that cannot allocate device memory (code under graph
// capture, tight serving loops, harnesses that forbid allocation) use
// sgemm_pairwise_sqdist_noalloc instead: the norms go to a fixed array in the
// library's own device memory, `scratch`, of kScratchFloats floats.  Every GPU
// the library runs on holds its own copy of the array (4 MiB) from the time the
// code object is loaded until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device array, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever handed to kernels.
//
// Every call on one GPU shares that GPU's array.  Nothing in it has to start
// at zero: the norm launches overwrite every float the product then reads.
// Calls that overlap in time on one GPU (two streams, or two host threads)
// race on the array; a caller that overlaps calls must order them (same
// stream, or events).
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "entry.hpp"
#include "sgemm_strided.h"

namespace {

constexpr long long kScratchFloats = SGEMM_SCRATCH_FLOATS;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device id, once looked up

}  // namespace

static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

// Device address of the current device's `scratch`, looked up on the first
// call on each device with that device current.
int scratch_for_current_device(float **out, std::string &why) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        why = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return SGEMM_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        why = "device id " + std::to_string(dev) + " is beyond the scratch table's " +
              std::to_string(kMaxDevices) + " devices";
        return SGEMM_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            why = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
            return SGEMM_ERR_HIP;
        }
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return SGEMM_OK;
}

}  // namespace

extern "C" int sgemm_pairwise_sqdist_noalloc(int64_t batch, int64_t m, int64_t n, int64_t k, const float *X,
                                             int64_t sX_batch, int64_t sX_row, int64_t sX_col, const float *Y,
                                             int64_t sY_batch, int64_t sY_row, int64_t sY_col, float *D,
                                             int64_t sD_batch, int64_t sD_row, int64_t sD_col, void *stream) {
    return sgemm::pairwise_sqdist(batch, m, n, k, X, sX_batch, sX_row, sX_col, Y, sY_batch, sY_row, sY_col, D,
                                  sD_batch, sD_row, sD_col, nullptr, 0, kScratchFloats,
                                  scratch_for_current_device, stream);
}
