// abi.cpp -- the C ABI declared in include/sgemm_strided.h.
//
// Each entry point validates every size, stride and pointer before anything
// is enqueued (StaleyNET "GPU Implementation", section "Safety": a launch
// wrapper checks each size the kernel depends on and only then launches),
// plans the launch, and enqueues it on the caller's stream without
// synchronising (kael book ch. 09 "CUDA backend", section "Synchronous and
// asynchronous work").
#include "sgemm_strided.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstring>
#include <string>

#include "kernels.hpp"
#include "plan.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string &why) {
    g_last_error = why;
    return status;
}

// Compute units of the current device, cached per device id.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int current_cus(int &cus, std::string &why) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        why = std::string("hipGetDevice: ") + hipGetErrorString(e);
        return sgemm::kErrHip;
    }
    if (dev >= 0 && dev < kMaxDevices) {
        int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            cus = c;
            return sgemm::kOk;
        }
    }
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || v <= 0) {
        why = std::string("hipDeviceGetAttribute(multiprocessor count): ") + hipGetErrorString(e);
        return sgemm::kErrHip;
    }
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(v, std::memory_order_relaxed);
    cus = v;
    return sgemm::kOk;
}

sgemm::GemmArgs pack(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha, const float *A,
                     int64_t sA_batch, int64_t sA_row, int64_t sA_col, const float *B,
                     int64_t sB_batch, int64_t sB_row, int64_t sB_col, int accumulate, float *C,
                     int64_t sC_batch, int64_t sC_row, int64_t sC_col) {
    sgemm::GemmArgs a;
    a.batch = batch; a.m = m; a.n = n; a.k = k; a.alpha = alpha;
    a.A = reinterpret_cast<uintptr_t>(A); a.sA_batch = sA_batch; a.sA_row = sA_row; a.sA_col = sA_col;
    a.B = reinterpret_cast<uintptr_t>(B); a.sB_batch = sB_batch; a.sB_row = sB_row; a.sB_col = sB_col;
    a.accumulate = accumulate;
    a.C = reinterpret_cast<uintptr_t>(C); a.sC_batch = sC_batch; a.sC_row = sC_row; a.sC_col = sC_col;
    return a;
}

bool path_ok(int path) { return path >= SGEMM_PATH_AUTO && path <= SGEMM_PATH_GENERIC; }

}  // namespace

extern "C" {

int sgemm_strided_batched_path(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                               const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                               const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                               int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                               int64_t sC_col, int path, void *stream) {
    if (!path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "unknown path code");
    sgemm::GemmArgs a = pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                             sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col);
    std::string why;
    int st = sgemm::validate(a, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (batch == 0 || m == 0 || n == 0) return SGEMM_OK;
    int cus = 0;
    st = current_cus(cus, why);
    if (st != sgemm::kOk) return fail(st, why);
    sgemm::Plan plan;
    st = sgemm::make_plan(a, static_cast<sgemm::Family>(path), cus, plan, why);
    if (st != sgemm::kOk) return fail(st, why);
    st = sgemm::launch_plan(plan, static_cast<hipStream_t>(stream), why);
    if (st != sgemm::kOk) return fail(st, why);
    return SGEMM_OK;
}

int sgemm_strided_batched(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                          const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                          const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                          int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                          int64_t sC_col, void *stream) {
    return sgemm_strided_batched_path(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B,
                                      sB_batch, sB_row, sB_col, accumulate, C, sC_batch, sC_row,
                                      sC_col, SGEMM_PATH_AUTO, stream);
}

int sgemm_plan_describe(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                        const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                        const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                        int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                        int64_t sC_col, int path, int num_cus, sgemm_plan_info *info) {
    if (!path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "unknown path code");
    if (!info) return fail(SGEMM_ERR_NULL_POINTER, "info is NULL");
    sgemm::GemmArgs a = pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                             sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col);
    std::string why;
    int st = sgemm::validate(a, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (num_cus <= 0) {
        st = current_cus(num_cus, why);
        if (st != sgemm::kOk) return fail(st, why);
    }
    sgemm::Plan plan;
    st = sgemm::make_plan(a, static_cast<sgemm::Family>(path), num_cus, plan, why);
    if (st != sgemm::kOk) return fail(st, why);
    std::memset(info, 0, sizeof *info);
    info->path = plan.empty ? SGEMM_PATH_AUTO : static_cast<int>(plan.family);
    info->transposed = plan.transposed ? 1 : 0;
    if (plan.tile >= 0 && plan.persist) {
        const sgemm::PersistCfg &t = sgemm::kPersistTiles[plan.tile];
        info->tile_m = t.bm; info->tile_n = t.bn; info->tile_k = t.kmax;
        info->waves = t.waves();
    } else if (plan.tile >= 0 && plan.family == sgemm::Family::Wave) {
        const sgemm::WaveCfg &t = sgemm::kWaveTiles[plan.tile];
        info->tile_m = t.bm; info->tile_n = t.bn; info->tile_k = 16;
        info->waves = 1;
    } else if (plan.tile >= 0) {
        const sgemm::TileCfg &t = sgemm::kTiles[plan.tile];
        info->tile_m = t.bm; info->tile_n = t.bn; info->tile_k = t.bk;
        info->waves = t.waves();
    } else if (!plan.empty) {
        info->tile_m = 64; info->tile_n = 64; info->tile_k = 16; info->waves = 4;
    }
    info->vec_a = plan.vec_a;
    info->vec_b = plan.vec_b;
    info->a_kfast = plan.a_kfast ? 1 : 0;
    info->b_kfast = plan.b_kfast ? 1 : 0;
    info->launches = plan.empty ? 0 : 1;
    info->workgroups = plan.empty ? 0 : plan.workgroups;
    std::strncpy(info->kernel, plan.kernel_name.c_str(), sizeof info->kernel - 1);
    return SGEMM_OK;
}

const char *sgemm_status_string(int status) {
    switch (status) {
    case SGEMM_OK: return "SGEMM_OK";
    case SGEMM_ERR_INVALID_SIZE: return "SGEMM_ERR_INVALID_SIZE: negative batch, m, n or k";
    case SGEMM_ERR_INVALID_STRIDE: return "SGEMM_ERR_INVALID_STRIDE: negative stride";
    case SGEMM_ERR_NULL_POINTER: return "SGEMM_ERR_NULL_POINTER: required pointer is NULL";
    case SGEMM_ERR_C_ALIAS: return "SGEMM_ERR_C_ALIAS: C overlaps itself, A or B";
    case SGEMM_ERR_UNSUPPORTED: return "SGEMM_ERR_UNSUPPORTED: extent or offset overflow";
    case SGEMM_ERR_HIP: return "SGEMM_ERR_HIP: HIP runtime error";
    case SGEMM_ERR_INVALID_PATH: return "SGEMM_ERR_INVALID_PATH: unknown path code";
    default: return "unknown sgemm status";
    }
}

const char *sgemm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
