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

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <string>

#include "attention.hpp"
#include "entry.hpp"
#include "kernels.hpp"
#include "plan.hpp"
#include "splitk.hpp"

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
    a.beta = accumulate ? 1.0f : 0.0f;
    a.C = reinterpret_cast<uintptr_t>(C); a.sC_batch = sC_batch; a.sC_row = sC_row; a.sC_col = sC_col;
    return a;
}

bool path_ok(int path) { return path >= SGEMM_PATH_AUTO && path <= SGEMM_PATH_GENERIC; }

uint32_t bits(float x) {
    uint32_t u;
    std::memcpy(&u, &x, sizeof u);
    return u;
}

// Every field of two argument sets equal (floats bit for bit).
bool same_args(const sgemm::GemmArgs &x, const sgemm::GemmArgs &y) {
    return x.batch == y.batch && x.m == y.m && x.n == y.n && x.k == y.k && bits(x.alpha) == bits(y.alpha) &&
           x.A == y.A && x.sA_batch == y.sA_batch && x.sA_row == y.sA_row && x.sA_col == y.sA_col &&
           x.B == y.B && x.sB_batch == y.sB_batch && x.sB_row == y.sB_row && x.sB_col == y.sB_col &&
           x.accumulate == y.accumulate && x.C == y.C && x.sC_batch == y.sC_batch && x.sC_row == y.sC_row &&
           x.sC_col == y.sC_col && bits(x.beta) == bits(y.beta) && x.row_add == y.row_add &&
           x.sR_batch == y.sR_batch && x.sR_row == y.sR_row && x.col_add == y.col_add &&
           x.sL_batch == y.sL_batch && x.sL_col == y.sL_col && x.inner == y.inner && x.sA_inner == y.sA_inner &&
           x.gA == y.gA && x.sB_inner == y.sB_inner && x.gB == y.gB && x.sC_inner == y.sC_inner;
}

// The plans of the last few products planned on this thread.  A plan is a
// function of the arguments, the path and the CU count alone, and only
// arguments that validated are stored, so a call that repeats one (the same
// tensors in a loop) skips validation and planning on the host, about 2.5 us.
// Tuning overrides in the environment (which the planner reads) bypass it.
struct CachedPlan {
    sgemm::GemmArgs args{};
    int path = -1, cus = 0;
    sgemm::Plan plan;
};
constexpr int kPlanCacheSize = 8;
thread_local CachedPlan g_plans[kPlanCacheSize];
thread_local int g_plan_next = 0;

struct CachedSplit {
    sgemm::GemmArgs args{};
    int cus = 0;
    uintptr_t workspace = 0;
    int64_t floats = -1;
    sgemm::SplitPlan plan;
};
thread_local CachedSplit g_splits[kPlanCacheSize];
thread_local int g_split_next = 0;

bool planner_overrides() {
    return std::getenv("SGEMM_FORCE_TILE") || std::getenv("SGEMM_PERSIST_WGS") || std::getenv("SGEMM_WAVE_SPLIT");
}

// Validate, plan and enqueue one product.
int run_gemm(const sgemm::GemmArgs &a, int path, void *stream) {
    std::string why;
    int cus = 0;
    const bool cacheable = !planner_overrides();
    if (cacheable && current_cus(cus, why) == sgemm::kOk) {
        for (const CachedPlan &c : g_plans)
            if (c.path == path && c.cus == cus && same_args(c.args, a)) {
                const int st = sgemm::launch_plan(c.plan, static_cast<hipStream_t>(stream), why);
                return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
            }
    }
    int st = sgemm::validate(a, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (a.batch == 0 || a.m == 0 || a.n == 0) return SGEMM_OK;
    st = current_cus(cus, why);
    if (st != sgemm::kOk) return fail(st, why);
    sgemm::Plan plan;
    st = sgemm::make_plan(a, static_cast<sgemm::Family>(path), cus, plan, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (cacheable) {
        CachedPlan &c = g_plans[g_plan_next];
        g_plan_next = (g_plan_next + 1) % kPlanCacheSize;
        c.args = a;
        c.path = path;
        c.cus = cus;
        c.plan = plan;
    }
    st = sgemm::launch_plan(plan, static_cast<hipStream_t>(stream), why);
    if (st != sgemm::kOk) return fail(st, why);
    return SGEMM_OK;
}

bool ranges_meet(uintptr_t p, int64_t p_floats, uintptr_t q, int64_t q_floats) {
    return p < q + 4u * uintptr_t(q_floats) && q < p + 4u * uintptr_t(p_floats);
}

// True if a [e0][e1] view with strides (s0, s1) gives every element its own
// address: sorted by stride, each axis of extent > 1 must step past all the
// smaller axes reach.
bool distinct_2d(int64_t e0, int64_t s0, int64_t e1, int64_t s1) {
    if (s0 > s1) { std::swap(e0, e1); std::swap(s0, s1); }
    int64_t reach = 0;
    if (e0 > 1) {
        if (s0 <= reach) return false;
        reach = (e0 - 1) * s0;
    }
    return e1 <= 1 || s1 > reach;
}

// Elements spanned by a [batch][count][len] view (0 if empty), or -1 on overflow.
int64_t span3(int64_t e0, int64_t s0, int64_t e1, int64_t s1, int64_t e2, int64_t s2) {
    if (e0 == 0 || e1 == 0 || e2 == 0) return 0;
    int64_t a, b, c, t, r;
    if (__builtin_mul_overflow(e0 - 1, s0, &a) || __builtin_mul_overflow(e1 - 1, s1, &b) ||
        __builtin_mul_overflow(e2 - 1, s2, &c) || __builtin_add_overflow(a, b, &t) ||
        __builtin_add_overflow(t, c, &r) || r == INT64_MAX)
        return -1;
    return r + 1;
}

// Two batch levels packed into GemmArgs (flat batch = nb_outer * nb_inner).
int pack2(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k, float alpha,
          const float *A, int64_t sA_outer, int64_t sA_inner, int64_t gA, int64_t sA_row,
          int64_t sA_col, const float *B, int64_t sB_outer, int64_t sB_inner, int64_t gB,
          int64_t sB_row, int64_t sB_col, int accumulate, float *C, int64_t sC_outer,
          int64_t sC_inner, int64_t sC_row, int64_t sC_col, sgemm::GemmArgs &a) {
    if (nb_outer < 0 || nb_inner < 1 || gA < 1 || gB < 1)
        return fail(SGEMM_ERR_INVALID_SIZE, "nb_outer must be >= 0; nb_inner, gA and gB >= 1");
    int64_t batch;
    if (__builtin_mul_overflow(nb_outer, nb_inner, &batch))
        return fail(SGEMM_ERR_UNSUPPORTED, "nb_outer*nb_inner overflows int64");
    a = pack(batch, m, n, k, alpha, A, sA_outer, sA_row, sA_col, B, sB_outer, sB_row, sB_col,
             accumulate, C, sC_outer, sC_row, sC_col);
    a.inner = nb_inner;
    a.sA_inner = sA_inner; a.gA = gA;
    a.sB_inner = sB_inner; a.gB = gB;
    a.sC_inner = sC_inner;
    return SGEMM_OK;
}

sgemm::AttnCall pack_attention(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                               float alpha, int causal, const float *Q, int64_t sQ_outer,
                               int64_t sQ_inner, int64_t sQ_row, int64_t sQ_col, const float *K,
                               int64_t sK_outer, int64_t sK_inner, int64_t g, int64_t sK_row,
                               int64_t sK_col, const float *V, int64_t sV_outer, int64_t sV_inner,
                               int64_t sV_row, int64_t sV_col, float *O, int64_t sO_outer,
                               int64_t sO_inner, int64_t sO_row, int64_t sO_col) {
    sgemm::AttnCall c;
    c.nb_outer = nb_outer; c.nb_inner = nb_inner; c.tq = tq; c.tk = tk; c.d = d; c.g = g;
    c.alpha = alpha; c.causal = causal;
    c.Q = reinterpret_cast<uintptr_t>(Q); c.K = reinterpret_cast<uintptr_t>(K);
    c.V = reinterpret_cast<uintptr_t>(V); c.O = reinterpret_cast<uintptr_t>(O);
    const int64_t sq[4] = {sQ_outer, sQ_inner, sQ_row, sQ_col}, sk[4] = {sK_outer, sK_inner, sK_row, sK_col},
                  sv[4] = {sV_outer, sV_inner, sV_row, sV_col}, so[4] = {sO_outer, sO_inner, sO_row, sO_col};
    for (int a = 0; a < 4; ++a) { c.sQ[a] = sq[a]; c.sK[a] = sk[a]; c.sV[a] = sv[a]; c.sO[a] = so[a]; }
    return c;
}

bool attention_path_ok(int path) {
    return path == SGEMM_PATH_AUTO || path == SGEMM_PATH_MFMA || path == SGEMM_PATH_GENERIC;
}

int plan_attention(const sgemm::AttnCall &c, int path, sgemm::AttnPlan &plan) {
    if (!attention_path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "attention runs on AUTO, MFMA or GENERIC");
    std::string why;
    int st = sgemm::validate_attention(c, why);
    if (st != sgemm::kOk) return fail(st, why);
    st = sgemm::make_attention_plan(c, static_cast<sgemm::AttnPath>(path), plan, why);
    return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
}

}  // namespace

extern "C" {

int sgemm_attention_path(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                         float alpha, int causal, const float *Q, int64_t sQ_outer, int64_t sQ_inner,
                         int64_t sQ_row, int64_t sQ_col, const float *K, int64_t sK_outer,
                         int64_t sK_inner, int64_t g, int64_t sK_row, int64_t sK_col, const float *V,
                         int64_t sV_outer, int64_t sV_inner, int64_t sV_row, int64_t sV_col, float *O,
                         int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col, int path,
                         void *stream) {
    sgemm::AttnPlan plan;
    int st = plan_attention(pack_attention(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer,
                                           sQ_inner, sQ_row, sQ_col, K, sK_outer, sK_inner, g, sK_row,
                                           sK_col, V, sV_outer, sV_inner, sV_row, sV_col, O, sO_outer,
                                           sO_inner, sO_row, sO_col),
                            path, plan);
    if (st != SGEMM_OK) return st;
    std::string why;
    st = sgemm::launch_attention(plan, static_cast<hipStream_t>(stream), why);
    return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
}

int sgemm_attention(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d, float alpha,
                    int causal, const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row,
                    int64_t sQ_col, const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                    int64_t sK_row, int64_t sK_col, const float *V, int64_t sV_outer, int64_t sV_inner,
                    int64_t sV_row, int64_t sV_col, float *O, int64_t sO_outer, int64_t sO_inner,
                    int64_t sO_row, int64_t sO_col, void *stream) {
    return sgemm_attention_path(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner,
                                sQ_row, sQ_col, K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer,
                                sV_inner, sV_row, sV_col, O, sO_outer, sO_inner, sO_row, sO_col,
                                SGEMM_PATH_AUTO, stream);
}

int sgemm_attention_splitkv(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d, float alpha,
                            int causal, const float *Q, int64_t sQ_outer, int64_t sQ_inner, int64_t sQ_row,
                            int64_t sQ_col, const float *K, int64_t sK_outer, int64_t sK_inner, int64_t g,
                            int64_t sK_row, int64_t sK_col, const float *V, int64_t sV_outer, int64_t sV_inner,
                            int64_t sV_row, int64_t sV_col, float *O, int64_t sO_outer, int64_t sO_inner,
                            int64_t sO_row, int64_t sO_col, float *workspace, int64_t workspace_floats,
                            void *stream) {
    const sgemm::AttnCall c = pack_attention(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner,
                                             sQ_row, sQ_col, K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer,
                                             sV_inner, sV_row, sV_col, O, sO_outer, sO_inner, sO_row, sO_col);
    std::string why;
    int st = sgemm::validate_attention(c, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (workspace_floats < 0) return fail(SGEMM_ERR_INVALID_SIZE, "workspace_floats must be >= 0");
    if (workspace_floats > 0 && !workspace)
        return fail(SGEMM_ERR_NULL_POINTER, "workspace is NULL but workspace_floats > 0");
    if (sgemm::attention_overlaps(c, reinterpret_cast<uintptr_t>(workspace), workspace_floats))
        return fail(SGEMM_ERR_C_ALIAS, "workspace overlaps Q, K, V or O");
    int cus = 0;
    st = current_cus(cus, why);
    if (st != sgemm::kOk) return fail(st, why);
    sgemm::SplitKvPlan sp;
    sgemm::make_splitkv_plan(c, cus, reinterpret_cast<uintptr_t>(workspace), workspace ? workspace_floats : 0, sp);
    if (sp.chunks > 0) {
        st = sgemm::launch_splitkv(sp, static_cast<hipStream_t>(stream), why);
        return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
    }
    sgemm::AttnPlan plan;
    st = plan_attention(c, SGEMM_PATH_AUTO, plan);
    if (st != SGEMM_OK) return st;
    st = sgemm::launch_attention(plan, static_cast<hipStream_t>(stream), why);
    return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
}

int sgemm_attention_splitkv_describe(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                                     float alpha, int causal, const float *Q, int64_t sQ_outer, int64_t sQ_inner,
                                     int64_t sQ_row, int64_t sQ_col, const float *K, int64_t sK_outer,
                                     int64_t sK_inner, int64_t g, int64_t sK_row, int64_t sK_col, const float *V,
                                     int64_t sV_outer, int64_t sV_inner, int64_t sV_row, int64_t sV_col, float *O,
                                     int64_t sO_outer, int64_t sO_inner, int64_t sO_row, int64_t sO_col,
                                     int64_t workspace_floats, int num_cus, int64_t *chunks, int64_t *chunk_keys,
                                     int64_t *floats_used) {
    if (!chunks || !chunk_keys || !floats_used) return fail(SGEMM_ERR_NULL_POINTER, "an output pointer is NULL");
    const sgemm::AttnCall c = pack_attention(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner,
                                             sQ_row, sQ_col, K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer,
                                             sV_inner, sV_row, sV_col, O, sO_outer, sO_inner, sO_row, sO_col);
    std::string why;
    int st = sgemm::validate_attention(c, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (num_cus <= 0) {
        st = current_cus(num_cus, why);
        if (st != sgemm::kOk) return fail(st, why);
    }
    sgemm::SplitKvPlan sp;
    sgemm::make_splitkv_plan(c, num_cus, 0, workspace_floats, sp);
    *chunks = sp.chunks;
    *chunk_keys = sp.chunk_keys;
    *floats_used = sp.workspace_floats;
    return SGEMM_OK;
}

int sgemm_attention_describe(int64_t nb_outer, int64_t nb_inner, int64_t tq, int64_t tk, int64_t d,
                             float alpha, int causal, const float *Q, int64_t sQ_outer,
                             int64_t sQ_inner, int64_t sQ_row, int64_t sQ_col, const float *K,
                             int64_t sK_outer, int64_t sK_inner, int64_t g, int64_t sK_row,
                             int64_t sK_col, const float *V, int64_t sV_outer, int64_t sV_inner,
                             int64_t sV_row, int64_t sV_col, float *O, int64_t sO_outer,
                             int64_t sO_inner, int64_t sO_row, int64_t sO_col, int path,
                             sgemm_plan_info *info) {
    if (!info) return fail(SGEMM_ERR_NULL_POINTER, "info is NULL");
    sgemm::AttnPlan plan;
    int st = plan_attention(pack_attention(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer,
                                           sQ_inner, sQ_row, sQ_col, K, sK_outer, sK_inner, g, sK_row,
                                           sK_col, V, sV_outer, sV_inner, sV_row, sV_col, O, sO_outer,
                                           sO_inner, sO_row, sO_col),
                            path, plan);
    if (st != SGEMM_OK) return st;
    std::memset(info, 0, sizeof *info);
    info->path = plan.empty ? SGEMM_PATH_AUTO
                            : (plan.path == sgemm::AttnPath::Mfma ? SGEMM_PATH_MFMA : SGEMM_PATH_GENERIC);
    if (!plan.empty && plan.path == sgemm::AttnPath::Mfma) {
        info->tile_m = plan.waves * 16; info->tile_n = 64; info->tile_k = 64;
        info->vec_a = 4; info->vec_b = 4;
    } else if (!plan.empty) {
        info->tile_m = 4; info->tile_n = 1; info->tile_k = 1;
        info->vec_a = 1; info->vec_b = 1;
    }
    info->waves = plan.empty ? 0 : plan.waves;
    info->launches = plan.empty ? 0 : 1;
    info->workgroups = plan.empty ? 0 : plan.workgroups;
    std::strncpy(info->kernel, plan.kernel_name.c_str(), sizeof info->kernel - 1);
    return SGEMM_OK;
}

int sgemm_strided_batched_path(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                               const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                               const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                               int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                               int64_t sC_col, int path, void *stream) {
    if (!path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "unknown path code");
    return run_gemm(pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                         sB_col, accumulate, C, sC_batch, sC_row, sC_col),
                    path, stream);
}

int sgemm_strided_batched_ex_path(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                                  const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                                  const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                                  float beta, float *C, int64_t sC_batch, int64_t sC_row,
                                  int64_t sC_col, const float *row_add, int64_t sR_batch,
                                  int64_t sR_row, const float *col_add, int64_t sL_batch,
                                  int64_t sL_col, int path, void *stream) {
    if (!path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "unknown path code");
    sgemm::GemmArgs a = pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                             sB_row, sB_col, beta != 0.0f, C, sC_batch, sC_row, sC_col);
    a.beta = beta;
    a.row_add = reinterpret_cast<uintptr_t>(row_add); a.sR_batch = sR_batch; a.sR_row = sR_row;
    a.col_add = reinterpret_cast<uintptr_t>(col_add); a.sL_batch = sL_batch; a.sL_col = sL_col;
    return run_gemm(a, path, stream);
}

int sgemm_strided_batched_ex(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                             const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                             const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                             float beta, float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                             const float *row_add, int64_t sR_batch, int64_t sR_row,
                             const float *col_add, int64_t sL_batch, int64_t sL_col, void *stream) {
    return sgemm_strided_batched_ex_path(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B,
                                         sB_batch, sB_row, sB_col, beta, C, sC_batch, sC_row,
                                         sC_col, row_add, sR_batch, sR_row, col_add, sL_batch,
                                         sL_col, SGEMM_PATH_AUTO, stream);
}

int sgemm_strided_batched2_path(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                                float alpha, const float *A, int64_t sA_outer, int64_t sA_inner,
                                int64_t gA, int64_t sA_row, int64_t sA_col, const float *B,
                                int64_t sB_outer, int64_t sB_inner, int64_t gB, int64_t sB_row,
                                int64_t sB_col, int accumulate, float *C, int64_t sC_outer,
                                int64_t sC_inner, int64_t sC_row, int64_t sC_col, int path,
                                void *stream) {
    if (!path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "unknown path code");
    sgemm::GemmArgs a;
    int st = pack2(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA, sA_row, sA_col,
                   B, sB_outer, sB_inner, gB, sB_row, sB_col, accumulate, C, sC_outer, sC_inner,
                   sC_row, sC_col, a);
    if (st != SGEMM_OK) return st;
    return run_gemm(a, path, stream);
}

int sgemm_strided_batched2(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                           float alpha, const float *A, int64_t sA_outer, int64_t sA_inner,
                           int64_t gA, int64_t sA_row, int64_t sA_col, const float *B,
                           int64_t sB_outer, int64_t sB_inner, int64_t gB, int64_t sB_row,
                           int64_t sB_col, int accumulate, float *C, int64_t sC_outer,
                           int64_t sC_inner, int64_t sC_row, int64_t sC_col, void *stream) {
    return sgemm_strided_batched2_path(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA,
                                       sA_row, sA_col, B, sB_outer, sB_inner, gB, sB_row, sB_col,
                                       accumulate, C, sC_outer, sC_inner, sC_row, sC_col,
                                       SGEMM_PATH_AUTO, stream);
}

int sgemm_sqnorms(int64_t batch, int64_t count, int64_t len, const float *X, int64_t sX_batch,
                  int64_t sX_item, int64_t sX_elem, float *out, int64_t sO_batch, int64_t sO_item,
                  void *stream) {
    if (batch < 0 || count < 0 || len < 0)
        return fail(SGEMM_ERR_INVALID_SIZE, "negative size (batch, count, len must be >= 0)");
    if (sX_batch < 0 || sX_item < 0 || sX_elem < 0 || sO_batch < 0 || sO_item < 0)
        return fail(SGEMM_ERR_INVALID_STRIDE, "negative stride");
    if (batch == 0 || count == 0) return SGEMM_OK;
    if (!out || (len > 0 && !X)) return fail(SGEMM_ERR_NULL_POINTER, out ? "X is NULL" : "out is NULL");
    const int64_t xs = span3(batch, sX_batch, count, sX_item, len, sX_elem);
    const int64_t os = span3(batch, sO_batch, count, sO_item, 1, 0);
    int64_t bytes;
    if (xs < 0 || os < 0 || __builtin_mul_overflow(std::max(xs, os), int64_t(4), &bytes))
        return fail(SGEMM_ERR_UNSUPPORTED, "an extent times its strides overflows int64");
    if (!distinct_2d(batch, sO_batch, count, sO_item))
        return fail(SGEMM_ERR_C_ALIAS, "out's strides map two norms to one element");
    if (len > 0 && ranges_meet(reinterpret_cast<uintptr_t>(X), xs, reinterpret_cast<uintptr_t>(out), os))
        return fail(SGEMM_ERR_C_ALIAS, "out overlaps X");
    std::string why;
    int st = sgemm::launch_sqnorms(batch, count, len, X, sX_batch, sX_item, sX_elem, out, sO_batch,
                                   sO_item, static_cast<hipStream_t>(stream), why);
    return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
}

int sgemm_pairwise_sqdist(int64_t batch, int64_t m, int64_t n, int64_t k, const float *X,
                          int64_t sX_batch, int64_t sX_row, int64_t sX_col, const float *Y,
                          int64_t sY_batch, int64_t sY_row, int64_t sY_col, float *D,
                          int64_t sD_batch, int64_t sD_row, int64_t sD_col, float *workspace,
                          int64_t workspace_floats, void *stream) {
    return sgemm::pairwise_sqdist(batch, m, n, k, X, sX_batch, sX_row, sX_col, Y, sY_batch, sY_row, sY_col, D,
                                  sD_batch, sD_row, sD_col, workspace, workspace_floats, 0, nullptr, stream);
}

}  // extern "C"

int sgemm::pairwise_sqdist(int64_t batch, int64_t m, int64_t n, int64_t k, const float *X, int64_t sX_batch,
                           int64_t sX_row, int64_t sX_col, const float *Y, int64_t sY_batch, int64_t sY_row,
                           int64_t sY_col, float *D, int64_t sD_batch, int64_t sD_row, int64_t sD_col,
                           float *workspace, int64_t workspace_floats, int64_t fixed_floats,
                           ScratchAddressFn fixed_address, void *stream) {
    // Validate the whole call first (as the product D <- -2 X Y^T), so that
    // an error enqueues nothing.
    sgemm::GemmArgs a = pack(batch, m, n, k, -2.0f, X, sX_batch, sX_row, sX_col, Y, sY_batch,
                             sY_col, sY_row, 0, D, sD_batch, sD_row, sD_col);
    std::string why;
    int st = sgemm::validate(a, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (batch == 0 || m == 0 || n == 0) return SGEMM_OK;
    const int64_t ny = sY_batch == 0 ? 1 : batch;
    int64_t need, ny_n;
    if (__builtin_mul_overflow(batch, m, &need) || __builtin_mul_overflow(ny, n, &ny_n) ||
        __builtin_add_overflow(need, ny_n, &need))
        return fail(SGEMM_ERR_UNSUPPORTED, "workspace size overflows int64");
    if (fixed_floats > 0) {
        if (need > fixed_floats)
            return fail(SGEMM_ERR_WORKSPACE,
                        "the call needs batch*m + nY*n = " + std::to_string(need) +
                            " floats of norms; the allocation-free entry point's fixed device scratch holds " +
                            std::to_string(fixed_floats) + " (use sgemm_pairwise_sqdist with a workspace)");
        st = fixed_address(&workspace, why);
        if (st != SGEMM_OK) return fail(st, why);
        workspace_floats = fixed_floats;
    }
    if (!workspace || workspace_floats < need)
        return fail(SGEMM_ERR_WORKSPACE, "workspace needs batch*m + nY*n floats");
    const uintptr_t ws = reinterpret_cast<uintptr_t>(workspace);
    const int64_t xs = span3(batch, sX_batch, m, sX_row, k, sX_col);
    const int64_t ys = span3(ny, sY_batch, n, sY_row, k, sY_col);
    const int64_t ds = span3(batch, sD_batch, m, sD_row, n, sD_col);
    if ((k > 0 && (ranges_meet(ws, need, reinterpret_cast<uintptr_t>(X), xs) ||
                   ranges_meet(ws, need, reinterpret_cast<uintptr_t>(Y), ys))) ||
        ranges_meet(ws, need, reinterpret_cast<uintptr_t>(D), ds))
        return fail(SGEMM_ERR_C_ALIAS, "workspace overlaps X, Y or D");
    float *nx = workspace, *nyv = workspace + batch * m;
    st = sgemm_sqnorms(batch, m, k, X, sX_batch, sX_row, sX_col, nx, m, 1, stream);
    if (st != SGEMM_OK) return st;
    st = sgemm_sqnorms(ny, n, k, Y, sY_batch, sY_row, sY_col, nyv, n, 1, stream);
    if (st != SGEMM_OK) return st;
    a.row_add = reinterpret_cast<uintptr_t>(nx); a.sR_batch = m; a.sR_row = 1;
    a.col_add = reinterpret_cast<uintptr_t>(nyv); a.sL_batch = sY_batch == 0 ? 0 : n; a.sL_col = 1;
    return run_gemm(a, SGEMM_PATH_AUTO, stream);
}

extern "C" {

int sgemm_strided_batched(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                          const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                          const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                          int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                          int64_t sC_col, void *stream) {
    return sgemm_strided_batched_path(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B,
                                      sB_batch, sB_row, sB_col, accumulate, C, sC_batch, sC_row,
                                      sC_col, SGEMM_PATH_AUTO, stream);
}

}  // extern "C"

namespace {

void fill_info(const sgemm::Plan &plan, sgemm_plan_info *info);

// Validate and plan `a` without touching the device; fill *info.
int describe(const sgemm::GemmArgs &a, int path, int num_cus, sgemm_plan_info *info) {
    if (!path_ok(path)) return fail(SGEMM_ERR_INVALID_PATH, "unknown path code");
    if (!info) return fail(SGEMM_ERR_NULL_POINTER, "info is NULL");
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
    fill_info(plan, info);
    return SGEMM_OK;
}

}  // namespace

namespace {

// The launch `plan` makes, as the public plan record.
void fill_info(const sgemm::Plan &plan, sgemm_plan_info *info) {
    std::memset(info, 0, sizeof *info);
    info->path = plan.empty ? SGEMM_PATH_AUTO : static_cast<int>(plan.family);
    info->transposed = plan.transposed ? 1 : 0;
    if (plan.tile >= 0 && plan.persist) {
        const sgemm::PersistCfg &t = sgemm::kPersistTiles[plan.tile];
        info->tile_m = t.bm; info->tile_n = t.bn; info->tile_k = t.kmax;
        info->waves = t.waves();
    } else if (plan.tile >= 0 && plan.strip) {
        const sgemm::StripCfg &t = sgemm::kStripTiles[plan.tile];
        info->tile_m = t.rows; info->tile_n = int(std::min<int64_t>(plan.n, INT32_MAX)); info->tile_k = t.kmax;
        info->waves = t.waves;
    } else if (plan.tile >= 0 && plan.family == sgemm::Family::Wave) {
        const sgemm::WaveCfg &t = sgemm::kWaveTiles[plan.tile];
        info->tile_m = t.bm; info->tile_n = t.bn; info->tile_k = 16;
        info->waves = plan.ksplit;
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
    info->fixed_offsets = plan.fixed_offsets ? 1 : 0;
    info->workgroups = plan.empty ? 0 : plan.workgroups;
    std::strncpy(info->kernel, plan.kernel_name.c_str(), sizeof info->kernel - 1);
}

// Checks of the split-k entry points beyond the product's own: the
// workspace size, its pointer, and its overlap with A, B and C.
int check_workspace(const sgemm::GemmArgs &a, const float *workspace, int64_t workspace_floats) {
    if (workspace_floats < 0) return fail(SGEMM_ERR_INVALID_SIZE, "workspace_floats must be >= 0");
    if (workspace_floats > 0 && !workspace)
        return fail(SGEMM_ERR_NULL_POINTER, "workspace is NULL but workspace_floats > 0");
    if (!workspace || workspace_floats == 0 || a.batch == 0 || a.m == 0 || a.n == 0) return SGEMM_OK;
    const uintptr_t w = reinterpret_cast<uintptr_t>(workspace);
    const int64_t cs = span3(a.batch, a.sC_batch, a.m, a.sC_row, a.n, a.sC_col);
    if (ranges_meet(w, workspace_floats, a.C, cs)) return fail(SGEMM_ERR_C_ALIAS, "workspace overlaps C");
    if (a.k > 0) {
        const int64_t as = span3(a.batch, a.sA_batch, a.m, a.sA_row, a.k, a.sA_col);
        const int64_t bs = span3(a.batch, a.sB_batch, a.k, a.sB_row, a.n, a.sB_col);
        if (ranges_meet(w, workspace_floats, a.A, as)) return fail(SGEMM_ERR_C_ALIAS, "workspace overlaps A");
        if (ranges_meet(w, workspace_floats, a.B, bs)) return fail(SGEMM_ERR_C_ALIAS, "workspace overlaps B");
    }
    return SGEMM_OK;
}

}  // namespace

extern "C" {

int sgemm_strided_batched_splitk(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                                 const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                                 const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                                 int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                                 int64_t sC_col, float *workspace, int64_t workspace_floats,
                                 void *stream) {
    const sgemm::GemmArgs a = pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                                   sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col);
    std::string why;
    int st = sgemm::validate(a, why);
    if (st != sgemm::kOk) return fail(st, why);
    st = check_workspace(a, workspace, workspace_floats);
    if (st != SGEMM_OK) return st;
    if (a.batch == 0 || a.m == 0 || a.n == 0) return SGEMM_OK;
    int cus = 0;
    st = current_cus(cus, why);
    if (st != sgemm::kOk) return fail(st, why);
    const uintptr_t w = reinterpret_cast<uintptr_t>(workspace);
    const int64_t floats = workspace ? workspace_floats : 0;
    // The split plan (up to nine product plans) is cached per thread like
    // the product's, keyed by the workspace as well.
    const bool cacheable = !planner_overrides() && !std::getenv("SGEMM_SPLITK");
    if (cacheable)
        for (const CachedSplit &c : g_splits)
            if (c.cus == cus && c.workspace == w && c.floats == floats && same_args(c.args, a)) {
                st = sgemm::launch_split_plan(a, c.plan, w, static_cast<hipStream_t>(stream), why);
                return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
            }
    sgemm::SplitPlan sp;
    st = sgemm::make_split_plan(a, cus, w, floats, sp, why);
    if (st != sgemm::kOk) return fail(st, why);
    if (cacheable) {
        CachedSplit &c = g_splits[g_split_next];
        g_split_next = (g_split_next + 1) % kPlanCacheSize;
        c.args = a;
        c.cus = cus;
        c.workspace = w;
        c.floats = floats;
        c.plan = sp;
    }
    st = sgemm::launch_split_plan(a, sp, w, static_cast<hipStream_t>(stream), why);
    return st == sgemm::kOk ? SGEMM_OK : fail(st, why);
}

int sgemm_splitk_describe(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                          const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                          const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                          int accumulate, float *C, int64_t sC_batch, int64_t sC_row, int64_t sC_col,
                          const float *workspace, int64_t workspace_floats, int num_cus,
                          sgemm_splitk_info *info) {
    if (!info) return fail(SGEMM_ERR_NULL_POINTER, "info is NULL");
    const sgemm::GemmArgs a = pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                                   sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col);
    std::string why;
    int st = sgemm::validate(a, why);
    if (st != sgemm::kOk) return fail(st, why);
    const bool query = workspace_floats < 0;   // no cap: the size the best split needs
    if (!query) {
        st = check_workspace(a, workspace, workspace_floats);
        if (st != SGEMM_OK) return st;
    }
    if (num_cus <= 0) {
        st = current_cus(num_cus, why);
        if (st != sgemm::kOk) return fail(st, why);
    }
    sgemm::SplitPlan sp;
    st = sgemm::make_split_plan(a, num_cus, query ? 0 : reinterpret_cast<uintptr_t>(workspace),
                                query ? -1 : (workspace ? workspace_floats : 0), sp, why);
    if (st != sgemm::kOk) return fail(st, why);
    std::memset(info, 0, sizeof *info);
    info->splits = sp.splits;
    info->kc = sp.splits > 1 ? sp.kc : k;
    info->k_last = sp.splits > 1 ? sp.k_last : k;
    info->workspace_floats = sp.splits > 1 ? sp.workspace_floats : 0;
    info->launches = sp.whole.empty ? 0 : sp.splits == 1 ? 1 : (sp.full < sp.splits ? 3 : 2);
    fill_info(sp.splits > 1 ? sp.parts : sp.whole, &info->parts);
    return SGEMM_OK;
}

int sgemm_plan_describe(int64_t batch, int64_t m, int64_t n, int64_t k, float alpha,
                        const float *A, int64_t sA_batch, int64_t sA_row, int64_t sA_col,
                        const float *B, int64_t sB_batch, int64_t sB_row, int64_t sB_col,
                        int accumulate, float *C, int64_t sC_batch, int64_t sC_row,
                        int64_t sC_col, int path, int num_cus, sgemm_plan_info *info) {
    return describe(pack(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                         sB_col, accumulate, C, sC_batch, sC_row, sC_col),
                    path, num_cus, info);
}

int sgemm_plan_describe2(int64_t nb_outer, int64_t nb_inner, int64_t m, int64_t n, int64_t k,
                         float alpha, const float *A, int64_t sA_outer, int64_t sA_inner,
                         int64_t gA, int64_t sA_row, int64_t sA_col, const float *B,
                         int64_t sB_outer, int64_t sB_inner, int64_t gB, int64_t sB_row,
                         int64_t sB_col, int accumulate, float *C, int64_t sC_outer,
                         int64_t sC_inner, int64_t sC_row, int64_t sC_col, int path, int num_cus,
                         sgemm_plan_info *info) {
    sgemm::GemmArgs a;
    int st = pack2(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA, sA_row, sA_col,
                   B, sB_outer, sB_inner, gB, sB_row, sB_col, accumulate, C, sC_outer, sC_inner,
                   sC_row, sC_col, a);
    return st != SGEMM_OK ? st : describe(a, path, num_cus, info);
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
    case SGEMM_ERR_WORKSPACE: return "SGEMM_ERR_WORKSPACE: workspace missing or too small";
    default: return "unknown sgemm status";
    }
}

const char *sgemm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
