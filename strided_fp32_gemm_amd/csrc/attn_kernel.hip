// attn_kernel.hip -- fused scaled dot-product attention kernels for gfx950.
//
// Scores, softmax and the product with V in one pass per query block (the
// rvllm post, "What's basic about it": a fused kernel keeps the scores out of
// global memory).  The softmax is the online form of the post's three steps
// (max, sum of exponentials, divide; "The kernels"): the running maximum and
// sum are rescaled as each block of keys arrives, and the division happens
// once at the end.
//
// attn_mfma_d64 (head dimension 64, unit column strides):
//  - A wavefront owns 16 query rows.  It forms the scores transposed,
//    S^T = K Q^T, with v_mfma_f32_16x16x4_f32, so lane l holds query l%16 and
//    16 of its scores in accumulator registers (keys 4*(l/16) + r of each
//    16-key block).  Those registers are already the B operand of
//    O^T = V^T P^T, so the probabilities never leave registers, and each lane
//    ends with 4 consecutive head-dimension outputs of its query per block
//    (one 16-byte store).
//  - The head-dimension sum of the scores runs in the order d = 16*(l/16) + s
//    for step s, so each lane reads its 16 K values of a key with four 16-byte
//    LDS reads.  The key sum of P V follows the score layout.  Both orders are
//    fixed, so results are reproducible bit for bit.
//  - Keys arrive in blocks of 64, K and V staged through double-buffered LDS
//    (row pitch 68 floats: the 4-byte V reads are free of bank conflicts; the
//    16-byte K reads take two cycles per 16-lane group instead of one, which
//    no row pitch avoids with this head-dimension order, but LDS time stays a
//    small fraction of the matrix-core time); the next block's global loads
//    are in flight while the current one is multiplied; one barrier per block.
//  - Weights are exp2(s * alpha*log2(e) - running max), with v_exp_f32.  The
//    row maximum needs two lane swaps per key block (v_permlane16_swap,
//    v_permlane32_swap: vector instructions, no LDS round trip); the row sum
//    stays per lane until the end.
//  - Causal: a workgroup pairs an early and a late block of query rows (one
//    per half of its wavefronts) so that workgroups carry equal work; it
//    stops at the last key its queries see, and a wavefront skips the blocks
//    entirely past its own diagonal.  Keys past a
//    query's last visible key (or past the end) get weight exp2(-inf) = 0
//    through one compare and select per score.
//
// attn_generic: any head dimension up to 256 and any strides, 64-bit
// addressing; one wavefront per query row, the score of each key summed
// across the wavefront, the same online softmax.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>

#include "attention.hpp"
#include "buffer.hpp"
#include "kernels.hpp"

namespace sgemm {

namespace {

constexpr int kD = 64;                      // head dimension of the matrix-core kernel
constexpr int kBKV = 64;                    // keys per LDS block
constexpr int kPitch = kD + 4;              // LDS row pitch (floats)
constexpr int kTileFloats = kBKV * kPitch;  // one K or V block in LDS
constexpr int kQW = 16;                     // query rows per wavefront
constexpr int kLdsBytes = 2 * 2 * kTileFloats * 4;

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine the four lanes l%16 + 16*h (h = 0..3) of a wavefront with `op`,
// leaving the result in all four: lanes swap 16-lane rows (v_permlane16_swap:
// row 0 with 1, 2 with 3), then 32-lane halves (v_permlane32_swap), both plain
// vector instructions.  A self-swap returns this lane's value and its
// partner's in some order, so op(r[0], r[1]) is the pair's result in both
// lanes; the association is (row 0 op row 1) op (row 2 op row 3).
// (The two results are copied to scalars before the bit casts: a bit cast of
// a subscripted vector element reads the vector's first element.)
template <typename Op>
__device__ __forceinline__ float across_rows(float v, Op op) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned a0 = r16[0], a1 = r16[1];
    v = op(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
    const unsigned w = __builtin_bit_cast(unsigned, v);
    const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    const unsigned b0 = r32[0], b1 = r32[1];
    return op(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_mfma_d64(AttnArgs p) {
    constexpr int NT = NW * 64;
    constexpr int BQ = NW * kQW;
    constexpr int SL = kBKV * kD / 4 / NT;   // 16-byte slots per thread per K (or V) block
    static_assert(kBKV * kD / 4 % NT == 0, "every thread stages the same number of slots");
    extern __shared__ float lds[];           // [2 buffers][K block, V block]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 15, lh = lane >> 4;

    // Workgroup -> (outer o, inner i, query block qb); KV head kv = i / g.
    unsigned w = blockIdx.x;
    if (p.xcd_remap) w = (w & 7u) * unsigned(p.blocks >> 3) + (w >> 3);
    const unsigned b = divide(w, p.qblocks);
    const unsigned qb = w - b * p.qblocks.d;
    const unsigned o = divide(b, p.inner);
    const unsigned i = b - o * p.inner.d;
    const unsigned kv = divide(i, p.group);

    const int tq = p.tq, tk = p.tk;
    const int shift = tk - tq;                    // causal: query q sees keys j <= q + shift
    // First query row of this wavefront, and the last row of the workgroup.
    // Zigzag (causal): waves of the first half take rows of half-block qb,
    // the second half those of the mirrored block half_blocks-1-qb (idle
    // when the two coincide, the middle of an odd count).
    constexpr int HB = BQ / 2;
    int qwave, wg_last_row;
    bool wave_on = true;
    if (p.zigzag) {
        const int half = wave >= NW / 2 ? 1 : 0;
        const int mirror = p.half_blocks - 1 - int(qb);
        wave_on = half == 0 || mirror != int(qb);
        qwave = (half ? mirror : int(qb)) * HB + (wave - half * (NW / 2)) * kQW;
        wg_last_row = max(mirror, int(qb)) * HB + HB - 1;
    } else {
        qwave = int(qb) * BQ + wave * kQW;
        wg_last_row = int(qb) * BQ + BQ - 1;
    }
    const int qrow = qwave + lq;
    const bool qok = wave_on && qrow < tq;

    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(p.Q + o * p.sQ_o + i * p.sQ_i);
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.K + o * p.sK_o + kv * p.sK_i);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.V + o * p.sV_o + kv * p.sV_i);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(p.O + o * p.sO_o + i * p.sO_i);
    const unsigned sQr = unsigned(p.sQ_r), sKr = unsigned(p.sK_r), sVr = unsigned(p.sV_r),
                   sOr = unsigned(p.sO_r);

    // This lane's Q values: query qrow, head dimensions 16*lh .. 16*lh + 15.
    f32x4 qf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        qf[j] = load4(rQ, qok ? (unsigned(qrow) * sQr + unsigned(16 * lh + 4 * j)) * 4u : kOutOfRange);

    // K and V blocks: slot s of a block is key s/16, head dimensions 4*(s%16) .. +3.
    f32x4 kst[SL], vst[SL];
    auto issue = [&](int kv0) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int s = tid + u * NT;
            const int key = kv0 + (s >> 4);
            const unsigned c = unsigned(s & 15) * 4u;
            const bool ok = key < tk;
            kst[u] = load4(rK, ok ? (unsigned(key) * sKr + c) * 4u : kOutOfRange);
            vst[u] = load4(rV, ok ? (unsigned(key) * sVr + c) * 4u : kOutOfRange);
        }
    };
    auto put = [&](int buf) {
        float *Kl = lds + buf * 2 * kTileFloats;
        float *Vl = Kl + kTileFloats;
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int s = tid + u * NT;
            const int at = (s >> 4) * kPitch + (s & 15) * 4;
            *reinterpret_cast<f32x4 *>(Kl + at) = kst[u];
            *reinterpret_cast<f32x4 *>(Vl + at) = vst[u];
        }
    };

    int last_key = tk - 1;
    if (p.causal) last_key = min(last_key, wg_last_row + shift);
    const int nblocks = last_key / kBKV + 1;
    const int wave_last = qwave + kQW - 1 + shift;   // last key this wavefront sees (causal)

    const float c2 = p.scale_log2;
    float m = -INFINITY;   // running maximum of c2 * score over the keys seen
    float l = 0.0f;        // this lane's share of the running sum of weights
    f32x4 oacc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) oacc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    issue(0);
    put(0);
    if (nblocks > 1) issue(kBKV);
    __syncthreads();

    for (int t = 0; t < nblocks; ++t) {
        const int kv0 = t * kBKV;
        const float *Kl = lds + (t & 1) * 2 * kTileFloats;
        const float *Vl = Kl + kTileFloats;
        if (wave_on && (!p.causal || kv0 <= wave_last)) {
            // Scores^T for keys kv0 + 16*kb + (0..15): sacc[kb][r] is key
            // kv0 + 16*kb + 4*lh + r of query qrow.
            f32x4 sacc[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sacc[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            // K fragments of step group j (head dimensions 16*lh + 4*j + e),
            // read one group ahead; the four accumulators take turns.
            f32x4 kf[2][4];
            auto read_k = [&](int j, f32x4 (&dst)[4]) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    dst[kb] = *reinterpret_cast<const f32x4 *>(Kl + (16 * kb + lq) * kPitch + 16 * lh + 4 * j);
            };
            read_k(0, kf[0]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j + 1 < 4) read_k(j + 1, kf[(j + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) sacc[kb] = mfma16(kf[j & 1][kb][e], qf[j][e], sacc[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Last key of this block the lane's query sees, relative to the
            // lane's first key (kv0 + 4*lh); >= 63 when the block is all visible.
            int lim = tk - 1;
            if (p.causal) lim = min(lim, qrow + shift);
            lim -= kv0 + 4 * lh;
            float x[4][4];
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = sacc[kb][r] * c2;
                    x[kb][r] = 16 * kb + r <= lim ? v : -INFINITY;
                    mt = fmaxf(mt, x[kb][r]);
                }
            mt = across_rows(mt, [](float x, float y) { return fmaxf(x, y); });
            const float mnew = fmaxf(m, mt);
            const float corr = exp2_fast(m - mnew);
            m = mnew;
            float ls = 0.0f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[kb][r] = exp2_fast(x[kb][r] - mnew);
                    ls += x[kb][r];
                }
            l = l * corr + ls;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) oacc[nb] *= corr;
            // O^T += V^T P^T over the 64 keys of this block; the V values of
            // 16-key group kb are read one group ahead.
            float vf[2][4][4];   // [buffer][r][nb]: V[kv0 + 16*kb + 4*lh + r][16*nb + lq]
            auto read_v = [&](int kb, float (&dst)[4][4]) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        dst[r][nb] = Vl[(16 * kb + 4 * lh + r) * kPitch + 16 * nb + lq];
            };
            read_v(0, vf[0]);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                if (kb + 1 < 4) read_v(kb + 1, vf[(kb + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) oacc[nb] = mfma16(vf[kb & 1][r][nb], x[kb][r], oacc[nb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (t + 1 < nblocks) {
            put((t + 1) & 1);
            if (t + 2 < nblocks) issue((t + 2) * kBKV);
        }
        __syncthreads();
    }

    // The four lanes of a query hold disjoint key subsets of its sum.
    l = across_rows(l, [](float x, float y) { return x + y; });
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const f32x4 v = oacc[nb] / l;
        store4_device(rO, qok ? (unsigned(qrow) * sOr + unsigned(16 * nb + 4 * lh)) * 4u : kOutOfRange, v);
    }
}

__global__ __launch_bounds__(256) void attn_generic(AttnArgs p) {
    constexpr int CPL = kAttnMaxDim / 64;   // head-dimension columns per lane
    const int lane = threadIdx.x & 63;
    const long long first = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long step = (long long)gridDim.x * 4;
    const float c2 = p.scale_log2;
    for (long long w = first; w < p.rows; w += step) {   // uniform across the wavefront
        const long long q = w % p.tq, head = w / p.tq;
        const long long o = head / p.nb_inner_ll, i = head % p.nb_inner_ll, kv = i / p.g_ll;
        const float *Qr = p.Q + o * p.sQ_o + i * p.sQ_i + q * p.sQ_r;
        const float *Kb = p.K + o * p.sK_o + kv * p.sK_i;
        const float *Vb = p.V + o * p.sV_o + kv * p.sV_i;
        float *Or = p.O + o * p.sO_o + i * p.sO_i + q * p.sO_r;
        float qv[CPL], acc[CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int c = lane + 64 * u;
            qv[u] = c < p.d ? Qr[c * p.sQ_c] : 0.0f;
            acc[u] = 0.0f;
        }
        const long long seen = p.causal ? q + (p.tk - p.tq) + 1 : p.tk;
        float m = -INFINITY, l = 0.0f;
        for (long long j = 0; j < seen; ++j) {
            float part = 0.0f;
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                const int c = lane + 64 * u;
                if (c < p.d) part = fmaf(qv[u], Kb[j * p.sK_r + c * p.sK_c], part);
            }
            // Butterfly sum: partners add the same two values, so every lane
            // ends with the same bits.
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
            const float x = part * c2;
            const float mnew = fmaxf(m, x);
            const float corr = exp2_fast(m - mnew);
            const float pj = exp2_fast(x - mnew);
            m = mnew;
            l = l * corr + pj;
#pragma unroll
            for (int u = 0; u < CPL; ++u) {
                const int c = lane + 64 * u;
                if (c < p.d) acc[u] = fmaf(pj, Vb[j * p.sV_r + c * p.sV_c], acc[u] * corr);
            }
        }
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int c = lane + 64 * u;
            if (c < p.d) Or[c * p.sO_c] = acc[u] / l;
        }
    }
}

template <int NW>
void launch_mfma_attention(const AttnArgs &a, unsigned grid, hipStream_t s) {
    static std::atomic<unsigned long long> lds_set{0};
    allow_dynamic_lds(reinterpret_cast<const void *>(&attn_mfma_d64<NW>), kLdsBytes, lds_set);
    hipLaunchKernelGGL(attn_mfma_d64<NW>, dim3(grid), dim3(NW * 64), kLdsBytes, s, a);
}

}  // namespace

int launch_attention(const AttnPlan &plan, hipStream_t stream, std::string &why) {
    if (plan.empty) return kOk;
    (void)hipGetLastError();   // clear a stale error left by unrelated work
    if (plan.path == AttnPath::Mfma) {
        if (plan.waves == 8)
            launch_mfma_attention<8>(plan.args, unsigned(plan.workgroups), stream);
        else
            launch_mfma_attention<4>(plan.args, unsigned(plan.workgroups), stream);
    } else {
        hipLaunchKernelGGL(attn_generic, dim3(unsigned(plan.workgroups)), dim3(256), 0, stream, plan.args);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        why = std::string("attention launch failed: ") + hipGetErrorString(e);
        return kErrHip;
    }
    return kOk;
}

}  // namespace sgemm
