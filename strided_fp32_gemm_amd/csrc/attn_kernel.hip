// attn_kernel.hip -- fused scaled dot-product attention kernels for gfx950.
//
// Scores, softmax and the product with V in one pass per query block (the
// rvllm post, "What's basic about it": a fused kernel keeps the scores out of
// global memory).  The softmax is the online form of the post's three steps
// (max, sum of exponentials, divide; "The kernels"): the weights of each
// block of keys are taken relative to a reference maximum that moves as
// larger scores arrive, the sums already formed are rescaled when it moves,
// and the division happens once at the end.
//
// On gfx950 the fp32 matrix instructions and ordinary vector instructions
// share one issue path per SIMD and never run at the same time, so every
// vector instruction in the key loop adds to the time of the products.  The
// matrix-core kernel is built around keeping that count small.
//
// attn_mfma_d64 (head dimension 64, unit column strides):
//  - A wavefront owns 16 query rows.  It forms the scores transposed,
//    S^T = K Q^T, with v_mfma_f32_16x16x4_f32, so lane l holds query l%16 and
//    16 of its scores in accumulator registers (keys 4*(l/16) + r of each
//    16-key block).  Those registers are already the B operand of
//    O^T = V^T P^T, so the probabilities never leave registers.
//  - Q is loaded once, scaled by alpha*log2(e), and the score products start
//    from minus the row's reference maximum m instead of zero, so they end
//    as the exponent of each weight, exp2(alpha*log2(e)*s - m), with no
//    vector work in between.
//  - The reference maximum moves only when a score exceeds it by more than
//    kSlack (weights stay below 2^kSlack); the test is one compare and a
//    wavefront vote, and the rescaling (a lane swap reduction, one exp2,
//    multiplies of the output and the sum) runs only when the vote says so.
//    Softmax is invariant to the reference, so this changes no result
//    beyond rounding.  The first key block sets the reference from its own
//    row maxima.
//  - Keys past a query's last visible key (causal, or past the end) are
//    masked with one compare and select per score, only in the blocks that
//    hold such keys; every other block skips the test.
//  - Keys arrive in blocks of 64, K and V staged through double-buffered LDS;
//    the next block's global loads are in flight while the current one is
//    multiplied; one barrier per block.  K rows have a pitch of 68 floats
//    with the 16-byte chunks of rows whose bits 2 and 3 differ swapped in
//    pairs (chunk c stored at c ^ 4), and V rows a pitch of 64: under
//    gfx950's LDS lane groups every 16-byte read and write is free of bank
//    conflicts.  Each lane's LDS addresses are fixed for the whole loop
//    (immediate offsets), and the global load offsets too (the buffer
//    resource moves with the block), so the loop spends no vector
//    instructions on addresses.
//  - In O^T = V^T P^T, matrix instruction nb takes head dimensions 4i + nb
//    for its rows i, so a lane's V operands for the four instructions of a
//    step are four consecutive floats of one V row (one 16-byte LDS read),
//    and the four accumulators hold, per element e, four consecutive outputs
//    (16*(l/16) + 4e .. +3) of the lane's query: one 16-byte store each.
//  - The head-dimension sum of the scores runs in the order d = 16*(l/16) + s
//    for step s, and the key sum of P V follows the score layout.  Both
//    orders are fixed, so results are reproducible bit for bit.
//  - Causal: a workgroup pairs an early and a late block of query rows (one
//    per half of its wavefronts) so that workgroups carry equal work; it
//    stops at the last key its queries see, and a wavefront skips the blocks
//    entirely past its own diagonal.
//
// attn_generic: any head dimension up to 256 and any strides, 64-bit
// addressing; one wavefront per query row, the score of each key summed
// across the wavefront, the online softmax with the exact running maximum.
#include <hip/hip_runtime.h>

#include <cmath>
#include <string>
#include <type_traits>

#include "attention.hpp"
#include "attn_layout.hpp"
#include "buffer.hpp"
#include "kernels.hpp"

namespace sgemm {

namespace {

constexpr int kD = kAttnD;                        // head dimension of the matrix-core kernel
constexpr int kBKV = kAttnBlockKeys;              // keys per LDS block
constexpr int kKPitch = kAttnKPitch;              // K rows in LDS (floats)
constexpr int kVPitch = kAttnVPitch;              // V rows in LDS (floats)
constexpr int kBufFloats = kAttnBufFloats;        // one K block and one V block
constexpr int kQW = 16;                           // query rows per wavefront
constexpr int kLdsBytes = 2 * kBufFloats * 4;
constexpr float kSlack = 8.0f;                    // log2 of the largest weight before the reference moves

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
    constexpr int SR = NT / 16;              // key rows between a thread's slots
    static_assert(kBKV * kD / 4 % NT == 0, "every thread stages the same number of slots");
    extern __shared__ float lds[];           // [2 buffers][K block, V block]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    const float *Kb = p.K + o * p.sK_o + kv * p.sK_i;
    const float *Vb = p.V + o * p.sV_o + kv * p.sV_i;
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(p.Q + o * p.sQ_o + i * p.sQ_i);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(p.O + o * p.sO_o + i * p.sO_i);
    const unsigned sQr = unsigned(p.sQ_r), sKr = unsigned(p.sK_r), sVr = unsigned(p.sV_r),
                   sOr = unsigned(p.sO_r);
    const float c2 = p.scale_log2;

    // This lane's Q values, scaled by alpha*log2(e): query qrow, head
    // dimensions 16*lh .. 16*lh + 15.
    f32x4 qf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        qf[j] = c2 * load4(rQ, qok ? (unsigned(qrow) * sQr + unsigned(16 * lh + 4 * j)) * 4u : kOutOfRange);

    // Staging: slot u of a block is key row kr + SR*u, head dimensions
    // 4*c .. 4*c + 3.  Global offsets are relative to the block's first row
    // (the second slot's distance is a scalar offset), LDS addresses are
    // fixed per thread.
    const int kr = tid >> 4, c = tid & 15;   // slot 0: key row, head dimensions 4*c .. +3
    const unsigned kgo = (unsigned(kr) * sKr + 4u * unsigned(c)) * 4u;
    const unsigned vgo = (unsigned(kr) * sVr + 4u * unsigned(c)) * 4u;
    // LDS layout (attn_layout.hpp): slot tid + SR*16*u sits SR*u rows below
    // slot tid, with the same K chunk order.
    float *const kwr = lds + attn_k_slot(tid);
    float *const vwr = lds + attn_v_slot(tid);
    static_assert(SR % 16 == 0, "a thread's slots share the K chunk order");
    f32x4 kst[SL], vst[SL];
    auto issue = [&](int kv0) {
        const __amdgpu_buffer_rsrc_t rK = make_rsrc(Kb + size_t(kv0) * p.sK_r);
        const __amdgpu_buffer_rsrc_t rV = make_rsrc(Vb + size_t(kv0) * p.sV_r);
        const int left = tk - kv0;   // keys of this block that exist
        if (left >= kBKV) {
#pragma unroll
            for (int u = 0; u < SL; ++u) {
                kst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rK, int(kgo), int(unsigned(SR * u) * sKr * 4u), 0));
                vst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rV, int(vgo), int(unsigned(SR * u) * sVr * 4u), 0));
            }
        } else {
#pragma unroll
            for (int u = 0; u < SL; ++u) {
                // Rows past the end get an offset beyond the resource's range.
                const unsigned past = unsigned(kr + SR * u >= left) << 31;
                kst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rK, int(kgo + past), int(unsigned(SR * u) * sKr * 4u), 0));
                vst[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rV, int(vgo + past), int(unsigned(SR * u) * sVr * 4u), 0));
            }
        }
    };
    auto put = [&](auto bufc) {
        constexpr int off = decltype(bufc)::value * kBufFloats;
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            *reinterpret_cast<f32x4 *>(kwr + off + SR * u * kKPitch) = kst[u];
            *reinterpret_cast<f32x4 *>(vwr + off + SR * u * kVPitch) = vst[u];
        }
    };

    int last_key = tk - 1;
    if (p.causal) last_key = min(last_key, wg_last_row + shift);
    const int nblocks = last_key / kBKV + 1;
    const int wave_last = qwave + kQW - 1 + shift;   // last key this wavefront sees (causal)
    // Keys before wave_full are visible to every query row of the wavefront.
    const int wave_full = p.causal ? min(tk, qwave + shift + 1) : tk;

    // This lane's LDS read addresses (attn_layout.hpp): fragment (kb, j) of
    // K and (kb, r) of V sit 16*kb*kKPitch + 4*j and (16*kb + r)*kVPitch
    // floats past fragment (0, 0).
    const float *const krd = lds + attn_k_frag(lane, 0, 0);
    const float *const vrd = lds + attn_v_frag(lane, 0, 0);

    float m = 0.0f;        // reference maximum of this lane's query (log2 units)
    f32x4 negm = f32x4{0.0f, 0.0f, 0.0f, 0.0f};   // -m in every element
    float l = 0.0f;        // this lane's share of the sum of weights
    f32x4 oacc[4];         // oacc[nb][e]: output 16*lh + 4*e + nb of query qrow
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) oacc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int t, auto bufc, bool active, auto &&stage_put, auto &&stage_issue) {
        constexpr int off = decltype(bufc)::value * kBufFloats;
        const int kv0 = t * kBKV;
        // Exponents for keys kv0 + 16*kb + (0..15): sacc[kb][r] is
        // alpha*log2(e)*score - m for key kv0 + 16*kb + 4*lh + r of query qrow.
        f32x4 sacc[4];
        f32x4 kf[2][4];   // K fragments of step group j: head dimensions 16*lh + 4*j + e
        auto read_k = [&](int j, f32x4 (&dst)[4]) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                dst[kb] = *reinterpret_cast<const f32x4 *>(krd + off + 16 * kb * kKPitch + 4 * j);
        };
        if (active) read_k(0, kf[0]);
        stage_put();
        if (!active) {
            stage_issue();
            return;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j + 1 < 4) read_k(j + 1, kf[(j + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    sacc[kb] = mfma16(kf[j & 1][kb][e], qf[j][e], j == 0 && e == 0 ? negm : sacc[kb]);
            __builtin_amdgcn_sched_barrier(0);
        }
        stage_issue();
        if (kv0 + kBKV > wave_full) {
            // Some key of this block is hidden from some row: the last key of
            // the block the lane's query sees, relative to its first key.
            int lim = tk - 1;
            if (p.causal) lim = min(lim, qrow + shift);
            lim -= kv0 + 4 * lh;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * kb + r > lim) sacc[kb][r] = -INFINITY;
        }
        float lm = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (kb + r > 0) lm = fmaxf(lm, sacc[kb][r]);
        if (t == 0 || __builtin_amdgcn_ballot_w64(lm > kSlack)) {
            // Move the reference: to the row maxima on the first block (every
            // row sees key 0), else up to them where they exceed it.
            float dm = across_rows(lm, [](float x, float y) { return fmaxf(x, y); });
            if (t != 0) {
                dm = fmaxf(dm, 0.0f);
                const float corr = exp2_fast(-dm);
                l *= corr;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) oacc[nb] *= corr;
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sacc[kb] -= dm;
            m += dm;
            negm = f32x4{-m, -m, -m, -m};
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sacc[kb][r] = exp2_fast(sacc[kb][r]);
                l += sacc[kb][r];
            }
        // O^T += V^T P^T over the 64 keys of this block; vf[r] is V row
        // kv0 + 16*kb + 4*lh + r, columns 4*lq .. 4*lq + 3, read one key
        // group ahead.
        f32x4 vf[2][4];
        auto read_v = [&](int kb, f32x4 (&dst)[4]) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[r] = *reinterpret_cast<const f32x4 *>(vrd + off + (16 * kb + r) * kVPitch);
        };
        read_v(0, vf[0]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb + 1 < 4) read_v(kb + 1, vf[(kb + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) oacc[nb] = mfma16(vf[kb & 1][r][nb], sacc[kb][r], oacc[nb]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Block t: its K and V are in buffer t % 2.  The next block's data,
    // loaded one block ago, goes to the other buffer as soon as the block
    // starts (every wavefront finished reading that buffer before the last
    // barrier), right after this wavefront's first K reads, so the LDS writes
    // complete during the products and the barrier waits only for them; the
    // loads of the block after it are issued once the score products are done.
    auto block = [&](int t, auto bufc) {
        constexpr int next = 1 - decltype(bufc)::value;
        auto stage_put = [&]() {
            if (t + 1 < nblocks) put(std::integral_constant<int, next>{});
        };
        auto stage_issue = [&]() {
            if (t + 2 < nblocks) issue((t + 2) * kBKV);
        };
        compute(t, bufc, wave_on && (!p.causal || t * kBKV <= wave_last), stage_put, stage_issue);
        __syncthreads();
    };

    issue(0);
    put(std::integral_constant<int, 0>{});
    if (nblocks > 1) issue(kBKV);
    __syncthreads();
    for (int t = 0; t < nblocks; t += 2) {
        block(t, std::integral_constant<int, 0>{});
        if (t + 1 < nblocks) block(t + 1, std::integral_constant<int, 1>{});
    }

    // The four lanes of a query hold disjoint key subsets of its sum.  Each
    // store writes 16 of the 64 bytes of four row segments; the default
    // (write-back) policy lets L2 merge the four stores of a segment before
    // it goes to memory, where device-scope stores would write each piece.
    l = across_rows(l, [](float x, float y) { return x + y; });
    const float rl = 1.0f / l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const f32x4 v = f32x4{oacc[0][e], oacc[1][e], oacc[2][e], oacc[3][e]} * rl;
        store4(rO, qok ? (unsigned(qrow) * sOr + unsigned(16 * lh + 4 * e)) * 4u : kOutOfRange, v);
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
