// attn_splitkv_kernel.hip -- split-KV attention for decode (few queries).
//
// With one or a few query rows per head, the fused kernel's workgroup of 128
// query rows has one busy wavefront and streams the whole KV cache at one
// wavefront's pace.  Here the g query heads that share a KV head, times their
// tq queries, are the rows of 16-row tiles, up to four (rvllm post, "Matmuls
// go to cuBLAS": grouped query heads stacked as rows of one product), so K and
// V are read once per tile rather than once per query head; and the keys are
// cut into chunks, one wavefront per (outer, KV head, row tile, chunk), so the
// whole chip streams the cache.  Row tile, then KV head, vary fastest across
// wavefronts: the four wavefronts of a workgroup read the same key positions,
// of one head (several row tiles) or of neighbouring heads, which sit side by
// side in a token-major cache.
//
// attn_splitkv_d64: per chunk, the online softmax of the fused kernel (the
// same score layout, S^T = K Q^T on v_mfma_f32_16x16x4_f32 with Q scaled by
// alpha*log2(e) and the products started from minus the reference maximum,
// the reference moved only past a slack of 2^8) over 32-key blocks whose K
// and V fragments come straight from global memory (no other wavefront
// shares them); it writes the chunk's unnormalised output rows, reference
// maxima and weight sums.
// attn_splitkv_merge: per output row, M = max m_c and
// O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c (softmax over the union
// of the chunks' keys), formed over four runs of consecutive chunks (one
// pass per run, its reference moving up to each new chunk maximum) and then
// over the runs, each in order.  Fixed orders throughout: reproducible bits.
#include <hip/hip_runtime.h>

#include <cmath>

#include "attention.hpp"
#include "buffer.hpp"

namespace sgemm {

namespace {

constexpr int kBlock = 32;             // keys per block (two 16-key MFMA blocks)
constexpr float kSlackSkv = 8.0f;      // log2 of the largest weight before the reference moves

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine the four lanes l%16 + 16*h (h = 0..3) with `op` (xor shuffles over
// the lane bits 4 and 5; every lane of the four ends with the same bits:
// (l0 op l1) op (l2 op l3) in both orders the shuffles pair them).
template <typename Op>
__device__ __forceinline__ float across_quads(float v, Op op) {
    v = op(v, __shfl_xor(v, 16));
    return op(v, __shfl_xor(v, 32));
}

// Three wavefronts per SIMD fit without spills (the compiler would otherwise
// take a few registers more and drop to two).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_splitkv_d64(SplitKvArgs p) {
    const int lane = threadIdx.x & 63, lq = lane & 15, lh = lane >> 4;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= p.items) return;   // uniform across the wavefront; no barrier in this kernel
    // Row tile fastest, then KV head: the wavefronts of a workgroup read the
    // same keys (one KV head's for several row tiles, or neighbouring heads').
    const int rt = int(item % p.row_tiles);
    const long long rest = item / p.row_tiles;
    const int kv = int(rest % p.n_kv);
    const long long oc = rest / p.n_kv;
    const int c = int(oc % p.chunks);
    const long long o = oc / p.chunks;
    // Partials of one (outer, KV head, row tile) are consecutive.
    const long long slot = ((o * p.n_kv + kv) * p.row_tiles + rt) * p.chunks + c;

    // Row lq of the tile is row rt*16 + lq of the group: query head
    // kv*g + row / tq, query row % tq (rows past gq*tq idle).
    const int gq = min(p.g, p.nb_inner - kv * p.g);
    if (rt * kSkvRows >= gq * p.tq) return;   // a tile of the short last group with no row
    const int row = rt * kSkvRows + lq;
    const bool rok = row < gq * p.tq;
    const int qi = rok ? row / p.tq : 0, t = rok ? row - qi * p.tq : 0;
    const int shift = p.tk - p.tq;                  // causal: query t sees keys j <= t + shift
    const int k0 = c * p.chunk_keys, k1 = min(p.tk, k0 + p.chunk_keys);
    // Last key of the chunk any row sees, and the keys every row sees.
    const int wave_last = p.causal ? min(k1 - 1, p.tq - 1 + shift) : k1 - 1;
    const int all_see = p.causal ? min(k1, shift + 1) : k1;
    int lim = k1 - 1;                               // last key this lane's query sees
    if (p.causal) lim = min(lim, t + shift);
    const int nblocks = wave_last >= k0 ? (wave_last - k0) / kBlock + 1 : 0;

    const __amdgpu_buffer_rsrc_t rQ =
        make_rsrc(p.Q + o * p.sQ_o + (long long)kv * p.g * p.sQ_i);
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(p.K + o * p.sK_o + (long long)kv * p.sK_i + (long long)k0 * p.sK_r);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(p.V + o * p.sV_o + (long long)kv * p.sV_i + (long long)k0 * p.sV_r);
    const unsigned sKr = unsigned(p.sK_r), sVr = unsigned(p.sV_r);
    const float c2 = p.scale_log2;

    f32x4 qf[4];   // dims 16*j + 4*lh .. +3 of this lane's query, scaled
    const unsigned qrow = unsigned(qi) * unsigned(p.sQ_i) + unsigned(t) * unsigned(p.sQ_r);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        qf[j] = c2 * load4(rQ, rok ? (qrow + unsigned(16 * j + 4 * lh)) * 4u : kOutOfRange);

    float m = 0.0f, l = 0.0f;
    f32x4 negm = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 oacc[4];   // oacc[nb][e]: output dim 16*lh + 4*e + nb, unnormalised
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) oacc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int b = 0; b < nblocks; ++b) {
        const int kb0 = k0 + b * kBlock;   // first key of the block
        // K fragments: key kb0 + 16*kb + lq, dims 16*j + 4*lh (one load reads
        // 64 contiguous bytes of each of 16 key rows); V fragments:
        // key kb0 + 16*kb + 4*lh + r, dims 4*lq .. +3.  Keys past tk are
        // never read (out-of-range offset: zeros); keys past the chunk are
        // read but masked.
        f32x4 kf[4][2], vf[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = kb0 + 16 * kb + lq;
            const unsigned rowo = unsigned(key - k0) * sKr;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kf[j][kb] = load4(rK, key < p.tk ? (rowo + unsigned(16 * j + 4 * lh)) * 4u : kOutOfRange);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kb0 + 16 * kb + 4 * lh + r;
                vf[kb][r] = load4(rV, key < p.tk ? (unsigned(key - k0) * sVr + unsigned(4 * lq)) * 4u : kOutOfRange);
            }
        // sacc[kb][r]: alpha*log2(e)*score - m for key kb0 + 16*kb + 4*lh + r.
        f32x4 sacc[2];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sacc[kb] = mfma16(kf[j][kb][e], qf[j][e], j == 0 && e == 0 ? negm : sacc[kb]);
        if (kb0 + kBlock > all_see) {
            const int rel = lim - (kb0 + 4 * lh);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * kb + r > rel) sacc[kb][r] = -INFINITY;
        }
        float lm = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (kb + r > 0) lm = fmaxf(lm, sacc[kb][r]);
        if (b == 0 || __builtin_amdgcn_ballot_w64(lm > kSlackSkv)) {
            // First block: the reference goes to the row maxima (a row that
            // sees none of the chunk's keys keeps 0; its weights are all 0).
            float dm = across_quads(lm, [](float x, float y) { return fmaxf(x, y); });
            if (b == 0) {
                if (dm == -INFINITY) dm = 0.0f;
            } else {
                dm = fmaxf(dm, 0.0f);
                const float corr = exp2_fast(-dm);
                l *= corr;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) oacc[nb] *= corr;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) sacc[kb] -= dm;
            m += dm;
            negm = f32x4{-m, -m, -m, -m};
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sacc[kb][r] = exp2_fast(sacc[kb][r]);
                l += sacc[kb][r];
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) oacc[nb] = mfma16(vf[kb][r][nb], sacc[kb][r], oacc[nb]);
    }

    // Partial of this chunk: rows lq < gq*tq only.
    l = across_quads(l, [](float x, float y) { return x + y; });
    float *w = p.W + slot * kSkvItemFloats;
    if (rok) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<f32x4 *>(w + lq * 64 + 16 * lh + 4 * e) =
                f32x4{oacc[0][e], oacc[1][e], oacc[2][e], oacc[3][e]};
        if (lh == 0) {
            w[kSkvRows * 64 + lq] = l > 0.0f ? m : -INFINITY;   // an empty chunk weighs nothing
            w[kSkvRows * 64 + kSkvRows + lq] = l;
        }
    }
}

// One workgroup per output row (outer, KV head, row of the group), lane = head
// dimension.  Its four wavefronts take consecutive runs of the chunks; each
// issues the loads of up to sixteen chunks at once and folds them in chunk
// order into its run's maximum M_w, weighted output sum and weight sum
// (rescaling both sums when a chunk raises M_w); the first wavefront then
// combines the four runs in run order through LDS.
__global__ __launch_bounds__(256) void attn_splitkv_merge(SplitKvArgs p) {
    __shared__ float run_m[4], run_den[4], run_num[4][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // One workgroup per row of a group (g * tq of them; the short last
    // group's surplus rows return at once).
    const long long rowi = blockIdx.x;
    const int row = int(rowi % (p.g * p.tq));    // row of the group
    const long long okv = rowi / (p.g * p.tq);   // (outer, KV head)
    const int kv = int(okv % p.n_kv);
    const long long o = okv / p.n_kv;
    const int gq = min(p.g, p.nb_inner - kv * p.g);
    if (row >= gq * p.tq) return;   // uniform across the workgroup
    const int r = row % kSkvRows;                // row of its tile
    const long long tile = okv * p.row_tiles + row / kSkvRows;   // (outer, KV head, row tile)
    const int per = (p.chunks + 3) / 4;
    const int c0 = min(wv * per, p.chunks), c1 = min(c0 + per, p.chunks);
    const float *w = p.W + tile * p.chunks * kSkvItemFloats;
    // Chunk c's m, l and output element sit at these plus c * kSkvItemFloats.
    const float *wm = w + kSkvRows * 64 + r, *wl = w + kSkvRows * 64 + kSkvRows + r, *wo = w + r * 64 + lane;
    float M = -INFINITY, num = 0.0f, den = 0.0f;
    for (int c = c0; c < c1; c += 16) {
        float mc[16], oc[16], lc[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            mc[x] = -INFINITY;
            oc[x] = lc[x] = 0.0f;
            if (c + x < c1) {   // uniform: nothing past the run is read
                const long long off = (long long)(c + x) * kSkvItemFloats;
                mc[x] = wm[off];
                oc[x] = wo[off];
                lc[x] = wl[off];
            }
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            if (mc[x] == -INFINITY) continue;   // past the run, or a chunk that saw no key
            if (mc[x] > M) {
                const float f = exp2_fast(M - mc[x]);   // 0 while M is still -inf
                num *= f;
                den *= f;
                M = mc[x];
            }
            const float f = exp2_fast(mc[x] - M);
            num += f * oc[x];
            den += f * lc[x];
        }
    }
    run_num[wv][lane] = num;
    if (lane == 0) {
        run_m[wv] = M;
        run_den[wv] = den;
    }
    __syncthreads();
    if (wv != 0) return;
    float Mt = run_m[0];
    for (int x = 1; x < 4; ++x) Mt = fmaxf(Mt, run_m[x]);
    float tn = 0.0f, td = 0.0f;
    for (int x = 0; x < 4; ++x) {
        if (run_m[x] == -INFINITY) continue;   // an empty run (or one whose chunks saw no key)
        const float f = exp2_fast(run_m[x] - Mt);
        tn += f * run_num[x][lane];
        td += f * run_den[x];
    }
    const int qi = row / p.tq, t = row - qi * p.tq;
    p.O[o * p.sO_o + (long long)(kv * p.g + qi) * p.sO_i + (long long)t * p.sO_r + lane] = tn / td;
}

}  // namespace

int launch_splitkv(const SplitKvPlan &sp, hipStream_t stream, std::string &why) {
    const SplitKvArgs &a = sp.args;
    const long long rows = a.items / a.chunks / a.row_tiles * a.g * a.tq;   // (outer, KV head) x g * tq
    hipLaunchKernelGGL(attn_splitkv_d64, dim3(unsigned((a.items + 3) / 4)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {   // the merge only after the partials' launch went in
        hipLaunchKernelGGL(attn_splitkv_merge, dim3(unsigned(rows)), dim3(256), 0, stream, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess) {
        why = std::string("split-KV attention launch failed: ") + hipGetErrorString(e);
        return kErrHip;
    }
    return kOk;
}

}  // namespace sgemm
