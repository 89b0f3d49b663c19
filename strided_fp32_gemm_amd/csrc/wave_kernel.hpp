// wave_kernel.hpp -- the direct wavefront kernel for gfx950.
//
// C[b,i,j] <- alpha * sum_p A[b,i,p] B[b,p,j] (+ C[b,i,j]) (StaleyNET "GPU
// Implementation", section "The matrix product").
//
// One wavefront per workgroup owns a WM x WN output tile made of 16 x 16
// matrix-core blocks (v_mfma_f32_16x16x4_f32).  Operand fragments go straight
// from global memory into the registers the matrix core reads: no LDS and no
// barriers, so a SIMD can hold many such wavefronts and interleave their
// memory latency.  This is the path for products whose k is short or whose
// tiles are few (attention scores, skinny and tiny shapes), where a
// workgroup-wide LDS pipeline spends most of its life waiting for one slice.
//
//  - Fragment of a 16-row block for k group g (16 consecutive k): lane l
//    holds rows l%16 and k = 16g + 4*(l/16) + q, q = 0..3.  A k-contiguous
//    operand delivers those 4 values with one 16-byte load; otherwise 4
//    element loads, each of which reads 16 consecutive lanes' worth of the
//    contiguous axis.
//  - The matrix core is fed B's fragment as its first operand and A's as its
//    second, so it produces C^T blocks: register r of lane l is
//    C[row l%16][column 4*(l/16) + r].  Each lane therefore owns 4 adjacent
//    columns of one row and writes them with a single 16-byte store.
//  - Two fragment sets alternate: group g+1 is in flight while group g is
//    multiplied.  Loads past the end of k fail the buffer range check and
//    read zeros, so the load sequence is the same in every iteration.
//
// Split variant (SPLIT, p.ksplit = S wavefronts per workgroup, 2 <= S <=
// the tile's max_split): the S wavefronts share one output tile; wavefront w takes
// the k groups w, w + S, w + 2S, ... and keeps its own partial tile.  After
// the loop wavefronts 1 .. S-1 leave their partials in LDS and wavefront 0
// adds them to its own in the order w = 1, 2, ..., S-1 and runs the
// epilogue.  This is for products with few tiles and a long k (skinny
// shapes: a few rows or columns), where one wavefront per tile leaves most
// of the chip idle and too few loads in flight to stream the long operand
// at HBM speed.
//
// Summation order per output is fixed (k groups in order, then the split
// partials in wavefront order), so results are reproducible bit for bit.
// No atomics.
#pragma once

#include "mfma_kernel.hpp"

namespace sgemm {

template <int W, bool AK, bool BKF, bool AV4, bool BV4, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 64 * kWaveTiles[W].max_split : 64) void sgemm_wave(MfmaArgs p) {
    constexpr WaveCfg cfg = kWaveTiles[W];
    constexpr int WM = cfg.bm, WN = cfg.bn;
    constexpr int TM = WM / 16, TN = WN / 16;
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile shape");

    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lh = lane >> 4;
    // This wavefront's share of k: groups wid, wid + S, ... (wid = 0, S = 1
    // unless SPLIT).
    const int S = SPLIT ? p.ksplit : 1;
    const int wid = SPLIT ? __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6) : 0;
    int b, tm, tn;
    tile_coords(p.map, blockIdx.x, b, tm, tn);
    const int i0 = tm * WM, j0 = tn * WN;

    uint32_t bo, ba, bb, bc;
    batch_entry(p.split, uint32_t(b), bo, ba, bb, bc);
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A + (long long)bo * p.sA_b + (long long)ba * p.sA_i + (long long)i0 * p.sA_m);
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(p.B + (long long)bo * p.sB_b + (long long)bb * p.sB_i + (long long)j0 * p.sB_n);
    const unsigned m_left = unsigned(p.m - i0), n_left = unsigned(p.n - j0);
    const unsigned K = unsigned(p.k);
    const unsigned sAm = unsigned(p.sA_m), sAk = unsigned(p.sA_k);
    const unsigned sBk = unsigned(p.sB_k), sBn = unsigned(p.sB_n);

    // Per-lane row (of A) and column (of B) offsets, fixed for the tile.
    unsigned a_row[TM], b_col[TN];
    bool a_ok[TM], b_ok[TN];
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const unsigned row = unsigned(a * 16 + lr);
        a_ok[a] = row < m_left;
        a_row[a] = row * sAm;
    }
#pragma unroll
    for (int c = 0; c < TN; ++c) {
        const unsigned col = unsigned(c * 16 + lr);
        b_ok[c] = col < n_left;
        b_col[c] = col * sBn;
    }

    auto fetch = [&](unsigned g, f32x4 (&fa)[TM], f32x4 (&fb)[TN]) {
        const unsigned kb = 16u * g + 4u * unsigned(lh);
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            if constexpr (AK && AV4) {
                fa[a] = load4(rA, (a_ok[a] && kb < K) ? (a_row[a] + kb) * 4u : kOutOfRange);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const unsigned k = kb + unsigned(q);
                    fa[a][q] = load1(rA, (a_ok[a] && k < K) ? (a_row[a] + k * sAk) * 4u : kOutOfRange);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < TN; ++c) {
            if constexpr (BKF && BV4) {
                fb[c] = load4(rB, (b_ok[c] && kb < K) ? (b_col[c] + kb) * 4u : kOutOfRange);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const unsigned k = kb + unsigned(q);
                    fb[c][q] = load1(rB, (b_ok[c] && k < K) ? (b_col[c] + k * sBk) * 4u : kOutOfRange);
                }
            }
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int c = 0; c < TN; ++c) acc[a][c] = f32x4{};

    auto multiply = [&](const f32x4 (&fa)[TM], const f32x4 (&fb)[TN]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int c = 0; c < TN; ++c)
                    acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[c][q], fa[a][q], acc[a][c], 0, 0, 0);
    };

    // Pairs of groups per iteration with nothing conditional inside (a
    // multiply conditional on the group count would give the accumulators
    // two incoming paths and cost register copies every iteration); an odd
    // last group is multiplied after the loop.
    const int NG_all = (p.k + 15) / 16;
    const int NG = NG_all > wid ? (NG_all - wid + S - 1) / S : 0;   // this wavefront's groups
    if (NG > 0) {
        const unsigned g0 = unsigned(wid), gs = unsigned(S);
        f32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
        fetch(g0, fa0, fb0);
        fetch(g0 + gs, fa1, fb1);
        int g = 0;
        for (; g + 1 < NG; g += 2) {
            multiply(fa0, fb0);
            fetch(g0 + unsigned(g + 2) * gs, fa0, fb0);
            multiply(fa1, fb1);
            fetch(g0 + unsigned(g + 3) * gs, fa1, fb1);
        }
        if (g < NG) multiply(fa0, fb0);
    }

    if constexpr (SPLIT) {
        // Partials of wavefronts 1 .. S-1: part[(w - 1) * TM * TN + block][lane].
        extern __shared__ f32x4 part[];
        if (wid > 0) {
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int c = 0; c < TN; ++c) part[((wid - 1) * TM * TN + a * TN + c) * 64 + lane] = acc[a][c];
        }
        __syncthreads();
        if (wid > 0) return;
        for (int w = 1; w < S; ++w) {
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int c = 0; c < TN; ++c) {
                    const f32x4 q = part[((w - 1) * TM * TN + a * TN + c) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[a][c][e] += q[e];
                }
        }
    }

    // Epilogue: lane (lr, lh) of block (a, c) holds C[a*16 + lr][c*16 + 4*lh + r]
    // (epilogue_value; the general epilogue's vector terms come through
    // their own buffer resources, out-of-range convention as for C).
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(p.C + (long long)bo * p.sC_b + (long long)bc * p.sC_i +
                                                 (long long)i0 * p.sC_m + (long long)j0 * p.sC_n);
    const unsigned sCm = unsigned(p.sC_m), sCn = unsigned(p.sC_n);
    const float alpha = p.alpha;
    const bool accumulate = p.accumulate != 0;
    const Epilogue &ep = p.epi;
    const bool has_row = ep.has_row != 0, has_col = ep.has_col != 0;
    const __amdgpu_buffer_rsrc_t rR =
        make_rsrc(has_row ? ep.row + (long long)b * ep.sR_b + (long long)i0 * ep.sR_m : p.C);
    const __amdgpu_buffer_rsrc_t rL =
        make_rsrc(has_col ? ep.col + (long long)b * ep.sL_b + (long long)j0 * ep.sL_n : p.C);
    const unsigned sRm = unsigned(ep.sR_m), sLn = unsigned(ep.sL_n);
    auto col_term = [&](unsigned col) {
        return has_col ? load1(rL, col < n_left ? col * sLn * 4u : kOutOfRange) : 0.0f;
    };
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const unsigned row = unsigned(a * 16 + lr);
        const bool rv = row < m_left;
        const float rterm = has_row ? load1(rR, rv ? row * sRm * 4u : kOutOfRange) : 0.0f;
#pragma unroll
        for (int c = 0; c < TN; ++c) {
            const unsigned col = unsigned(c * 16 + 4 * lh);
            const f32x4 v = acc[a][c];
            if (p.c_vec4) {
                const unsigned off = (rv && col < n_left) ? (row * sCm + col) * 4u : kOutOfRange;
                const f32x4 old = accumulate ? load4(rC, off) : f32x4{};
                f32x4 cv;
                if (has_col && ep.col_vec4) {
                    cv = load4(rL, col < n_left ? col * 4u : kOutOfRange);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) cv[e] = col_term(col + unsigned(e));
                }
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = epilogue_value(alpha, v[e], accumulate, ep.beta, old[e], has_row, rterm, has_col, cv[e]);
                store4(rC, off, o);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned ce = col + unsigned(e);
                    const unsigned off = (rv && ce < n_left) ? (row * sCm + ce * sCn) * 4u : kOutOfRange;
                    const float old = accumulate ? load1(rC, off) : 0.0f;
                    store1(rC, off, epilogue_value(alpha, v[e], accumulate, ep.beta, old, has_row, rterm,
                                                   has_col, col_term(ce)));
                }
            }
        }
    }
}

// LDS of the split variant: the partial tiles of wavefronts 1 .. S-1.
constexpr int wave_split_lds(int w, int splits) { return (splits - 1) * kWaveTiles[w].bm * kWaveTiles[w].bn * 4; }

template <int W, bool AK, bool BKF, bool AV4, bool BV4>
void launch_wave(const MfmaArgs &a, unsigned grid, hipStream_t s) {
    if (a.ksplit > 1) {
        const int lds = wave_split_lds(W, a.ksplit);
        static std::atomic<unsigned long long> lds_set{0};
        const void *fn = reinterpret_cast<const void *>(&sgemm_wave<W, AK, BKF, AV4, BV4, true>);
        if (lds > 64 * 1024) allow_dynamic_lds(fn, lds, lds_set);
        hipLaunchKernelGGL((sgemm_wave<W, AK, BKF, AV4, BV4, true>), dim3(grid), dim3(64 * a.ksplit), lds, s, a);
    } else {
        hipLaunchKernelGGL((sgemm_wave<W, AK, BKF, AV4, BV4, false>), dim3(grid), dim3(64), 0, s, a);
    }
}

template <int W, bool AK, bool BKF>
void fill_wave_layout(WaveTable &tab) {
    tab.f[W][AK][BKF][0][0] = launch_wave<W, AK, BKF, false, false>;
    tab.f[W][AK][BKF][0][1] = launch_wave<W, AK, BKF, false, true>;
    tab.f[W][AK][BKF][1][0] = launch_wave<W, AK, BKF, true, false>;
    tab.f[W][AK][BKF][1][1] = launch_wave<W, AK, BKF, true, true>;
}

template <int W>
void fill_wave(WaveTable &tab) {
    fill_wave_layout<W, false, false>(tab);
    fill_wave_layout<W, false, true>(tab);
    fill_wave_layout<W, true, false>(tab);
    fill_wave_layout<W, true, true>(tab);
}

}  // namespace sgemm
