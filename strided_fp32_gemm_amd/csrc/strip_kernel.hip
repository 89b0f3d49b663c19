// strip_kernel.hip -- short-k matrix-core kernel with A held in registers.
//
// For k <= 64 with A and B both contiguous along k (the attention scores
// Q K^T: K read transposed is k-contiguous), the per-tile fill and drain of
// the LDS-tiled kernels dominates.  Here a workgroup owns a strip of rows
// across every column instead: each wavefront loads its 16 (or 32) rows of A once,
// into the registers the matrix core reads, and B streams through
// double-buffered LDS in 64-column blocks (the next block's loads in flight
// while the current one is multiplied, one barrier per block).  The products
// are formed as C^T = B^T A^T with v_mfma_f32_16x16x4_f32, so each lane ends
// with 4 adjacent columns of one row of C: one 16-byte store per 16x16 block,
// written while the next block's products run.
//
// The k order is that of the other 16x16 matrix-core kernels (instruction q
// of the 16-deep group g gives lane group h the element k = 16g + 4h + q), so
// this kernel writes the same bits they do.
#include <hip/hip_runtime.h>

#include "buffer.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace sgemm {

namespace {

constexpr int kSK = 64;                    // k held per row
constexpr int kSN = StripCfg::kBlockCols;  // columns per LDS block
constexpr int kSPitch = kSK + 8;           // LDS row pitch (floats): conflict-free 16-byte reads
constexpr int kSBlock = kSN * kSPitch;
static_assert(2 * kSBlock * 4 == StripCfg::lds_bytes(), "two B blocks fill the planned LDS");

// FULL: n is a multiple of the 64-column block, so every block's columns
// exist.  Then each thread's load and store offsets are computed once and a
// block only moves the buffer resources' bases along n (scalar work); per-
// block offset arithmetic and bounds checks in the loop cost the LDS-tiled
// kernel 5% of its time.
template <int NW, int RW, bool ACC, bool FULL>
__global__ __launch_bounds__(NW * 64) void sgemm_strip(MfmaArgs p) {
    constexpr int NT = NW * 64;
    constexpr int ROWS = NW * 16 * RW;
    constexpr int SL = kSN * kSK / 4 / NT;   // 16-byte slots per thread per B block
    static_assert(kSN * kSK / 4 % NT == 0, "every thread stages the same number of slots");
    extern __shared__ float lds[];           // two B blocks, [column][k]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 15, lh = lane >> 4;

    int b, tm, tn;
    tile_coords(p.map, int(blockIdx.x), b, tm, tn);
    uint32_t bo, ba, bb, bc;
    batch_entry(p.split, uint32_t(b), bo, ba, bb, bc);
    // Sub-strip r of this wavefront: rows row0 + 16*r + (0..15); lane row lq.
    const int row0 = tm * ROWS + wave * 16 * RW + lq;
    const int n = p.n, k = p.k;

    const float *const baseB = p.B + (long long)bo * p.sB_b + (long long)bb * p.sB_i;
    float *const baseC = p.C + (long long)bo * p.sC_b + (long long)bc * p.sC_i;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + (long long)bo * p.sA_b + (long long)ba * p.sA_i);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(baseB);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(baseC);
    const unsigned sAm = unsigned(p.sA_m), sBn = unsigned(p.sB_n), sCm = unsigned(p.sC_m);

    // Lane's rows of A: lane group lh holds k = 16g + 4lh + (0..3) in af[r][g].
    f32x4 af[RW][4];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = row0 + 16 * r;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int kk = 16 * g + 4 * lh;
            af[r][g] = load4(rA, row < p.m && kk < k ? (unsigned(row) * sAm + unsigned(kk)) * 4u : kOutOfRange);
        }
    }

    // B block slot s: column s/16 of the block, k = 4*(s%16) .. +3.
    f32x4 st[SL];
    // FULL: slot offsets from the block's first column, k bound folded in.
    unsigned boff[SL];
#pragma unroll
    for (int u = 0; u < SL; ++u) {
        const int s = tid + u * NT, kk = (s & 15) * 4;
        boff[u] = kk < k ? (unsigned(s >> 4) * sBn + unsigned(kk)) * 4u : kOutOfRange;
    }
    // Loads of the block at column n0; a block past the end reads zeros
    // (FULL: a resource of size 0, scalar select; otherwise the column check).
    auto issue = [&](int n0) {
        if constexpr (FULL) {
            const __amdgpu_buffer_rsrc_t rBn = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float *>(baseB + (long long)n0 * sBn), 0, n0 < n ? kRecordBytes : 0, kRsrcWord3);
#pragma unroll
            for (int u = 0; u < SL; ++u) st[u] = load4(rBn, boff[u]);
        } else {
#pragma unroll
            for (int u = 0; u < SL; ++u) {
                const int s = tid + u * NT;
                const int col = n0 + (s >> 4);
                const int kk = (s & 15) * 4;
                st[u] = load4(rB, col < n && kk < k ? (unsigned(col) * sBn + unsigned(kk)) * 4u : kOutOfRange);
            }
        }
    };
    // FULL: the lane's output offsets from a block's first column, row bound
    // folded in (row r, columns 16 kb + 4 lh .. +3).
    unsigned coff[RW][4];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int row = row0 + 16 * r;
            coff[r][kb] = row < p.m ? (unsigned(row) * sCm + unsigned(16 * kb + 4 * lh)) * 4u : kOutOfRange;
        }
    // Resource and offset of output block r, kb of the block at column n0
    // (n0 < 0: no block, every store dropped).
    auto c_rsrc = [&](int n0) {
        if constexpr (FULL)
            return __builtin_amdgcn_make_buffer_rsrc(baseC + n0, 0, n0 >= 0 ? kRecordBytes : 0, kRsrcWord3);
        else
            return rC;
    };
    auto c_off = [&](int r, int kb, int n0) {
        const int row = row0 + 16 * r, col = n0 + 16 * kb + 4 * lh;
        return FULL ? coff[r][kb]
                    : n0 >= 0 && row < p.m && col < n ? (unsigned(row) * sCm + unsigned(col)) * 4u : kOutOfRange;
    };
    auto put = [&](int buf) {
        float *Bl = lds + buf * kSBlock;
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int s = tid + u * NT;
            *reinterpret_cast<f32x4 *>(Bl + (s >> 4) * kSPitch + (s & 15) * 4) = st[u];
        }
    };

    const int nblocks = (n + kSN - 1) / kSN;
    const float alpha = p.alpha, beta = p.epi.beta;
    issue(0);
    put(0);
    issue(kSN);
    __syncthreads();

    // Software pipeline over the 64-column blocks: while block t is
    // multiplied, block t+1 (loaded during block t-1) goes into the idle LDS
    // buffer, block t+2's loads go out, and block t-1's outputs are stored,
    // each slotted between the products by scheduling-group barriers, so the
    // matrix core never waits for a store to issue.  Nothing in the loop body
    // is conditional: loads past the end read zeros, the idle buffer is never
    // read after the last block, and the stores of the block before the
    // first are dropped.
    f32x4 prev[RW][4];   // block t-1's outputs, stored during block t
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) prev[r][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int kStores = RW * 4;
    for (int t = 0; t < nblocks; ++t) {
        const int n0 = t * kSN;
        const float *Bl = lds + (t & 1) * kSBlock;
        // C_old of this block's outputs, requested before the products.
        f32x4 old[RW][4];
        if constexpr (ACC) {
            const __amdgpu_buffer_rsrc_t rCo = c_rsrc(n0);
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) old[r][kb] = load4(rCo, c_off(r, kb, n0));
        }
        f32x4 acc[RW][4];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc[r][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const __amdgpu_buffer_rsrc_t rCp = c_rsrc(n0 - kSN);
        // Fragments of k group g (4 column blocks), read one group ahead.
        f32x4 bf[2][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            bf[0][kb] = *reinterpret_cast<const f32x4 *>(Bl + (16 * kb + lq) * kSPitch + 4 * lh);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (g + 1 < 4) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    bf[(g + 1) & 1][kb] = *reinterpret_cast<const f32x4 *>(Bl + (16 * kb + lq) * kSPitch +
                                                                           16 * (g + 1) + 4 * lh);
            }
            // Each fragment feeds one 4-deep chain per sub-strip (back-to-back
            // products into one accumulator run fastest here).
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < RW; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[r][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[g & 1][kb][q], af[r][g][q],
                                                                          acc[r][kb], 0, 0, 0);
            // Group 0: next block into the idle buffer; group 1: loads of the
            // block after it; groups 2 and 3: half of the previous block's
            // stores each.
            if (g == 0) put((t + 1) & 1);
            if (g == 1) issue((t + 2) * kSN);
            if (g >= 2) {
#pragma unroll
                for (int i = (g - 2) * kStores / 2; i < (g - 1) * kStores / 2; ++i)
                    store4_device(rCp, c_off(i / 4, i % 4, n0 - kSN), prev[i / 4][i % 4]);
            }
            constexpr int kProducts = 16 * RW;
            if (g + 1 < 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kProducts / 8, 0);
                }
            }
            if (g == 0) {
#pragma unroll
                for (int i = 0; i < SL; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedLdsWrite, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
                }
            } else if (g == 1) {
#pragma unroll
                for (int i = 0; i < SL; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kStores / 2; ++i) {
                    __builtin_amdgcn_sched_group_barrier(kSchedVmemWrite, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // acc[r][kb][e] is C[row0 + 16*r][n0 + 16*kb + 4*lh + e].
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    prev[r][kb][e] = epilogue_value(alpha, acc[r][kb][e], ACC, beta, ACC ? old[r][kb][e] : 0.0f,
                                                    false, 0.0f, false, 0.0f);
    }
    const int nl = (nblocks - 1) * kSN;
    const __amdgpu_buffer_rsrc_t rCl = c_rsrc(nl);
#pragma unroll
    for (int i = 0; i < kStores; ++i) store4_device(rCl, c_off(i / 4, i % 4, nl), prev[i / 4][i % 4]);
}

template <int NW, int RW, bool ACC>
void launch_one(const MfmaArgs &a, unsigned grid, hipStream_t s) {
    constexpr int lds = StripCfg::lds_bytes();
    if (a.n % kSN == 0)
        hipLaunchKernelGGL((sgemm_strip<NW, RW, ACC, true>), dim3(grid), dim3(NW * 64), lds, s, a);
    else
        hipLaunchKernelGGL((sgemm_strip<NW, RW, ACC, false>), dim3(grid), dim3(NW * 64), lds, s, a);
}

template <int T>
void launch_tile(const MfmaArgs &a, bool accumulate, unsigned grid, hipStream_t s) {
    constexpr StripCfg c = kStripTiles[T];
    constexpr int rw = c.rows / (16 * c.waves);
    static_assert(rw * 16 * c.waves == c.rows, "rows = 16 * waves * sub-strips");
    accumulate ? launch_one<c.waves, rw, true>(a, grid, s) : launch_one<c.waves, rw, false>(a, grid, s);
}

}  // namespace

void launch_strip(const MfmaArgs &a, int tile, bool accumulate, unsigned grid, hipStream_t stream) {
    static_assert(kNumStripTiles == 4, "launch table covers every strip tile");
    switch (tile) {
    case 0: launch_tile<0>(a, accumulate, grid, stream); break;
    case 1: launch_tile<1>(a, accumulate, grid, stream); break;
    case 2: launch_tile<2>(a, accumulate, grid, stream); break;
    default: launch_tile<3>(a, accumulate, grid, stream); break;
    }
}

}  // namespace sgemm
