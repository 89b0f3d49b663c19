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

template <int NW, int RW, bool ACC>
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

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + (long long)bo * p.sA_b + (long long)ba * p.sA_i);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.B + (long long)bo * p.sB_b + (long long)bb * p.sB_i);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(p.C + (long long)bo * p.sC_b + (long long)bc * p.sC_i);
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
    auto issue = [&](int n0) {
#pragma unroll
        for (int u = 0; u < SL; ++u) {
            const int s = tid + u * NT;
            const int col = n0 + (s >> 4);
            const int kk = (s & 15) * 4;
            st[u] = load4(rB, col < n && kk < k ? (unsigned(col) * sBn + unsigned(kk)) * 4u : kOutOfRange);
        }
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
    if (nblocks > 1) issue(kSN);
    __syncthreads();

    for (int t = 0; t < nblocks; ++t) {
        const int n0 = t * kSN;
        const float *Bl = lds + (t & 1) * kSBlock;
        // C_old of this block's outputs, requested before the products.
        f32x4 old[RW][4];
        if constexpr (ACC) {
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int row = row0 + 16 * r, col = n0 + 16 * kb + 4 * lh;
                    old[r][kb] = load4(rC, row < p.m && col < n ? (unsigned(row) * sCm + unsigned(col)) * 4u
                                                                : kOutOfRange);
                }
        }
        f32x4 acc[RW][4];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc[r][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // Each fragment read from LDS feeds one 4-deep chain per sub-strip
        // (back-to-back products into one accumulator run fastest here).
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const f32x4 bf =
                    *reinterpret_cast<const f32x4 *>(Bl + (16 * kb + lq) * kSPitch + 16 * g + 4 * lh);
#pragma unroll
                for (int r = 0; r < RW; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[r][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[q], af[r][g][q], acc[r][kb], 0, 0, 0);
            }
        }
        // acc[r][kb][e] is C[row0 + 16*r][n0 + 16*kb + 4*lh + e].
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int row = row0 + 16 * r, col = n0 + 16 * kb + 4 * lh;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = epilogue_value(alpha, acc[r][kb][e], ACC, beta, ACC ? old[r][kb][e] : 0.0f, false,
                                          0.0f, false, 0.0f);
                store4_device(rC, row < p.m && col < n ? (unsigned(row) * sCm + unsigned(col)) * 4u : kOutOfRange, v);
            }
        if (t + 1 < nblocks) {
            put((t + 1) & 1);
            if (t + 2 < nblocks) issue((t + 2) * kSN);
        }
        __syncthreads();
    }
}

template <int NW, int RW, bool ACC>
void launch_one(const MfmaArgs &a, unsigned grid, hipStream_t s) {
    constexpr int lds = StripCfg::lds_bytes();
    hipLaunchKernelGGL((sgemm_strip<NW, RW, ACC>), dim3(grid), dim3(NW * 64), lds, s, a);
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
