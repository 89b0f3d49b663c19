// kernels.hip -- gfx950 (CDNA4) kernels of the strided batched fp32 product.
//
// C[b,i,j] <- alpha * sum_p A[b,i,p] B[b,p,j] (+ C[b,i,j]); operands are
// addressed through (batch, row, col) element strides (StaleyNET "GPU
// Implementation", section "The matrix product").
//
// Two kernel families:
//
//  * sgemm_mfma<Tile, AK, BK, ACC>: one workgroup per BM x BN output tile.
//    Each k step copies a BM x BK slice of A and a BK x BN slice of B from
//    global memory into LDS, then the wavefronts run fp32 matrix-core
//    instructions (v_mfma_f32_32x32x2_f32) on 32 x 32 blocks held in
//    registers.  This is the same idea as the pages' shared-memory tiled and
//    register-blocked kernels (StaleyNET "The matrix product": tiles staged in
//    fast shared memory, many outputs per thread so every value read feeds
//    several products) mapped onto CDNA4's 64-wide wavefronts, LDS and
//    matrix cores instead of 16 x 16 thread blocks.
//      - Global loads run along each operand's contiguous axis ("fast"
//        axis), whichever it is, so all four transpose cases read whole
//        cache lines (the page "PyTorch demystified 3", section "Opt. 6 -
//        Tiled matmul kernel", loads both operands the same way, which
//        strides the transposed ones).  The LDS copy keeps the global
//        orientation, padded so that fragment reads are bank-conflict free.
//      - LDS is double buffered: the next k slice is loaded into registers
//        while the matrix cores work on the current one; one barrier per k
//        step.
//      - Loads and stores go through buffer resources.  A lane outside the
//        matrix gets an offset past the resource's range, so the hardware
//        returns zero for its load and drops its store: no branch, and no
//        access outside the operands.
//      - Workgroup ids are remapped so that neighbouring tiles (which share
//        A rows and B columns) run on the same XCD and share its L2.
//  * sgemm_generic: any strides, 64-bit addressing, 64 x 64 tiles with a
//    4 x 4 register block per thread and plain fp32 FMA.  It serves layouts
//    whose offsets exceed the 32-bit buffer range.
//
// Every output element is summed by exactly one lane in an order fixed by
// the kernel and tile, so results are reproducible bit for bit.  No atomics.
#include <hip/hip_runtime.h>

#include <string>

#include "kernels.hpp"
#include "plan.hpp"

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resources: stride 0, num_records = 2^31 bytes.  Offsets at or
// beyond kOutOfRange fail the hardware range check (loads read 0, stores are
// dropped).  Word 3 holds the gfx9-family data-format bits.
constexpr unsigned kOutOfRange = 0x80000000u;
constexpr int kRecordBytes = int(0x80000000u);
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, kRecordBytes, kRsrcWord3);
}

__device__ __forceinline__ f32x4 load4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}

__device__ __forceinline__ f32x4 load2x2(__amdgpu_buffer_rsrc_t r, unsigned off0, unsigned off1) {
    u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(r, int(off0), 0, 0);
    u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(r, int(off1), 0, 0);
    u32x4 v = {lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(f32x4, v);
}

__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
}

__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, unsigned off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, int(off), 0, 0);
}

// ---------------------------------------------------------------------------
// Tile loader: an R x F tile (F along the operand's contiguous axis) held as
// one f32x4 per slot; NT threads cover it in R*F/(4*NT) slots each.  In LDS
// the tile is stored [R][F + PAD].
// ---------------------------------------------------------------------------
template <int R, int F, int PAD, int NT>
struct TileLoader {
    static constexpr int kSlotsPerRow = F / 4;
    static constexpr int kSlots = R * F / 4 / NT;
    static_assert(R * F % (4 * NT) == 0, "tile must split evenly into 4-float slots");
    f32x4 v[kSlots];

    // Row r of the tile is global row r + r_off (valid below r_lim), column
    // f is global column f + f_off (valid below f_lim); element offsets are
    // row * s_r + col * s_f from the resource base.  vec is 4, 2 or 1; for 4
    // and 2, s_f == 1 and f_lim is a multiple of vec (checked by the planner).
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int tid, unsigned r_off,
                                         unsigned r_lim, unsigned f_off, unsigned f_lim,
                                         unsigned s_r, unsigned s_f, int vec) {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            const int s = tid + q * NT;
            const unsigned rg = unsigned(s / kSlotsPerRow) + r_off;
            const unsigned fg = unsigned(s % kSlotsPerRow) * 4u + f_off;
            const bool rv = rg < r_lim;
            const unsigned row_off = rg * s_r;
            if (vec == 4) {
                v[q] = load4(rs, (rv && fg < f_lim) ? (row_off + fg) * 4u : kOutOfRange);
            } else if (vec == 2) {
                unsigned o0 = (rv && fg < f_lim) ? (row_off + fg) * 4u : kOutOfRange;
                unsigned o1 = (rv && fg + 2u < f_lim) ? (row_off + fg + 2u) * 4u : kOutOfRange;
                v[q] = load2x2(rs, o0, o1);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    unsigned fe = fg + unsigned(e);
                    v[q][e] = load1(rs, (rv && fe < f_lim) ? (row_off + fe * s_f) * 4u : kOutOfRange);
                }
            }
        }
    }

    __device__ __forceinline__ void store(float *lds, int tid) const {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            const int s = tid + q * NT;
            const int r = s / kSlotsPerRow, f = (s % kSlotsPerRow) * 4;
            *reinterpret_cast<f32x4 *>(lds + r * (F + PAD) + f) = v[q];
        }
    }
};

// Workgroup -> (batch, tile row, tile column).  The hardware hands out
// workgroup ids round-robin over the 8 XCDs; the remap gives each XCD a
// contiguous range of tile ids, and tiles are ordered in groups of 8 tile
// rows so that consecutive ids share B columns and nearby A rows.
__device__ __forceinline__ void map_tile(int wg, int total, int tiles_m, int tiles_n, int &b,
                                         int &tm, int &tn) {
    if ((total & 7) == 0) {
        const int per = total >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int per_batch = tiles_m * tiles_n;
    b = wg / per_batch;
    const int t = wg - b * per_batch;
    constexpr int kGroup = 8;
    const int group = t / (kGroup * tiles_n);
    const int first = group * kGroup;
    const int gsz = min(tiles_m - first, kGroup);
    const int in = t - group * kGroup * tiles_n;
    tm = first + in % gsz;
    tn = in / gsz;
}

// ---------------------------------------------------------------------------
// MFMA tiled kernel.
//
// k ordering inside a BK slice: lanes 0-31 of a wavefront feed the matrix
// core's k = 0 operand and lanes 32-63 its k = 1 operand.  Over 8
// consecutive k (one "group"), instruction q in 0..3 gives lane half h the
// element k = 8g + 4h + q, so a lane reading a k-contiguous tile fetches its
// 4 values of a group with one 16-byte LDS read.  A and B use the same
// ordering, so every product A[i,p]*B[p,j] is formed exactly once.
//
// Output layout of v_mfma_f32_32x32x2_f32: accumulator register r of lane l
// holds row 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32 x 32 block.
// ---------------------------------------------------------------------------
template <int T, bool AK, bool BKF, bool ACC>
__global__ __launch_bounds__(kTiles[T].wgm * kTiles[T].wgn * 64) void sgemm_mfma(MfmaArgs p) {
    constexpr TileCfg cfg = kTiles[T];
    constexpr int BM = cfg.bm, BN = cfg.bn, BK = cfg.bk;
    constexpr int NT = cfg.wgm * cfg.wgn * 64;
    constexpr int WM = BM / cfg.wgm, WN = BN / cfg.wgn;
    constexpr int TM = WM / 32, TN = WN / 32;
    static_assert(WM % 32 == 0 && WN % 32 == 0 && BK % 8 == 0, "tile shape");

    // LDS tiles: A as [BM][BK+4] (k fast) or [BK][BM+8] (m fast);
    //            B as [BN][BK+4] (k fast) or [BK][BN+8] (n fast).
    constexpr int A_R = AK ? BM : BK, A_F = AK ? BK : BM, A_PAD = AK ? 4 : 8;
    constexpr int B_R = BKF ? BN : BK, B_F = BKF ? BK : BN, B_PAD = BKF ? 4 : 8;
    constexpr int A_LD = A_F + A_PAD, B_LD = B_F + B_PAD;
    constexpr int A_SIZE = A_R * A_LD, B_SIZE = B_R * B_LD;
    static_assert(2 * 4 * (A_SIZE + B_SIZE) == cfg.lds_bytes(AK, BKF), "LDS carve-up");
    __shared__ __attribute__((aligned(16))) float smem[2 * (A_SIZE + B_SIZE)];

    const int tid = threadIdx.x;
    int b, tm, tn;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, b, tm, tn);
    const int i0 = tm * BM, j0 = tn * BN;

    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(p.A + (long long)b * p.sA_b + (long long)i0 * p.sA_m);
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(p.B + (long long)b * p.sB_b + (long long)j0 * p.sB_n);

    const unsigned m_left = unsigned(p.m - i0), n_left = unsigned(p.n - j0);
    const unsigned K = unsigned(p.k);
    const unsigned sAm = unsigned(p.sA_m), sAk = unsigned(p.sA_k);
    const unsigned sBk = unsigned(p.sB_k), sBn = unsigned(p.sB_n);

    TileLoader<A_R, A_F, A_PAD, NT> la;
    TileLoader<B_R, B_F, B_PAD, NT> lb;
    auto load_slice = [&](unsigned k0) {
        if (AK) la.load(rA, tid, 0u, m_left, k0, K, sAm, sAk, p.vec_a);
        else    la.load(rA, tid, k0, K, 0u, m_left, sAk, sAm, p.vec_a);
        if (BKF) lb.load(rB, tid, 0u, n_left, k0, K, sBn, sBk, p.vec_b);
        else     lb.load(rB, tid, k0, K, 0u, n_left, sBk, sBn, p.vec_b);
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / cfg.wgn, wn = wave % cfg.wgn;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int c = 0; c < TN; ++c) acc[a][c] = f32x16{};

    const int KT = (p.k + BK - 1) / BK;
    if (KT > 0) {
        load_slice(0u);
        la.store(smem, tid);
        lb.store(smem + A_SIZE, tid);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const float *As = smem + (kt & 1) * (A_SIZE + B_SIZE);
            const float *Bs = As + A_SIZE;
            const bool more = kt + 1 < KT;
            if (more) load_slice(unsigned(kt + 1) * BK);
#pragma unroll
            for (int g = 0; g < BK / 8; ++g) {
                const int kq = 8 * g + 4 * lh;
                f32x4 af[TM], bf[TN];
#pragma unroll
                for (int a = 0; a < TM; ++a) {
                    const int mr = wm * WM + a * 32 + lr;
                    if (AK) {
                        af[a] = *reinterpret_cast<const f32x4 *>(As + mr * A_LD + kq);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) af[a][q] = As[(kq + q) * A_LD + mr];
                    }
                }
#pragma unroll
                for (int c = 0; c < TN; ++c) {
                    const int nc = wn * WN + c * 32 + lr;
                    if (BKF) {
                        bf[c] = *reinterpret_cast<const f32x4 *>(Bs + nc * B_LD + kq);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) bf[c][q] = Bs[(kq + q) * B_LD + nc];
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int a = 0; a < TM; ++a)
#pragma unroll
                        for (int c = 0; c < TN; ++c)
                            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a][q], bf[c][q],
                                                                              acc[a][c], 0, 0, 0);
            }
            if (more) {
                float *nA = smem + ((kt + 1) & 1) * (A_SIZE + B_SIZE);
                la.store(nA, tid);
                lb.store(nA + A_SIZE, tid);
            }
            __syncthreads();
        }
    }

    // Epilogue: C = alpha*acc (+ C_old), one fused multiply-add per element
    // when accumulating.  Lanes 0-31 of a store cover 32 consecutive columns.
    const __amdgpu_buffer_rsrc_t rC =
        make_rsrc(p.C + (long long)b * p.sC_b + (long long)i0 * p.sC_m + (long long)j0 * p.sC_n);
    const unsigned sCm = unsigned(p.sC_m), sCn = unsigned(p.sC_n);
    const float alpha = p.alpha;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int c = 0; c < TN; ++c) {
            const unsigned col = unsigned(wn * WN + c * 32 + lr);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const unsigned row = unsigned(wm * WM + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3));
                const bool ok = row < m_left && col < n_left;
                const unsigned off = ok ? (row * sCm + col * sCn) * 4u : kOutOfRange;
                float v;
                if (ACC) v = __builtin_fmaf(alpha, acc[a][c][r], load1(rC, off));
                else     v = alpha * acc[a][c][r];
                store1(rC, off, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Generic kernel: any strides, 64-bit addressing.  64 x 64 tile, 256
// threads, each thread a 4 x 4 block (rows ty + 16*r, columns tx + 16*c);
// 16-deep k slices staged through LDS; grid-stride loop over tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sgemm_generic(GenericArgs p) {
    __shared__ float As[16][64 + 1];
    __shared__ float Bs[16][64 + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const long long per_batch = p.tiles_m * p.tiles_n;
    const long long total = p.batch * per_batch;
    for (long long tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const long long b = tile / per_batch, t = tile - b * per_batch;
        const long long i0 = (t / p.tiles_n) * 64, j0 = (t % p.tiles_n) * 64;
        const float *A = p.A + b * p.sA_b;
        const float *B = p.B + b * p.sB_b;
        float acc[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;
        for (long long k0 = 0; k0 < p.k; k0 += 16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = tid + 256 * q;
                const int x = e & 63, kk = e >> 6;
                const long long kg = k0 + kk;
                const long long i = i0 + x, j = j0 + x;
                As[kk][x] = (i < p.m && kg < p.k) ? A[i * p.sA_m + kg * p.sA_k] : 0.0f;
                Bs[kk][x] = (j < p.n && kg < p.k) ? B[kg * p.sB_k + j * p.sB_n] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                float av[4], bv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) av[r] = As[kk][ty + 16 * r];
#pragma unroll
                for (int c = 0; c < 4; ++c) bv[c] = Bs[kk][tx + 16 * c];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
            }
            __syncthreads();
        }
        float *C = p.C + b * p.sC_b;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const long long i = i0 + ty + 16 * r;
            if (i >= p.m) continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const long long j = j0 + tx + 16 * c;
                if (j >= p.n) continue;
                float *dst = C + i * p.sC_m + j * p.sC_n;
                *dst = p.accumulate ? __builtin_fmaf(p.alpha, acc[r][c], *dst) : p.alpha * acc[r][c];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch table.
// ---------------------------------------------------------------------------
namespace {

using MfmaLaunch = void (*)(const MfmaArgs &, unsigned, hipStream_t);

template <int T, bool AK, bool BKF, bool ACC>
void launch_mfma(const MfmaArgs &a, unsigned grid, hipStream_t s) {
    constexpr int nt = kTiles[T].wgm * kTiles[T].wgn * 64;
    hipLaunchKernelGGL((sgemm_mfma<T, AK, BKF, ACC>), dim3(grid), dim3(nt), 0, s, a);
}

template <int T>
constexpr void fill_row(MfmaLaunch (&tab)[kNumTiles][2][2][2]) {
    tab[T][0][0][0] = launch_mfma<T, false, false, false>;
    tab[T][0][0][1] = launch_mfma<T, false, false, true>;
    tab[T][0][1][0] = launch_mfma<T, false, true, false>;
    tab[T][0][1][1] = launch_mfma<T, false, true, true>;
    tab[T][1][0][0] = launch_mfma<T, true, false, false>;
    tab[T][1][0][1] = launch_mfma<T, true, false, true>;
    tab[T][1][1][0] = launch_mfma<T, true, true, false>;
    tab[T][1][1][1] = launch_mfma<T, true, true, true>;
}

struct Table {
    MfmaLaunch f[kNumTiles][2][2][2];
    Table() {
        fill_row<0>(f);
        fill_row<1>(f);
        fill_row<2>(f);
        fill_row<3>(f);
        fill_row<4>(f);
        fill_row<5>(f);
        static_assert(kNumTiles == 6, "launch table covers every tile");
    }
};

const Table &table() {
    static const Table t;
    return t;
}

}  // namespace

int launch_plan(const Plan &p, hipStream_t stream, std::string &why) {
    if (p.empty) return kOk;
    (void)hipGetLastError();  // clear a stale error left by unrelated work
    if (p.family == Family::Generic) {
        GenericArgs g;
        g.A = reinterpret_cast<const float *>(p.A);
        g.B = reinterpret_cast<const float *>(p.B);
        g.C = reinterpret_cast<float *>(p.C);
        g.sA_b = p.sA_b; g.sA_m = p.sA_m; g.sA_k = p.sA_k;
        g.sB_b = p.sB_b; g.sB_k = p.sB_k; g.sB_n = p.sB_n;
        g.sC_b = p.sC_b; g.sC_m = p.sC_m; g.sC_n = p.sC_n;
        g.m = p.m; g.n = p.n; g.k = p.k; g.batch = p.batch;
        g.tiles_m = p.tiles_m; g.tiles_n = p.tiles_n;
        g.alpha = p.alpha; g.accumulate = p.accumulate;
        hipLaunchKernelGGL(sgemm_generic, dim3(unsigned(p.workgroups)), dim3(256), 0, stream, g);
    } else {
        MfmaArgs a;
        a.A = reinterpret_cast<const float *>(p.A);
        a.B = reinterpret_cast<const float *>(p.B);
        a.C = reinterpret_cast<float *>(p.C);
        a.sA_b = p.sA_b; a.sA_m = p.sA_m; a.sA_k = p.sA_k;
        a.sB_b = p.sB_b; a.sB_k = p.sB_k; a.sB_n = p.sB_n;
        a.sC_b = p.sC_b; a.sC_m = p.sC_m; a.sC_n = p.sC_n;
        a.m = int(p.m); a.n = int(p.n); a.k = int(p.k);
        a.tiles_m = int(p.tiles_m); a.tiles_n = int(p.tiles_n);
        a.vec_a = p.vec_a; a.vec_b = p.vec_b;
        a.alpha = p.alpha;
        table().f[p.tile][p.a_kfast][p.b_kfast][p.accumulate ? 1 : 0](a, unsigned(p.workgroups), stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        why = std::string("kernel launch failed: ") + hipGetErrorString(e);
        return kErrHip;
    }
    return kOk;
}

}  // namespace sgemm
