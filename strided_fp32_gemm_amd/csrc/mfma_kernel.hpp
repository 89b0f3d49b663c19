// mfma_kernel.hpp -- the LDS-tiled fp32 matrix-core kernel for gfx950.
//
// C[b,i,j] <- alpha * sum_p A[b,i,p] B[b,p,j] (+ C[b,i,j]); operands are
// addressed through (batch, row, col) element strides (StaleyNET "GPU
// Implementation", section "The matrix product").
//
// One workgroup owns a BM x BN output tile.  Each k step copies a BM x BK
// slice of A and a BK x BN slice of B from global memory into LDS; the
// wavefronts then run fp32 matrix-core instructions (v_mfma_f32_32x32x2_f32
// or v_mfma_f32_16x16x4_f32) on 32 x 32 or 16 x 16 blocks accumulated in
// registers.  It is the shared-memory tiled
// and register-blocked design the pages describe (StaleyNET "The matrix
// product": tiles staged in fast shared memory, many outputs per thread so
// each value read feeds several products) mapped onto CDNA4's 64-wide
// wavefronts, LDS and matrix cores.
//
//  - Global loads run along each operand's contiguous ("fast") axis,
//    whichever it is, so all four transpose cases read whole cache lines.
//    (The tiled kernel of "PyTorch demystified 3", section "Opt. 6 - Tiled
//    matmul kernel", loads both operands one way, which strides the
//    transposed ones.)  The LDS copy keeps the global orientation, padded so
//    fragment reads are free of bank conflicts.
//  - The load width is a template parameter: 16-byte loads (contiguous,
//    16-byte aligned, extent a multiple of 4) or element loads (any stride,
//    any alignment).  Straight-line load code lets the compiler keep every
//    load of the next k slice in flight while the matrix cores work.
//  - LDS is double buffered (one barrier per k step, placed before the
//    step's last k group) and the fragments of the next k group are read
//    from LDS while the current group's matrix-core instructions run; the
//    last group reads the first fragments of the next slice, so no step
//    starts by waiting on LDS.  Scheduling-group barriers space the LDS
//    reads, global loads and LDS writes among the products.
//  - Loads and stores go through buffer resources.  A lane outside the
//    matrix gets an offset beyond the resource's range, so the hardware
//    returns zero for its load and drops its store: no branch and no access
//    outside the operands.
//  - Workgroup ids are remapped so that neighbouring tiles (which share A
//    rows and B columns) run on the same XCD and share its L2.
//
// Every output element is summed by one lane in an order fixed by the tile
// configuration, so results are reproducible bit for bit.  No atomics.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "buffer.hpp"
#include "epilogue.hpp"
#include "kernels.hpp"
#include "plan.hpp"

namespace sgemm {

// An R x F tile (F along the operand's contiguous axis) held as one f32x4
// per slot; NT threads cover its R*F/4 slots in rounds, the last round
// possibly partial.  In LDS the tile is stored [R][F + PAD].  VW is the
// global load width in floats: 4 (16-byte loads), 2 (8-byte loads, fixed
// offsets only) or 1 (element loads, any stride).
template <int R, int F, int PAD, int NT, int VW>
struct TileLoader {
    static constexpr bool V4 = VW == 4;
    static constexpr int kPieces = 4 / VW;   // loads per slot
    static constexpr int kSlotsPerRow = F / 4;
    static constexpr int kTotal = R * F / 4;
    static constexpr int kSlots = (kTotal + NT - 1) / NT;
    static_assert(F % 4 == 0, "tile rows must split into 4-float slots");
    f32x4 v[kSlots];

    static __device__ __forceinline__ bool active(int q, int tid) {
        return (kTotal % NT == 0) || q + 1 < kSlots || tid + q * NT < kTotal;
    }

    // Tile row r is global row r + r_off (valid below r_lim); tile column f
    // is global column f + f_off (valid below f_lim).  Element offsets are
    // row * s_r + col * s_f from the resource base.  With V4, s_f == 1 and
    // f_lim is a multiple of 4 (the planner checks both).
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int tid, unsigned r_off,
                                         unsigned r_lim, unsigned f_off, unsigned f_lim,
                                         unsigned s_r, unsigned s_f) {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            if (!active(q, tid)) continue;
            const int s = tid + q * NT;
            const unsigned rg = unsigned(s / kSlotsPerRow) + r_off;
            const unsigned fg = unsigned(s % kSlotsPerRow) * 4u + f_off;
            const bool rv = rg < r_lim;
            const unsigned row_off = rg * s_r;
            if constexpr (V4) {
                v[q] = load4(rs, (rv && fg < f_lim) ? (row_off + fg) * 4u : kOutOfRange);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const unsigned fe = fg + unsigned(e);
                    v[q][e] = load1(rs, (rv && fe < f_lim) ? (row_off + fe * s_f) * 4u : kOutOfRange);
                }
            }
        }
    }

    // Fixed slot offsets (bytes within one k slice, kOutOfRange for a lane
    // outside the bound that does not move with k), computed once per
    // workgroup; per slice only the buffer resource changes (SliceOffsets).
    __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, const unsigned (&off)[kSlots][kPieces]) {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            if (!active(q, threadIdx.x)) continue;
            if constexpr (VW == 4) {
                v[q] = load4(rs, off[q][0]);
            } else if constexpr (VW == 2) {
                const f32x2 lo = load2(rs, off[q][0]), hi = load2(rs, off[q][1]);
                v[q] = f32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[q][e] = load1(rs, off[q][e]);
            }
        }
    }

    // The offsets fetch() reads.  kslow: tile rows run along k (bounded per
    // slice by the resource's size) and columns f along m or n, valid below
    // lim.  Otherwise tile rows run along m or n, valid below lim, and
    // columns along k (whole slices only).
    // With VW = 2 a pair is in or out as a whole (lim is even: the planner
    // checks the extent).
    static __device__ __forceinline__ void offsets(unsigned (&off)[kSlots][kPieces], int tid, bool kslow,
                                                   unsigned lim, unsigned s_r, unsigned s_f) {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            const int s = tid + q * NT;
            const unsigned r = unsigned(s / kSlotsPerRow), f = unsigned(s % kSlotsPerRow) * 4u;
#pragma unroll
            for (int e = 0; e < kPieces; ++e) {
                const unsigned fe = f + unsigned(e * VW);
                const bool valid = kslow ? fe < lim : r < lim;
                off[q][e] = valid ? (r * s_r + fe * s_f) * 4u : kOutOfRange;
            }
        }
    }

    __device__ __forceinline__ void store(float *lds, int tid) const {
#pragma unroll
        for (int q = 0; q < kSlots; ++q) {
            if (!active(q, tid)) continue;
            const int s = tid + q * NT;
            const int r = s / kSlotsPerRow, f = (s % kSlotsPerRow) * 4;
            *reinterpret_cast<f32x4 *>(lds + r * (F + PAD) + f) = v[q];
        }
    }
};

// Matrix-core block of MF x MF outputs.
//  MF = 32: v_mfma_f32_32x32x2_f32.  Lanes 0-31 feed the k = 0 operand and
//    lanes 32-63 the k = 1 operand; accumulator register r of lane l holds
//    row 8*(r/4) + 4*(l/32) + r%4, column l%32.
//  MF = 16: v_mfma_f32_16x16x4_f32.  Lane quarter l/16 feeds k = l/16;
//    register r of lane l holds row 4*(l/16) + r, column l%16.
// k order inside a BK slice: in a group of KG = 4 * (64/MF) consecutive k,
// instruction q (0..3) gives lane group h = l/MF the element k = KG*g + 4h + q,
// so a lane reading a k-contiguous tile fetches its 4 values of a group with
// one 16-byte LDS read.  A and B use the same order, so every product
// A[i,p]*B[p,j] is formed exactly once.
template <int MF>
struct Mfma;

template <>
struct Mfma<32> {
    typedef f32x16 acc_t;
    static constexpr int kRegs = 16;
    static __device__ __forceinline__ acc_t op(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int r, int lh) { return 8 * (r >> 2) + 4 * lh + (r & 3); }
};

template <>
struct Mfma<16> {
    typedef f32x4 acc_t;
    static constexpr int kRegs = 4;
    static __device__ __forceinline__ acc_t op(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int r, int lh) { return 4 * lh + r; }
};


// The 16-byte-load layouts of the 16-wide-block tiles whose LDS lets two
// workgroups share a CU are held to two wavefronts per SIMD (at most 256
// registers per lane); the register file otherwise tips some of them to one.
// Other tiles are left alone: the cap would only make them spill (the 32-wide
// tiles hold more accumulators, and one workgroup per CU gains nothing).
template <int T, bool AK, bool BKF>
constexpr bool kTwoPerSimd = kTiles[T].mf == 16 && 2 * kTiles[T].lds_bytes(AK, BKF, 2) <= 160 * 1024;

// FX: fixed slot offsets.  Each thread's load offsets within a k slice are
// computed once; per slice only the buffer resource moves: its base steps
// along k, and its size bounds k -- for an operand whose tile rows run along
// k the size ends at row K (rows must not overlap: the planner checks
// (extent - 1) * fast stride < row stride), and for one whose tile columns
// run along k a slice past the end gets size 0 (k must be a multiple of BK).
// Without FX every slice recomputes each slot's offset and bounds check, and
// that vector arithmetic in the loop cost the 4 x 4096^3 product 5% (timing
// copies: with loads from fixed addresses it ran at 97% of peak, with the
// per-slice arithmetic kept and the loads pointed at a 16 KB window at 92%,
// like the unchanged kernel).
template <int T, bool AK, bool BKF, int AW, int BW, bool FX>
__global__ __launch_bounds__(kTiles[T].wgm * kTiles[T].wgn * 64)
__attribute__((amdgpu_waves_per_eu(AW == 4 && BW == 4 && kTwoPerSimd<T, AK, BKF> ? 2 : 1))) void sgemm_mfma(MfmaArgs p) {
    constexpr TileCfg cfg = kTiles[T];
    constexpr int BM = cfg.bm, BN = cfg.bn, BK = cfg.bk, MF = cfg.mf;
    constexpr int NT = cfg.wgm * cfg.wgn * 64;
    constexpr int WM = BM / cfg.wgm, WN = BN / cfg.wgn;
    constexpr int TM = WM / MF, TN = WN / MF;
    constexpr int KG = 4 * (64 / MF);
    constexpr int G = BK / KG;
    using M = Mfma<MF>;
    using acc_t = typename M::acc_t;
    static_assert(WM % MF == 0 && WN % MF == 0 && BK % KG == 0, "tile shape");

    // LDS tiles: A as [BM][BK+pad] (k fast) or [BK][BM+pad] (m fast);
    //            B as [BN][BK+pad] (k fast) or [BK][BN+pad] (n fast).
    constexpr int A_R = AK ? BM : BK, A_F = AK ? BK : BM, A_PAD = cfg.pad(AK, cfg.a_blocks());
    constexpr int B_R = BKF ? BN : BK, B_F = BKF ? BK : BN, B_PAD = cfg.pad(BKF, cfg.b_blocks());
    constexpr int A_LD = A_F + A_PAD, B_LD = B_F + B_PAD;
    constexpr int A_SIZE = A_R * A_LD, B_SIZE = B_R * B_LD;
    static_assert(4 * (A_SIZE + B_SIZE) == cfg.buffer_lds_bytes(AK, BKF), "LDS carve-up");
    constexpr int E_LD = cfg.epi_pitch(BKF);  // staged-epilogue row pitch
    // Dynamic LDS of cfg.lds_bytes(AK, BKF, slices) bytes: one A/B buffer
    // when the k extent is a single slice, two otherwise, and at least the
    // staged epilogue's footprint.
    extern __shared__ __attribute__((aligned(16))) float smem[];

    const int tid = threadIdx.x;
    int b, tm, tn;
    tile_coords(p.map, blockIdx.x, b, tm, tn);
    const int i0 = tm * BM, j0 = tn * BN;

    uint32_t bo, ba, bb, bc;
    batch_entry(p.split, uint32_t(b), bo, ba, bb, bc);
    const float *const baseA = p.A + (long long)bo * p.sA_b + (long long)ba * p.sA_i + (long long)i0 * p.sA_m;
    const float *const baseB = p.B + (long long)bo * p.sB_b + (long long)bb * p.sB_i + (long long)j0 * p.sB_n;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(baseA);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(baseB);

    const unsigned m_left = unsigned(p.m - i0), n_left = unsigned(p.n - j0);
    const unsigned K = unsigned(p.k);
    const unsigned sAm = unsigned(p.sA_m), sAk = unsigned(p.sA_k);
    const unsigned sBk = unsigned(p.sB_k), sBn = unsigned(p.sB_n);

    using LoaderA = TileLoader<A_R, A_F, A_PAD, NT, AW>;
    using LoaderB = TileLoader<B_R, B_F, B_PAD, NT, BW>;
    static_assert(FX || (AW != 2 && BW != 2), "8-byte loads need fixed offsets");
    unsigned offA[FX ? LoaderA::kSlots : 1][LoaderA::kPieces], offB[FX ? LoaderB::kSlots : 1][LoaderB::kPieces];
    if constexpr (FX) {
        LoaderA::offsets(offA, tid, !AK, m_left, AK ? sAm : sAk, AK ? sAk : sAm);
        LoaderB::offsets(offB, tid, !BKF, n_left, BKF ? sBn : sBk, BKF ? sBk : sBn);
    }
    // The resource of one operand for the slice starting at k0 (FX): the base
    // steps along k; when tile rows run along k the size covers the slice's
    // rows below K (min(K - k0, BK) rows of s_k floats), when columns do it
    // is the usual range, or 0 for a slice past the end.  Scalar selects
    // only: a branch here would split the loop body, and the scheduling
    // barriers order instructions within one block.
    auto slice_rsrc = [&](const float *base, unsigned k0, auto kslow, unsigned s_k) {
        const float *at = base + (long long)k0 * s_k;
        const unsigned left = K > k0 ? K - k0 : 0u;
        unsigned rec;
        if constexpr (decltype(kslow)::value) rec = (left < unsigned(BK) ? left : unsigned(BK)) * s_k * 4u;
        else rec = left ? unsigned(kRecordBytes) : 0u;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(at), 0, int(rec), kRsrcWord3);
    };
    // Issue the global loads of the k slice starting at k0.  Slices past the
    // end of k fail the range check and read zeros without touching memory.
    auto issue = [&](LoaderA &la, LoaderB &lb, unsigned k0) {
        if constexpr (FX) {
            la.fetch(slice_rsrc(baseA, k0, std::integral_constant<bool, !AK>(), sAk), offA);
            lb.fetch(slice_rsrc(baseB, k0, std::integral_constant<bool, !BKF>(), sBk), offB);
        } else {
            if constexpr (AK) la.load(rA, tid, 0u, m_left, k0, K, sAm, sAk);
            else              la.load(rA, tid, k0, K, 0u, m_left, sAk, sAm);
            if constexpr (BKF) lb.load(rB, tid, 0u, n_left, k0, K, sBn, sBk);
            else               lb.load(rB, tid, k0, K, 0u, n_left, sBk, sBn);
        }
    };
    auto put = [&](const LoaderA &la, const LoaderB &lb, int buf) {
        float *base = smem + buf * (A_SIZE + B_SIZE);
        la.store(base, tid);
        lb.store(base + A_SIZE, tid);
    };

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / cfg.wgn, wn = wave % cfg.wgn;
    const int lr = lane % MF, lh = lane / MF;

    // Which tile row / column block a (c) holds at local index i.  Blocks of
    // an operand whose LDS tile is k-fast are contiguous (block a = rows
    // 16a .. 16a+15).  For an m- (n-) fast tile of 16-wide blocks with 2 or 4
    // blocks per wavefront the blocks interleave: block a holds rows TM*i + a,
    // so the TM values a lane needs for one k sit side by side in LDS and
    // come in one 8- or 16-byte read instead of TM single-float reads.
    constexpr bool A_IL = !AK && MF == 16 && (TM == 2 || TM == 4);
    constexpr bool B_IL = !BKF && MF == 16 && (TN == 2 || TN == 4);
    auto arow_w = [&](int a, int i) { return A_IL ? TM * i + a : a * MF + i; };  // within the wavefront's rows
    auto bcol_w = [&](int c, int j) { return B_IL ? TN * j + c : c * MF + j; };
    auto arow = [&](int a, int i) { return wm * WM + arow_w(a, i); };
    auto bcol = [&](int c, int j) { return wn * WN + bcol_w(c, j); };

    // Fragments of k group g: af[a][q] = A[arow(a, lr)][KG*g + 4*lh + q],
    // bf[c][q] = B[KG*g + 4*lh + q][bcol(c, lr)].
    auto read_frags = [&](const float *As, const float *Bs, int g, f32x4 (&af)[TM],
                          f32x4 (&bf)[TN]) {
        const int kq = KG * g + 4 * lh;
        if constexpr (A_IL) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float *src = As + (kq + q) * A_LD + arow(0, lr);
                if constexpr (TM == 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
                    for (int a = 0; a < 4; ++a) af[a][q] = v[a];
                } else {
                    const f32x2 v = *reinterpret_cast<const f32x2 *>(src);
                    af[0][q] = v[0];
                    af[1][q] = v[1];
                }
            }
        } else {
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                const int mr = arow(a, lr);
                if constexpr (AK) {
                    af[a] = *reinterpret_cast<const f32x4 *>(As + mr * A_LD + kq);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) af[a][q] = As[(kq + q) * A_LD + mr];
                }
            }
        }
        if constexpr (B_IL) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float *src = Bs + (kq + q) * B_LD + bcol(0, lr);
                if constexpr (TN == 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
                    for (int c = 0; c < 4; ++c) bf[c][q] = v[c];
                } else {
                    const f32x2 v = *reinterpret_cast<const f32x2 *>(src);
                    bf[0][q] = v[0];
                    bf[1][q] = v[1];
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < TN; ++c) {
                const int nc = bcol(c, lr);
                if constexpr (BKF) {
                    bf[c] = *reinterpret_cast<const f32x4 *>(Bs + nc * B_LD + kq);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) bf[c][q] = Bs[(kq + q) * B_LD + nc];
                }
            }
        }
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int c = 0; c < TN; ++c) acc[a][c] = acc_t{};

    // Fragments of two k groups: the products of group g run from one set
    // while the next group's fragments land in the other.
    f32x4 af[2][TM], bf[2][TN];
    auto products = [&](int set) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int c = 0; c < TN; ++c) acc[a][c] = M::op(af[set][a][q], bf[set][c][q], acc[a][c]);
    };
    static_assert(G >= 2 && G % 2 == 0, "a slice holds an even number (>= 2) of k groups");
    // Per k group: LDS reads of one group's fragments, products, and (once
    // per slice) the slice's global loads and LDS writes.
    constexpr int kFragReads = (A_IL ? 4 : AK ? TM : 4 * TM) + (B_IL ? 4 : BKF ? TN : 4 * TN);
    constexpr int kProducts = 4 * TM * TN;
    constexpr int kGlobalLoads = LoaderA::kSlots * LoaderA::kPieces + LoaderB::kSlots * LoaderB::kPieces;
    constexpr int kLdsWrites = LoaderA::kSlots + LoaderB::kSlots;
    // Spacing in products: the fragment reads spread over the first 3/8 of
    // the group's products, the LDS writes over half of them (measured
    // against denser spacings on the 4 x 4096^3 product: 1.5% faster).
    constexpr int kProductsPerRead = 3 * kProducts / (8 * kFragReads) > 0 ? 3 * kProducts / (8 * kFragReads) : 1;
    constexpr int kProductsPerWrite = kProducts / (2 * kLdsWrites) > 0 ? kProducts / (2 * kLdsWrites) : 1;
    // Where the slice's loads and LDS writes share the barrier's group and
    // that group holds few products (the 64 x 64 tile of 16-wide blocks: 16)
    // and few loads (16-byte loads on both operands), the writes go first, so
    // the barrier's wait for them overlaps the loads rather than following
    // the group's last product (linear layer dW 105.6 -> 100.6 us, dX 88.1 ->
    // 86.7; with single-float loads of B, as in the spectrogram, 2% slower).
    constexpr bool kWritesFirst = G == 2 && kProducts <= 16 && AW == 4 && BW == 4;

    const int KT = (p.k + BK - 1) / BK;
    if (KT > 0) {
        LoaderA la0, la1;
        LoaderB lb0, lb1;
        // Two register sets: while slice kt is multiplied, slice kt+1 is
        // landing in one set and slice kt+2 is being requested into the
        // other, so two slices of loads are in flight per workgroup.  The
        // loop runs pairs of steps so the sets alternate statically, and
        // nothing in its body is conditional: a step only conditional on the
        // slice count would give the accumulators two incoming paths at the
        // loop's end, and the compiler reconciles those with register copies
        // on every iteration.  Requests past the end of k read zeros, and
        // moving them to the idle buffer is harmless (the loop only runs when
        // k has at least two slices, so both buffers exist).  An odd last
        // slice, already in buffer 0, is multiplied after the loop; with a
        // single slice that is the only step and buffer 1 is never touched.
        issue(la0, lb0, 0u);
        issue(la1, lb1, unsigned(BK));
        put(la0, lb0, 0);
        __syncthreads();
        read_frags(smem, smem + A_SIZE, 0, af[0], bf[0]);
        // Slice kt from LDS buffer `buf`.  After group 0's products the
        // requests for slice kt+2 go out; after group G-2's, slice kt+1
        // (requested a step ago) is written into the other buffer and the
        // slice's one barrier follows.  That buffer was last read for slice
        // kt-1 before the previous barrier, which also waited for this
        // wavefront's reads.  Each group reads the next group's fragments
        // while its products run; the last group reads group 0 of slice kt+1
        // from the other buffer, made visible by the barrier, so the next
        // step starts on fragments already in registers.
        auto step = [&](int kt, int buf, bool last, LoaderA &la_next, LoaderB &lb_next, LoaderA &la_free,
                        LoaderB &lb_free) __attribute__((always_inline)) {
            const float *As = smem + buf * (A_SIZE + B_SIZE);
            const float *An = smem + (buf ^ 1) * (A_SIZE + B_SIZE);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g + 1 < G) read_frags(As, As + A_SIZE, g + 1, af[(g + 1) & 1], bf[(g + 1) & 1]);
                else if (!last) read_frags(An, An + A_SIZE, 0, af[0], bf[0]);
                products(g & 1);
                if (!last) {
                    if (kWritesFirst && g == G - 2) put(la_next, lb_next, buf ^ 1);
                    if (g == 0) issue(la_free, lb_free, unsigned(kt + 2) * BK);
                    if (!kWritesFirst && g == G - 2) put(la_next, lb_next, buf ^ 1);
                }
                // Instruction order of the group (scheduling-group barriers):
                // the fragment reads spaced over the first products, then each
                // global load after one product, then the LDS writes spaced
                // over the following products.  Left
                // to itself the compiler issues the reads late in the group
                // and in bursts that fill the LDS queue, where a wavefront
                // stalls with products still to issue.
                if (g + 1 < G || !last) {
#pragma unroll
                    for (int i = 0; i < kFragReads; ++i) {
                        __builtin_amdgcn_sched_group_barrier(kSchedLdsRead, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kProductsPerRead, 0);
                    }
                }
                auto writes = [&] {
#pragma unroll
                    for (int i = 0; i < kLdsWrites; ++i) {
                        __builtin_amdgcn_sched_group_barrier(kSchedLdsWrite, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(kSchedMfma, kProductsPerWrite, 0);
                    }
                };
                if (kWritesFirst && !last && g == G - 2) writes();
                if (!last && g == 0) {
#pragma unroll
                    for (int i = 0; i < kGlobalLoads; ++i) {
                        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                    }
                }
                if (!kWritesFirst && !last && g == G - 2) writes();
                if (!last && g == G - 2) {
                    // A wavefront at the barrier drops its issue priority so
                    // the other workgroup's wavefront on the SIMD keeps the
                    // matrix core busy; past the barrier it has a whole
                    // group of products ready and takes priority back
                    // (s_setprio; 4 x 4096^3: 3813 -> 3792 us).
                    __builtin_amdgcn_s_setprio(0);
                    __syncthreads();
                    __builtin_amdgcn_s_setprio(1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        int kt = 0;
        for (; kt + 1 < KT; kt += 2) {
            step(kt, 0, false, la1, lb1, la0, lb0);
            step(kt + 1, 1, false, la0, lb0, la1, lb1);
        }
        if (kt < KT) step(kt, 0, true, la1, lb1, la0, lb0);
        // The staged epilogue reuses the main loop's buffers.
        __syncthreads();
    }

    // Epilogue (epilogue_value): C = alpha*acc, or one fused multiply-add
    // onto beta*C_old (+ the row and column terms of the general epilogue).
    // The vector terms come through their own buffer resources with the same
    // out-of-range convention as C.
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
    auto row_term = [&](unsigned row) {
        return has_row ? load1(rR, row < m_left ? row * sRm * 4u : kOutOfRange) : 0.0f;
    };
    auto col_term = [&](unsigned col) {
        return has_col ? load1(rL, col < n_left ? col * sLn * 4u : kOutOfRange) : 0.0f;
    };
    constexpr int R = M::kRegs;
    if (p.c_vec4) {
        // Staged: each wavefront writes its WM x WN sub-tile to its own LDS
        // region (the main loop's buffers are free after its last barrier),
        // then stores whole rows with 16-byte stores, WN/4 lanes per row.
        float *stage = smem + wave * (WM * E_LD);
        if constexpr (B_IL && TN == 4) {
            // The 4 blocks of a row hold 4 adjacent columns: one 16-byte write.
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    *reinterpret_cast<f32x4 *>(stage + arow_w(a, M::row(r, lh)) * E_LD + bcol_w(0, lr)) =
                        f32x4{acc[a][0][r], acc[a][1][r], acc[a][2][r], acc[a][3][r]};
        } else if constexpr (B_IL && TN == 2) {
            // The 2 blocks of a row hold 2 adjacent columns: one 8-byte write.
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int r = 0; r < R; ++r)
                    *reinterpret_cast<f32x2 *>(stage + arow_w(a, M::row(r, lh)) * E_LD + bcol_w(0, lr)) =
                        f32x2{acc[a][0][r], acc[a][1][r]};
        } else {
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int c = 0; c < TN; ++c)
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        stage[arow_w(a, M::row(r, lh)) * E_LD + bcol_w(c, lr)] = acc[a][c][r];
        }
        __syncthreads();
        constexpr int kQuads = WM * WN / 4;
        constexpr int kPerRow = WN / 4;
        static_assert(kQuads % 64 == 0, "wave sub-tile must split into 64-lane rounds");
#pragma unroll
        for (int i = 0; i < kQuads / 64; ++i) {
            const int quad = lane + 64 * i;
            const int row = quad / kPerRow, c4 = (quad % kPerRow) * 4;
            const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + row * E_LD + c4);
            const unsigned grow = unsigned(wm * WM + row), gcol = unsigned(wn * WN + c4);
            const unsigned off = (grow < m_left && gcol < n_left) ? (grow * sCm + gcol) * 4u : kOutOfRange;
            f32x4 o;
            if (has_row || has_col) {
                const f32x4 old = accumulate ? load4(rC, off) : f32x4{};
                const float rv = row_term(grow);
                f32x4 cv;
                if (ep.col_vec4) {
                    cv = load4(rL, gcol < n_left ? gcol * 4u : kOutOfRange);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) cv[e] = col_term(gcol + unsigned(e));
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = epilogue_value(alpha, v[e], accumulate, ep.beta, old[e], has_row, rv, has_col, cv[e]);
            } else if (accumulate) {
                const f32x4 old = load4(rC, off);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(alpha, v[e], ep.beta * old[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = alpha * v[e];
            }
            store4(rC, off, o);
        }
        return;
    }
    // Direct: every lane stores its accumulators; the MF lanes of a lane
    // group cover MF consecutive columns of one row.
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int c = 0; c < TN; ++c) {
            const unsigned col = unsigned(bcol(c, lr));
            unsigned off[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const unsigned row = unsigned(arow(a, M::row(r, lh)));
                off[r] = (row < m_left && col < n_left) ? (row * sCm + col * sCn) * 4u : kOutOfRange;
            }
            if (has_row || has_col) {
                const float cv = col_term(col);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float old = accumulate ? load1(rC, off[r]) : 0.0f;
                    store1(rC, off[r], epilogue_value(alpha, acc[a][c][r], accumulate, ep.beta, old, has_row,
                                                      row_term(unsigned(arow(a, M::row(r, lh)))), has_col, cv));
                }
            } else if (accumulate) {
                float old[R];
#pragma unroll
                for (int r = 0; r < R; ++r) old[r] = load1(rC, off[r]);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    store1(rC, off[r], __builtin_fmaf(alpha, acc[a][c][r], ep.beta * old[r]));
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) store1(rC, off[r], alpha * acc[a][c][r]);
            }
        }
    }
}

// Launch-table rows for one tile: every (A fast axis, B fast axis, A load
// width, B load width) combination.
template <int T, bool AK, bool BKF, int AW, int BW, bool FX>
void launch_mfma(const MfmaArgs &a, unsigned grid, hipStream_t s) {
    constexpr TileCfg cfg = kTiles[T];
    constexpr int nt = cfg.wgm * cfg.wgn * 64;
    const long long slices = (a.k + cfg.bk - 1) / cfg.bk;
    const int lds = cfg.lds_bytes(AK, BKF, slices);
    // Allow this kernel the largest dynamic LDS any of its launches asks for.
    static std::atomic<unsigned long long> lds_set{0};
    allow_dynamic_lds(reinterpret_cast<const void *>(&sgemm_mfma<T, AK, BKF, AW, BW, FX>),
                      cfg.lds_bytes(AK, BKF, 2), lds_set);
    hipLaunchKernelGGL((sgemm_mfma<T, AK, BKF, AW, BW, FX>), dim3(grid), dim3(nt), lds, s, a);
}

// Launch-table row of one layout: load widths 1 and 4 with the per-slice
// loader; 1, 2 and 4 with fixed offsets.
template <int T, bool AK, bool BKF>
void fill_layout(MfmaTable &tab) {
    tab.f[T][AK][BKF][0][0][0] = launch_mfma<T, AK, BKF, 1, 1, false>;
    tab.f[T][AK][BKF][0][2][0] = launch_mfma<T, AK, BKF, 1, 4, false>;
    tab.f[T][AK][BKF][2][0][0] = launch_mfma<T, AK, BKF, 4, 1, false>;
    tab.f[T][AK][BKF][2][2][0] = launch_mfma<T, AK, BKF, 4, 4, false>;
    tab.f[T][AK][BKF][0][0][1] = launch_mfma<T, AK, BKF, 1, 1, true>;
    tab.f[T][AK][BKF][0][1][1] = launch_mfma<T, AK, BKF, 1, 2, true>;
    tab.f[T][AK][BKF][0][2][1] = launch_mfma<T, AK, BKF, 1, 4, true>;
    tab.f[T][AK][BKF][1][0][1] = launch_mfma<T, AK, BKF, 2, 1, true>;
    tab.f[T][AK][BKF][1][1][1] = launch_mfma<T, AK, BKF, 2, 2, true>;
    tab.f[T][AK][BKF][1][2][1] = launch_mfma<T, AK, BKF, 2, 4, true>;
    tab.f[T][AK][BKF][2][0][1] = launch_mfma<T, AK, BKF, 4, 1, true>;
    tab.f[T][AK][BKF][2][1][1] = launch_mfma<T, AK, BKF, 4, 2, true>;
    tab.f[T][AK][BKF][2][2][1] = launch_mfma<T, AK, BKF, 4, 4, true>;
}

template <int T>
void fill_tile(MfmaTable &tab) {
    fill_layout<T, false, false>(tab);
    fill_layout<T, false, true>(tab);
    fill_layout<T, true, false>(tab);
    fill_layout<T, true, true>(tab);
}

}  // namespace sgemm
