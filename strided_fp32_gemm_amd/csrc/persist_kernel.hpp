// persist_kernel.hpp -- the persistent short-k kernel for gfx950.
//
// C[b,i,j] <- alpha * sum_p A[b,i,p] B[b,p,j] (+ C[b,i,j]) (StaleyNET "GPU
// Implementation", section "The matrix product").
//
// For products whose whole k extent fits one LDS slab (k <= KMAX), such as
// attention scores over a 64-wide head: one tile is a single slab of A and B,
// so a workgroup per tile would spend most of its life filling its pipeline
// and draining its stores, and two workgroups sharing a SIMD drift into
// lock-step (both multiply, then both wait), leaving the matrix core idle.
// Here a fixed grid of workgroups (as many as the CUs hold) loops over the
// tiles, and each wavefront keeps everything but one barrier inside its own
// stream of matrix-core instructions:
//
//   step t (tile t in LDS slab t%2, accumulators set t%2):
//     k group 0: products | 16-byte stores of block 0 of tile t-1 |
//                requests for tile t+2's operands
//     k group 1: products | stores of block 1 | locate tile t+3
//     k group 2: products | stores of block 2 | tile t+1 (requested one
//                step earlier) from registers into slab (t+1)%2
//     k group 3: products | stores of block 3
//     barrier
//
// Loads for tiles past the end are out of range (zeros, no memory access),
// and the loop body has no run-time branches around memory operations (a
// merge of such branches makes the compiler wait for everything
// outstanding, prefetches included).
//
// Blocks are 16 x 16 (v_mfma_f32_16x16x4_f32), fed B-then-A so each lane
// owns 4 adjacent columns of C and stores them with one 16-byte store.
// Output ownership and summation order are fixed: results are reproducible
// bit for bit.  No atomics.
#pragma once

#include "mfma_kernel.hpp"

namespace sgemm {

template <int P, bool AK, bool BKF, bool ACC>
__global__ __launch_bounds__(kPersistTiles[P].wgm * kPersistTiles[P].wgn * 64) void sgemm_persist(MfmaArgs p) {
    constexpr PersistCfg cfg = kPersistTiles[P];
    constexpr int BM = cfg.bm, BN = cfg.bn, KM = cfg.kmax;
    constexpr int NT = cfg.wgm * cfg.wgn * 64;
    constexpr int WM = BM / cfg.wgm, WN = BN / cfg.wgn;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int G = KM / 16;
    static_assert(WM % 16 == 0 && WN % 16 == 0 && KM % 16 == 0, "tile shape");

    // LDS slab: A as [BM][KM+pad] (k fast) or [KM][BM+pad]; B likewise.  Two slabs.
    constexpr int A_R = AK ? BM : KM, A_F = AK ? KM : BM, A_PAD = PersistCfg::pad(AK);
    constexpr int B_R = BKF ? BN : KM, B_F = BKF ? KM : BN, B_PAD = PersistCfg::pad(BKF);
    constexpr int A_LD = A_F + A_PAD, B_LD = B_F + B_PAD;
    constexpr int A_SIZE = A_R * A_LD, B_SIZE = B_R * B_LD;
    static_assert(4 * (A_SIZE + B_SIZE) == cfg.slab_bytes(AK, BKF), "LDS carve-up");
    extern __shared__ __attribute__((aligned(16))) float smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / cfg.wgn, wn = wave % cfg.wgn;
    const int lr = lane & 15, lh = lane >> 4;
    const unsigned K = unsigned(p.k);
    const unsigned sAm = unsigned(p.sA_m), sAk = unsigned(p.sA_k);
    const unsigned sBk = unsigned(p.sB_k), sBn = unsigned(p.sB_n);
    const unsigned sCm = unsigned(p.sC_m);
    const int total = p.total_tiles;
    const int stride = gridDim.x;

    struct Tile {
        __amdgpu_buffer_rsrc_t rA, rB, rC;
        unsigned m_left, n_left;
    };
    // Tile v of the launch (v >= total gives an empty tile: every access out
    // of range).  Virtual ids keep v % 8 == this workgroup's XCD, so tile_coords
    // hands each XCD a contiguous range of tiles.
    auto locate = [&](int v) {
        Tile t;
        const bool ok = v < total;
        int b, tm, tn;
        tile_coords(p.map, ok ? v : 0, b, tm, tn);
        const int i0 = tm * BM, j0 = tn * BN;
        uint32_t bo, ba, bb, bc;
        batch_entry(p.split, uint32_t(b), bo, ba, bb, bc);
        t.rA = make_rsrc(p.A + (long long)bo * p.sA_b + (long long)ba * p.sA_i + (long long)i0 * p.sA_m);
        t.rB = make_rsrc(p.B + (long long)bo * p.sB_b + (long long)bb * p.sB_i + (long long)j0 * p.sB_n);
        t.rC = make_rsrc(p.C + (long long)bo * p.sC_b + (long long)bc * p.sC_i + (long long)i0 * p.sC_m +
                         (long long)j0 * p.sC_n);
        t.m_left = ok ? unsigned(p.m - i0) : 0u;
        t.n_left = ok ? unsigned(p.n - j0) : 0u;
        return t;
    };

    // Only 16-byte operand loads and 16-byte C rows are served here (the
    // planner checks), so the loop body has no run-time branches: a branch
    // around memory operations makes the compiler wait for every outstanding
    // one, which would also wait for the previous tile's stores.
    using LoaderA = TileLoader<A_R, A_F, A_PAD, NT, true>;
    using LoaderB = TileLoader<B_R, B_F, B_PAD, NT, true>;
    auto issue = [&](LoaderA &la, LoaderB &lb, const Tile &t) {
        if constexpr (AK) la.load(t.rA, tid, 0u, t.m_left, 0u, K, sAm, sAk);
        else              la.load(t.rA, tid, 0u, K, 0u, t.m_left, sAk, sAm);
        if constexpr (BKF) lb.load(t.rB, tid, 0u, t.n_left, 0u, K, sBn, sBk);
        else               lb.load(t.rB, tid, 0u, K, 0u, t.n_left, sBk, sBn);
    };
    auto put = [&](const LoaderA &la, const LoaderB &lb, int slab) {
        float *base = smem + slab * (A_SIZE + B_SIZE);
        la.store(base, tid);
        lb.store(base + A_SIZE, tid);
    };

    // Fragments of k group g (16 consecutive k): lane (lr, lh) reads k =
    // 16g + 4lh .. +3 of row lr of each 16-row block.
    auto read_frags = [&](const float *As, const float *Bs, int g, f32x4 (&af)[TM], f32x4 (&bf)[TN]) {
        const int kq = 16 * g + 4 * lh;
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int mr = wm * WM + a * 16 + lr;
            if constexpr (AK) {
                af[a] = *reinterpret_cast<const f32x4 *>(As + mr * A_LD + kq);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) af[a][q] = As[(kq + q) * A_LD + mr];
            }
        }
#pragma unroll
        for (int c = 0; c < TN; ++c) {
            const int nc = wn * WN + c * 16 + lr;
            if constexpr (BKF) {
                bf[c] = *reinterpret_cast<const f32x4 *>(Bs + nc * B_LD + kq);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) bf[c][q] = Bs[(kq + q) * B_LD + nc];
            }
        }
    };

    // Epilogue of the previous tile, one 16 x 16 block at a time: lane
    // (lr, lh) of block (a, c) holds C[a*16 + lr][c*16 + 4*lh + e] and writes
    // it with one 16-byte store.  When accumulating, C_old of a tile is
    // fetched at the start of the step that multiplies it, one step before
    // its stores, and ahead of the operand requests issued in that step.
    constexpr int NB = TM * TN;
    const float alpha = p.alpha, beta = p.epi.beta;  // no vector terms here (the planner checks)
    auto offset = [&](const Tile &t, int a, int c) {
        const unsigned row = unsigned(wm * WM + a * 16 + lr);
        const unsigned col = unsigned(wn * WN + c * 16 + 4 * lh);
        return (row < t.m_left && col < t.n_left) ? (row * sCm + col) * 4u : kOutOfRange;
    };
    auto fetch_old = [&](const Tile &t, f32x4 (&old)[NB]) {
#pragma unroll
        for (int x = 0; x < NB; ++x) old[x] = load4(t.rC, offset(t, x / TN, x % TN));
    };
    auto store_block = [&](const Tile &t, const f32x4 (&acc)[NB], const f32x4 (&old)[NB], int x) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = ACC ? __builtin_fmaf(alpha, acc[x][e], beta * old[x][e]) : alpha * acc[x][e];
        store4_device(t.rC, offset(t, x / TN, x % TN), o);
    };

    static_assert(G >= NB && G >= 3, "one store per k group; the other work needs 3 groups");
    auto drain = [&](const Tile &prev, const f32x4 (&pacc)[NB], const f32x4 (&pold)[NB]) {
#pragma unroll
        for (int x = 0; x < NB; ++x) store_block(prev, pacc, pold, x);
    };

    int v = blockIdx.x;
    if (v >= total) return;
    LoaderA la0, la1;
    LoaderB lb0, lb1;
    f32x4 acc0[NB], acc1[NB], old0[NB], old1[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) { acc0[x] = acc1[x] = old0[x] = old1[x] = f32x4{}; }
    Tile prev = locate(total);   // nothing to store before the first tile
    Tile cur = locate(v);
    Tile t1 = locate(v + stride);
    Tile t2 = locate(v + 2 * stride);
    issue(la0, lb0, cur);
    issue(la1, lb1, t1);
    put(la0, lb0, 0);
    __syncthreads();

    // One step multiplies tile t (slab t%2, accumulator set t%2).  Everything
    // else the step owes is slotted between its k groups, so a wavefront
    // keeps the matrix core fed while it does it:
    //   group 0: store block 0 of tile t-1; request tile t+2's operands
    //   group 1: store block 1; locate tile t+3 (scalar arithmetic)
    //   group 2: store block 2; move tile t+1 (requested a step ago) from
    //            registers to slab (t+1)%2, which nobody reads any more:
    //            tile t-1 was multiplied from it before the last barrier
    //   group 3: store block 3
    // then one barrier.  Register set "next" holds tile t+1's requests; set
    // "free" was moved to LDS a step ago and now requests tile t+2.  The loop
    // runs pairs of steps while both tiles of the pair exist, so its body has
    // no branch around memory operations (a merge of such branches would make
    // the compiler wait for everything outstanding, prefetches included); the
    // last tile and the final stores are handled after it.  Requests for
    // tiles past the end are out of range.
    auto step = [&](int slab, LoaderA &la_next, LoaderB &lb_next, LoaderA &la_free, LoaderB &lb_free,
                    f32x4 (&acc)[NB], f32x4 (&old)[NB], const f32x4 (&pacc)[NB], const f32x4 (&pold)[NB]) {
        const float *As = smem + slab * (A_SIZE + B_SIZE);
        const float *Bs = As + A_SIZE;
        if constexpr (ACC) fetch_old(cur, old);
#pragma unroll
        for (int x = 0; x < NB; ++x) acc[x] = f32x4{};
        f32x4 af[2][TM], bf[2][TN];
        read_frags(As, Bs, 0, af[0], bf[0]);
        Tile t3 = t2;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) read_frags(As, Bs, g + 1, af[(g + 1) & 1], bf[(g + 1) & 1]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int x = 0; x < NB; ++x)
                    acc[x] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[g & 1][x % TN][q], af[g & 1][x / TN][q],
                                                                  acc[x], 0, 0, 0);
            if (g < NB) store_block(prev, pacc, pold, g);
            if (g == 0) issue(la_free, lb_free, t2);
            if (g == 1) t3 = locate(v + 3 * stride);
            if (g == 2) put(la_next, lb_next, slab ^ 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        prev = cur;
        cur = t1;
        t1 = t2;
        t2 = t3;
        v += stride;
    };
    while (v + stride < total) {
        step(0, la1, lb1, la0, lb0, acc0, old0, acc1, old1);
        step(1, la0, lb0, la1, lb1, acc1, old1, acc0, old0);
    }
    if (v < total) {
        step(0, la1, lb1, la0, lb0, acc0, old0, acc1, old1);
        drain(prev, acc0, old0);
    } else {
        drain(prev, acc1, old1);
    }
}

template <int P, bool AK, bool BKF, bool ACC>
void launch_persist(const MfmaArgs &a, unsigned grid, hipStream_t s) {
    constexpr PersistCfg cfg = kPersistTiles[P];
    constexpr int nt = cfg.wgm * cfg.wgn * 64;
    constexpr int lds = 2 * cfg.slab_bytes(AK, BKF);
    static std::atomic<unsigned long long> lds_set{0};
    allow_dynamic_lds(reinterpret_cast<const void *>(&sgemm_persist<P, AK, BKF, ACC>), lds, lds_set);
    hipLaunchKernelGGL((sgemm_persist<P, AK, BKF, ACC>), dim3(grid), dim3(nt), lds, s, a);
}

// Launch-table rows: [A k-fast][B k-fast][accumulate]; the persistent
// kernel always uses 16-byte loads and stores.
template <int P, bool AK, bool BKF>
void fill_persist_layout(PersistTable &tab) {
    tab.f[P][AK][BKF][0] = launch_persist<P, AK, BKF, false>;
    tab.f[P][AK][BKF][1] = launch_persist<P, AK, BKF, true>;
}

template <int P>
void fill_persist(PersistTable &tab) {
    fill_persist_layout<P, false, false>(tab);
    fill_persist_layout<P, false, true>(tab);
    fill_persist_layout<P, true, false>(tab);
    fill_persist_layout<P, true, true>(tab);
}

}  // namespace sgemm
