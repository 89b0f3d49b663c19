// Host check of the tile-order and batch-split arithmetic in plan.hpp (built with g++ by
// test_plan_host.py; no GPU).  Exits 0 and prints "ok" when every case holds.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "plan.hpp"

using namespace sgemm;

static int fails = 0;

static void check_div(uint32_t d, uint32_t n) {
    const Divisor v = make_divisor(d);
    if (divide(n, v) != n / d) {
        if (fails++ < 10) std::printf("divide(%u, %u) = %u, want %u\n", n, d, divide(n, v), n / d);
    }
}

// The order spelled out with plain division: XCD remap, then groups of
// kGroupRows tile rows, column-major inside a group.
static void reference(int w, int count, int tiles_m, int tiles_n, int &b, int &tm, int &tn) {
    if (count % 8 == 0) w = (w % 8) * (count / 8) + w / 8;
    b = w / (tiles_m * tiles_n);
    const int t = w % (tiles_m * tiles_n);
    const int group = t / (kGroupRows * tiles_n);
    const int first = group * kGroupRows;
    const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
    const int in = t - group * kGroupRows * tiles_n;
    tm = first + in % rows;
    tn = in / rows;
}

static void check_map(int batch, int tiles_m, int tiles_n) {
    const int count = batch * tiles_m * tiles_n;
    const TileMap map = make_tile_map(batch, tiles_m, tiles_n);
    std::vector<char> seen(size_t(count), 0);
    for (int w = 0; w < count; ++w) {
        int b, tm, tn, rb, rtm, rtn;
        tile_coords(map, w, b, tm, tn);
        reference(w, count, tiles_m, tiles_n, rb, rtm, rtn);
        const bool in_range = b >= 0 && b < batch && tm >= 0 && tm < tiles_m && tn >= 0 && tn < tiles_n;
        if (b != rb || tm != rtm || tn != rtn || !in_range) {
            if (fails++ < 10)
                std::printf("map %dx%dx%d: w %d -> (%d,%d,%d), want (%d,%d,%d)\n", batch, tiles_m,
                            tiles_n, w, b, tm, tn, rb, rtm, rtn);
            return;
        }
        char &s = seen[(size_t(b) * tiles_m + tm) * tiles_n + tn];
        if (s++) {
            if (fails++ < 10) std::printf("map %dx%dx%d: tile visited twice\n", batch, tiles_m, tiles_n);
            return;
        }
    }
}

// Two batch levels: the flat index b splits into (outer, inner) entries, the
// inner entry of A and B divided by their groups, as plain division does.
static void check_split(int64_t inner, int64_t gA, int64_t gB, uint32_t b) {
    const BatchSplit s = make_batch_split(inner, gA, gB);
    uint32_t o, ia, ib, ic;
    batch_entry(s, b, o, ia, ib, ic);
    const int64_t wo = b / inner, wc = b % inner;
    if (o != wo || ic != wc || ia != wc / gA || ib != wc / gB) {
        if (fails++ < 10)
            std::printf("split b %u inner %lld groups %lld,%lld -> (%u,%u,%u,%u)\n", b, (long long)inner,
                        (long long)gA, (long long)gB, o, ia, ib, ic);
    }
}

int main() {
    std::mt19937_64 rng(12345);
    const uint32_t top = 0x7fffffffu;
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
    for (int e = 12; e <= 30; ++e) {
        const uint32_t p = 1u << e;
        ds.push_back(p - 1); ds.push_back(p); ds.push_back(p + 1);
    }
    ds.push_back(top); ds.push_back(top - 1); ds.push_back(3u << 29);
    for (int i = 0; i < 2000; ++i) ds.push_back(uint32_t(rng() % top) + 1);
    for (uint32_t d : ds) {
        const uint32_t qmax = top / d;
        const uint32_t fixed[] = {0u, 1u, d - 1, d, d + 1, top, top - 1, qmax * d - 1, qmax * d,
                                  (qmax / 2) * d - 1, (qmax / 2) * d};
        for (uint32_t n : fixed)
            if (n <= top) check_div(d, n);
        for (int i = 0; i < 64; ++i) check_div(d, uint32_t(rng() % (uint64_t(top) + 1)));
    }
    const int shapes[][3] = {{1, 1, 1}, {1, 5, 3}, {120, 8, 8}, {4, 64, 64}, {3, 13, 7}, {2, 9, 17},
                             {1, 17, 1}, {7, 3, 5}, {8, 1, 1}, {5, 16, 3}, {1, 100, 41}, {16, 12, 10}};
    for (auto &s : shapes) check_map(s[0], s[1], s[2]);
    for (int i = 0; i < 200; ++i)
        check_map(int(rng() % 9) + 1, int(rng() % 40) + 1, int(rng() % 40) + 1);
    const int64_t splits[][3] = {{1, 1, 1}, {16, 1, 4}, {16, 4, 1}, {32, 8, 8}, {12, 5, 7},
                                 {7, 7, 3}, {64, 64, 1}, {3, 2, 2}, {40, 40, 40}, {1000, 1, 999}};
    for (auto &t : splits) {
        for (uint32_t b = 0; b < 4096; ++b) check_split(t[0], t[1], t[2], b);
        for (int i = 0; i < 256; ++i) check_split(t[0], t[1], t[2], uint32_t(rng() % (uint64_t(top) + 1)));
    }
    for (int i = 0; i < 2000; ++i) {
        const int64_t inner = int64_t(rng() % 100000) + 1;
        check_split(inner, int64_t(rng() % inner) + 1, int64_t(rng() % inner) + 1,
                    uint32_t(rng() % (uint64_t(top) + 1)));
    }
    if (fails) {
        std::printf("%d failures\n", fails);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
