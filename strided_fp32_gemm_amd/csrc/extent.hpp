// extent.hpp -- overflow-checked extents of strided views and address-range
// overlap, for the host-side argument checks.
#pragma once

#include <cstdint>

namespace sgemm {

inline bool mul64(int64_t x, int64_t y, int64_t &r) { return !__builtin_mul_overflow(x, y, &r); }
inline bool add64(int64_t x, int64_t y, int64_t &r) { return !__builtin_add_overflow(x, y, &r); }

// Largest element offset of a [e0, e1, e2] view with strides s*, or -1 on
// overflow.  Extents are >= 1 here.
inline int64_t last_offset(int64_t e0, int64_t s0, int64_t e1, int64_t s1, int64_t e2, int64_t s2) {
    int64_t a, b, c, t, r;
    if (!mul64(e0 - 1, s0, a) || !mul64(e1 - 1, s1, b) || !mul64(e2 - 1, s2, c)) return -1;
    if (!add64(a, b, t) || !add64(t, c, r)) return -1;
    return r;
}

// Same for a [e0, e1, e2, e3] view.
inline int64_t last_offset4(int64_t e0, int64_t s0, int64_t e1, int64_t s1, int64_t e2, int64_t s2,
                            int64_t e3, int64_t s3) {
    int64_t head = last_offset(e0, s0, e1, s1, e2, s2), tail, r;
    if (head < 0 || !mul64(e3 - 1, s3, tail) || !add64(head, tail, r)) return -1;
    return r;
}

// Do the float ranges [p, p + last_p] and [q, q + last_q] share a byte?
inline bool ranges_overlap(uintptr_t p, int64_t last_p, uintptr_t q, int64_t last_q) {
    uintptr_t p_end = p + 4u * (uintptr_t)(last_p + 1);
    uintptr_t q_end = q + 4u * (uintptr_t)(last_q + 1);
    return p < q_end && q < p_end;
}

// True if a view with these (extent, stride) axes gives every element its
// own address: sorted by stride, each axis of extent > 1 has to step past
// everything the smaller axes reach.
template <int N>
inline bool distinct_axes(const int64_t (&extent)[N], const int64_t (&stride)[N]) {
    int idx[N];
    for (int a = 0; a < N; ++a) idx[a] = a;
    for (int a = 1; a < N; ++a)
        for (int b = a; b > 0 && stride[idx[b]] < stride[idx[b - 1]]; --b) {
            const int t = idx[b]; idx[b] = idx[b - 1]; idx[b - 1] = t;
        }
    int64_t reach = 0;
    for (int a = 0; a < N; ++a) {
        const int x = idx[a];
        if (extent[x] <= 1) continue;
        if (stride[x] <= reach) return false;
        reach += (extent[x] - 1) * stride[x];
    }
    return true;
}

}  // namespace sgemm
