// Division by a launch constant as a multiply-high and a shift (host set-up
// and host reference; kernels apply the same two steps with __umulhi).
//
// For 0 <= n < 2^31 and a divisor d >= 1 with l = ceil(log2 d), the
// multiplier m = floor(2^(31 + l) / d) + 1 lies in [2^31, 2^32) and
// floor(n / d) = floor(m n / 2^(31 + l)) (Granlund and Montgomery, "Division
// by invariant integers using multiplication", 1994, the N-bit case with
// N = 31). With the high word h = floor(m n / 2^32) that is h >> (l - 1):
// the low word adds less than one unit at that position. d = 1 is stored as
// m = 0 (the quotient is n).
#pragma once

#include <stdint.h>

namespace gqa {

struct FastDiv {
    unsigned int m;  // 0: d == 1
    int sh;          // l - 1
};

inline FastDiv fastdiv_for(int d) {
    FastDiv f{0u, 0};
    if (d <= 1) return f;
    int l = 0;
    while ((1LL << l) < d) ++l;
    f.m = (unsigned int)((1ULL << (31 + l)) / (unsigned long long)d + 1ULL);
    f.sh = l - 1;
    return f;
}

// floor(n / d) for 0 <= n < 2^31, as the kernels compute it
inline int fastdiv_apply(int n, FastDiv f) {
    if (!f.m) return n;
    return (int)((unsigned int)(((unsigned long long)(unsigned int)n * f.m) >> 32) >> f.sh);
}

}  // namespace gqa
