// Unsigned division by a runtime-invariant divisor d >= 1 through a multiply
// and a shift (Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, round-up variant): with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, n / d = (umulhi(n, m) + n) >> l.
// The sum is formed in 32 bits, which is exact for n < 2^31; every caller
// indexes tensors below 2^31 elements.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define CBW_HD __host__ __device__
#else
#define CBW_HD
#endif

namespace cbw {

struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f{d, 0, 0};
    uint32_t l = 0;
    while ((1ull << l) < d)
        ++l;
    f.l = l;
    f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    return f;
}

CBW_HD inline uint32_t fastdiv(uint32_t n, const FastDiv& f)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t t = __umulhi(n, f.m);
#else
    const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
#endif
    return (t + n) >> f.l;
}

}  // namespace cbw
