// fastdiv.hpp -- division by a loop-invariant divisor with a precomputed
// multiplier: one 32-bit high multiply and one correction instead of the long
// integer-division sequence.  Used by the implicit-GEMM address generator to
// split a K index into (filter tap, channel) and a tap into (r, s).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define IGC_FD_HD __host__ __device__
#else
#define IGC_FD_HD
#endif

namespace igc {

// Multiplier for divisor d >= 1: floor(2^32 / d) + 1, or 0 for d == 1.
IGC_FD_HD inline uint32_t fastdiv_magic(uint32_t d) {
    return d <= 1 ? 0u : (uint32_t)(0x100000000ull / d + 1);
}

// floor(n / d) for n, d < 2^31 given m = fastdiv_magic(d).  With m the
// rounded-up reciprocal, q = floor(n*m / 2^32) exceeds floor(n/d) by at most
// one (the rounding error of m adds less than n / 2^32 < 1), so one compare
// fixes it.
IGC_FD_HD inline uint32_t fastdiv(uint32_t n, uint32_t d, uint32_t m) {
    // both arms computed, then selected: no branch inside a caller's loop
    const uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
    const uint32_t q = m ? hi : n;
    return q * d > n ? q - 1 : q;
}

}  // namespace igc
