// Exact rounding of a double to IEEE binary16 (nearest, ties to even), in one
// step from the double's bits.  Converting through float would round twice
// and can land on a binary16 tie that the exact value is not on.
//
// Usable from device code (HIP) and from plain host C++ (DA_HD expands to
// nothing there), so the host build can check it against other converters.
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define DA_HD __host__ __device__
#else
#define DA_HD
#endif

namespace da {

DA_HD inline uint16_t f64_to_f16_rne(double x) {
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const int exp = (int)((u >> 52) & 0x7FF);
    const uint64_t frac = u & ((1ull << 52) - 1);
    if (exp == 0x7FF) return (uint16_t)(sign | 0x7C00u | (frac ? 0x200u : 0u));   // inf / nan
    if (exp == 0) return sign;            // zero or a double subnormal (< 2^-1022): rounds to 0
    const int e = exp - 1023;             // |x| = M * 2^(e-52), M = 2^52 + frac
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    const uint64_t M = (1ull << 52) | frac;
    // normal binary16 keeps 11 significant bits: shift 42; subnormal: units of 2^-24
    const int sh = (e >= -14) ? 42 : (28 - e);
    if (sh >= 64) return sign;
    uint64_t r = M >> sh;
    const uint64_t rem = M & ((1ull << sh) - 1);
    const uint64_t half = 1ull << (sh - 1);
    if (rem > half || (rem == half && (r & 1ull))) ++r;
    if (e >= -14) {
        int ee = e;
        if (r == 2048) { r = 1024; ++ee; }
        if (ee > 15) return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | (uint16_t)((ee + 15) << 10) | (uint16_t)(r - 1024));
    }
    return (uint16_t)(sign | (uint16_t)r);   // r == 1024 encodes the smallest normal
}

}  // namespace da
