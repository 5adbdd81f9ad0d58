// dq_div.h -- the exact division steps of the libdquant kernels.
//
// Host and device: the kernels use these on the GPU, and the CPU test
// tests/test_division_proofs.py compiles this same header on the host and
// checks every claim made below (tests/division_check.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dq {

// ---------------------------------------------------------------------------
// Division by a launch constant.
// floor(x / d) = (x * mult) >> shift for 0 <= x < 2^31 and d >= 1, with
// shift = 31 + ceil(log2 d) and mult = ceil(2^shift / d) (at most 2^32):
// the round-up reciprocal of Granlund and Montgomery's division by
// invariant integers.
// ---------------------------------------------------------------------------
struct DivMagic {
    uint64_t mult;
    int shift;
};

inline DivMagic div_magic(uint64_t d)
{
    int l = 0;
    while ((uint64_t{1} << l) < d)
        ++l;
    const unsigned __int128 num = static_cast<unsigned __int128>(1) << (31 + l);
    return DivMagic{static_cast<uint64_t>((num + d - 1) / d), 31 + l};
}

__host__ __device__ __forceinline__ uint32_t div_by(uint32_t x, const DivMagic& m)
{
    return static_cast<uint32_t>((static_cast<uint64_t>(x) * m.mult) >> m.shift);
}

// ---------------------------------------------------------------------------
// Correctly rounded division by a per-row divisor.
//
// For d in [2^-60, 2^60] and r = RN(1/d) (itself a correctly rounded
// division done once per row), q0 = RN(v*r) is within an ulp of v/d, the
// residual fma(-d, q0, v) is exact, and one more fma gives RN(v/d)
// (Markstein's correction step).  Quotients so small that the residual
// could underflow (|v/d| < 2^-40) only ever meet the rounding to an integer
// code, which maps them to 0 either way.  Rows whose divisor lies outside
// the range take a true division per element instead.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ float div_by_row(float v, float d, float r)
{
    const float q0 = v * r;
    const float e = __builtin_fmaf(-d, q0, v);
    return __builtin_fmaf(e, r, q0);
}

// RN(a / D) for a constant D with rD = RN(1 / D) (computed at compile time):
// the same correction step, which returns the IEEE quotient for every a in
// [2^-100, FLT_MAX] and D in {7, 15, 127, 255} (every such binary32 a is
// checked); other a (0, tiny, inf, NaN) take a true division.
__host__ __device__ __forceinline__ float div_by_const(float a, float D, float rD)
{
    if (a >= 0x1p-100f && a <= 3.40282347e38f)
        return div_by_row(a, D, rD);
    return a / D;
}

__host__ __device__ __forceinline__ bool row_divisor_in_range(float d)
{
    return d >= 0x1p-60f && d <= 0x1p60f;  // false for 0, NaN, inf
}

}  // namespace dq
