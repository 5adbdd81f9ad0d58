// wq_fma.h -- when the weight dequantization with offset is one FMA.
//
// Host and device: the decode matmul kernel uses this on the GPU, and the
// CPU test tests/test_fma_dequant_proof.py compiles this same header on the
// host and checks the claim below over every offset of each T with a spread
// of scales (tests/fma_dequant_check.cpp).
//
// The weight with offset is W = RN(RN(code + o) * s) in binary32, rounded
// to T afterwards (aclnnWeightQuantMatmulAllReduce, API function, whose
// missing formula this library reads with the AntiQuantize arithmetic).  It
// equals RN(code * s + RN(o * s)), one FMA, whenever code + o and o * s are
// exact in binary32 for every code: both sides then round the same real
// (code + o) s once.
//   - code + o is exact when its bits, from the top of |code| + |o| down to
//     the last bit of o (or 2^0, the last bit of an integer code), span at
//     most 24.  For |o| < 2^23 that holds above a floor set by how far
//     below 2^0 the last bit of o can fall: an 8-bit (bf16) or 11-bit
//     (fp16) significand under a top bit of 2^3 (int4) or 2^7 (int8) needs
//     |o| >= 2^-13 (int4, bf16), 2^-10 (int4, fp16), 2^-9 (int8, bf16) or
//     2^-6 (int8, fp16).  o = 0 is exact for any code.
//   - o * s, a product of two T values, has at most 22 significant bits, so
//     it is exact when it is finite and normal: at least 2^-125 after
//     rounding keeps the exact product above 2^-126.
//   - With o = 0 the FMA is RN(code * s), the formula, for any finite s.
// Only the sign of a zero weight can differ (an exact zero sum is +0 in the
// FMA, while the formula gives code + o = +0 times a negative s = -0); a sum
// of products that starts at +0 does not show it.
#pragma once

#include <hip/hip_runtime.h>

namespace dq {

// The least nonzero |o| of the one-FMA form, by code width and T.
__host__ __device__ constexpr float wq_fma_offset_floor(bool int4, bool bf16)
{
    return int4 ? (bf16 ? 0x1p-13f : 0x1p-10f) : (bf16 ? 0x1p-9f : 0x1p-6f);
}

// Whether RN(RN(code + o) * s) = RN(code * s + os) for every code, with
// os = RN(o * s) and lo = wq_fma_offset_floor(...).
__host__ __device__ __forceinline__ bool wq_fma_exact(float o, float s, float os, float lo)
{
    const float ao = __builtin_fabsf(o), aos = __builtin_fabsf(os);
    if (ao == 0.0f)
        return __builtin_isfinite(s);
    return ao >= lo && ao < 0x1p23f && aos >= 0x1p-125f && aos < __builtin_inff();
}

}  // namespace dq
