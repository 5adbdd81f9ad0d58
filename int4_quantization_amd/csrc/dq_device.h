// dq_device.h -- device helpers shared by the libdquant kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dq_div.h"

namespace dq {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // four waves

// ---------------------------------------------------------------------------
// XCD-aware block order.  The dispatcher hands workgroup `bid` to XCD
// bid % 8; this bijection on [0, nb) gives each XCD one contiguous range of
// logical blocks, so rows that share parameters (an expert's smooth row, a
// batch's modulation vectors) stay in that XCD's L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t xcd_block(int64_t bid, int64_t nb)
{
    const int64_t x = bid & 7, idx = bid >> 3;
    const int64_t per = nb >> 3, rem = nb & 7;
    return x * per + (x < rem ? x : rem) + idx;
}

// Division helpers (DivMagic, div_by, div_by_row, div_by_const,
// row_divisor_in_range) live in dq_div.h, which the CPU tests also compile.

// ---------------------------------------------------------------------------
// Wave-wide reductions.  Lanes combine in a fixed butterfly: quad swaps and
// row mirrors through DPP, the 16-lane swap through ds_swizzle, and the two
// 32-lane halves through readlane.  Every lane ends with the same value and
// the order never changes, so sums are deterministic.  All 64 lanes must be
// active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swz_xor16(float v)
{
    // BitMode swizzle within 32 lanes: and_mask 0x1F, or 0, xor 0x10.
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

__device__ __forceinline__ float lane_f(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
    v = op(v, dpp_f<kDppQuadXor1>(v));
    v = op(v, dpp_f<kDppQuadXor2>(v));
    v = op(v, dpp_f<kDppHalfMirror>(v));
    v = op(v, dpp_f<kDppMirror>(v));
    v = op(v, swz_xor16(v));
    return op(lane_f(v, 0), lane_f(v, 32));
}

struct MaxOp {
    __device__ float operator()(float a, float b) const { return __builtin_fmaxf(a, b); }
};
struct MinOp {
    __device__ float operator()(float a, float b) const { return __builtin_fminf(a, b); }
};
struct AddOp {
    __device__ float operator()(float a, float b) const { return a + b; }
};

// Order-preserving integer keys for float max / min reductions: for every
// non-NaN x, y: x < y  <=>  key(x) < key(y) as signed integers (-0 sorts just
// below +0).  Integer max/min need no NaN canonicalization, so each
// butterfly step is one DPP move and one integer op.
__device__ __forceinline__ int f2key(float f)
{
    const int b = __builtin_bit_cast(int, f);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key2f(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <bool MAX>
__device__ __forceinline__ int wave_reduce_key(int v)
{
    auto op = [](int a, int b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, dpp_i<0xB1>(v));
    v = op(v, dpp_i<0x4E>(v));
    v = op(v, dpp_i<0x141>(v));
    v = op(v, dpp_i<0x140>(v));
    v = op(v, __builtin_amdgcn_ds_swizzle(v, 0x401F));
    return op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}

// Wave-wide max / min of non-NaN floats (every lane gets the result).
__device__ __forceinline__ float wave_max_f(float v) { return key2f(wave_reduce_key<true>(f2key(v))); }
__device__ __forceinline__ float wave_min_f(float v) { return key2f(wave_reduce_key<false>(f2key(v))); }

__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp{}); }
__device__ __forceinline__ float wave_min(float v) { return wave_reduce(v, MinOp{}); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, AddOp{}); }

// ---------------------------------------------------------------------------
// Streaming memory access.  Tensors that are touched exactly once (the input
// rows, the codes, the dequantized output) go through non-temporal loads and
// stores, which do not allocate in the caches; measured on MI355X this
// raises sustained HBM bandwidth far above plain accesses (about 7.0 vs
// 5.2 TB/s for reads).  Parameters that many rows reuse (smooth scales,
// per-channel vectors) keep ordinary cached loads.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream16(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void* p)
{
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_stream4(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st_stream16(void* p, uint4 v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_stream8(void* p, uint2 v)
{
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_stream4(void* p, uint32_t v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ---------------------------------------------------------------------------
// Element widening (exact).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

template <int XT>  // 0: fp16, 1: bf16
__device__ __forceinline__ void widen8(const uint4 p, float (&v)[8])
{
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (XT == 1) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        } else {
            v[2 * i] = f16_lo(w[i]);
            v[2 * i + 1] = f16_hi(w[i]);
        }
    }
}

template <int XT>
__device__ __forceinline__ float widen1(const uint16_t h)
{
    if (XT == 1)
        return __builtin_bit_cast(float, static_cast<uint32_t>(h) << 16);
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Round-half-to-even to an integer code through the binary32 adder: for
// |t| < 2^22, t + 1.5*2^23 rounds at the units place with ties to even, and
// the low bits of the sum's encoding are the two's complement code.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ uint32_t code_bits(float t) { return __builtin_bit_cast(uint32_t, t + kRoundMagic); }

// Pack the low bytes of four code words into one dword (byte i = code i).
__device__ __forceinline__ uint32_t pack4_i8(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3)
{
    const uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0C0C0400u);  // [c0, c1, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x0C0C0400u);  // [c2, c3, 0, 0]
    return lo | (hi << 16);
}

// Pack eight 4-bit codes into one dword, code i in bits [4i, 4i+3].
__device__ __forceinline__ uint32_t pack8_i4(const uint32_t (&c)[8])
{
    const uint32_t even = pack4_i8(c[0], c[2], c[4], c[6]);  // byte k = code 2k
    const uint32_t odd = pack4_i8(c[1], c[3], c[5], c[7]);   // byte k = code 2k+1
    return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}

}  // namespace dq
