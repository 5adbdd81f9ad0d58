// antiquantize.hip -- element-wise dequantization on gfx950
// (AntiQuantize, 功能说明: PER_TENSOR / PER_CHANNEL / PER_TOKEN / PER_GROUP,
// 表1 kDim, 表2 groupSize).
//
// A wave owns a tile of RB rows x 1024 columns: lane l holds the 16
// contiguous elements [16c, 16c + 16) of column-vector c = strip*64 + l, so
// each row of the tile is one 16-byte load per lane (1 KiB per wave,
// coalesced) and 32 (bf16/fp16) or 64 (fp32) bytes of stores per lane.  All
// RB loads are issued before any arithmetic so RB KiB per wave are in
// flight.  Parameters that vary along n (PER_CHANNEL, PER_GROUP with
// kDim = 0) are loaded once per tile into VGPRs -- a 16-element vector
// never straddles a group because groupSize is a multiple of 32, and a
// 16-row tile never straddles a kDim = 0 group for the same reason.
// PER_TOKEN parameters are wave-uniform per row; PER_GROUP kDim = 1 needs
// one parameter per lane per row.
//
// Arithmetic (the page omits the formula; the library's reading):
//   dst = RN(RN(src + offset) * scale)   or   RN(src * scale)
// in binary32 (no contraction), then one round-to-nearest-even conversion
// to bf16 / fp16 (or none for fp32).

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

constexpr int kRB = 16;  // rows per wave tile

enum AqPolicyKind : int { PK_TENSOR = 0, PK_CHANNEL = 1, PK_TOKEN = 2, PK_GROUP_N = 3, PK_GROUP_M = 4 };

struct AqArgs {
    const void* src;
    const float* scale;
    const float* offset;
    int64_t m, n;
    int64_t gs;        // group size (PER_GROUP)
    int64_t n_groups;  // ceil(n / gs) for kDim = 1
    void* dst;
    int64_t strips;    // ceil(n / 1024)
    int64_t tiles;     // strips * ceil(m / kRB)
    int64_t nblocks;
};

// 16 source bytes -> 16 floats (exact).
template <int SRC>
__device__ __forceinline__ void decode16(const uint4 raw, float (&v)[16])
{
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (SRC == SRC_I8) {
            v[4 * i + 0] = static_cast<float>(static_cast<int8_t>(w[i] & 0xFFu));
            v[4 * i + 1] = static_cast<float>(static_cast<int8_t>((w[i] >> 8) & 0xFFu));
            v[4 * i + 2] = static_cast<float>(static_cast<int8_t>((w[i] >> 16) & 0xFFu));
            v[4 * i + 3] = static_cast<float>(static_cast<int8_t>(w[i] >> 24));
        } else {
            // gfx950 converts OCP E4M3FN (NaN only at 0x7F / 0xFF, max 448).
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
            v[4 * i + 0] = lo[0];
            v[4 * i + 1] = lo[1];
            v[4 * i + 2] = hi[0];
            v[4 * i + 3] = hi[1];
        }
    }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
    return lo | (hi << 16);
}

// The binary32 product must be rounded to fp32 before the fp16 rounding.
// hipcc otherwise folds "multiply, then convert to f16" into
// v_fma_mixlo_f16, which rounds once; the empty asm makes the fp32 value a
// materialized register (it emits no instruction).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    __asm__("" : "+v"(a));
    __asm__("" : "+v"(b));
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(a));
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(b));
    return lo | (hi << 16);
}

template <int DST>
__device__ __forceinline__ void store16(void* dst_row, int64_t j0, const float (&t)[16])
{
    if (DST == DST_F32) {
        float4* d = reinterpret_cast<float4*>(static_cast<float*>(dst_row) + j0);
        d[0] = make_float4(t[0], t[1], t[2], t[3]);
        d[1] = make_float4(t[4], t[5], t[6], t[7]);
        d[2] = make_float4(t[8], t[9], t[10], t[11]);
        d[3] = make_float4(t[12], t[13], t[14], t[15]);
    } else {
        uint32_t p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            p[i] = DST == DST_BF16 ? pack_bf16x2(t[2 * i], t[2 * i + 1]) : pack_f16x2(t[2 * i], t[2 * i + 1]);
        uint4* d = reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst_row) + j0);
        d[0] = make_uint4(p[0], p[1], p[2], p[3]);
        d[1] = make_uint4(p[4], p[5], p[6], p[7]);
    }
}

__device__ __forceinline__ void load16f(const float* p, float (&v)[16])
{
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 f = q[i];
        v[4 * i + 0] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}

template <int SRC, int DST, int PK, bool OFF>
__global__ __launch_bounds__(kBlock) void aq_kernel(AqArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t tile = xcd_block(blockIdx.x, a.nblocks) * 4 + wave;
    if (tile >= a.tiles)
        return;
    const int64_t strip = tile % a.strips;
    const int64_t i0 = (tile / a.strips) * kRB;
    const int64_t j0 = (strip * kWave + lane) * 16;
    if (j0 >= a.n)
        return;  // right edge of the last strip; nothing below synchronizes
    const int rows = static_cast<int>(a.m - i0 < kRB ? a.m - i0 : kRB);

    // Issue all loads of the tile first.
    const uint8_t* src = static_cast<const uint8_t*>(a.src);
    uint4 raw[kRB];
#pragma unroll
    for (int r = 0; r < kRB; ++r)
        if (r < rows)
            raw[r] = *reinterpret_cast<const uint4*>(src + (i0 + r) * a.n + j0);

    // Parameters that stay fixed over the tile.
    float sv[16], ov[16];
    float s_u = 0.0f, o_u = 0.0f;
    if (PK == PK_TENSOR) {
        s_u = a.scale[0];
        if (OFF)
            o_u = a.offset[0];
    } else if (PK == PK_CHANNEL || PK == PK_GROUP_M) {
        const int64_t base = PK == PK_CHANNEL ? j0 : (i0 / a.gs) * a.n + j0;
        load16f(a.scale + base, sv);
        if (OFF)
            load16f(a.offset + base, ov);
    }

    const int64_t out_elem = DST == DST_F32 ? 4 : 2;
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
        if (r >= rows)
            continue;  // predicated, keeps raw[] in registers
        const int64_t i = i0 + r;
        float v[16];
        decode16<SRC>(raw[r], v);
        float s1 = s_u, o1 = o_u;
        if (PK == PK_TOKEN) {
            s1 = a.scale[i];
            if (OFF)
                o1 = a.offset[i];
        } else if (PK == PK_GROUP_N) {
            const int64_t p = i * a.n_groups + j0 / a.gs;
            s1 = a.scale[p];
            if (OFF)
                o1 = a.offset[p];
        }
        float t[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const bool per_elem = PK == PK_CHANNEL || PK == PK_GROUP_M;
            const float s = per_elem ? sv[e] : s1;
            if (OFF) {
                const float o = per_elem ? ov[e] : o1;
                const float u = v[e] + o;
                t[e] = u * s;
            } else {
                t[e] = v[e] * s;
            }
        }
        store16<DST>(static_cast<uint8_t*>(a.dst) + i * a.n * out_elem, j0, t);
    }
}

using KernelFn = void (*)(AqArgs);

template <int SRC, int DST, bool OFF>
KernelFn pick_pk(int pk)
{
    switch (pk) {
    case PK_TENSOR: return aq_kernel<SRC, DST, PK_TENSOR, OFF>;
    case PK_CHANNEL: return aq_kernel<SRC, DST, PK_CHANNEL, OFF>;
    case PK_TOKEN: return aq_kernel<SRC, DST, PK_TOKEN, OFF>;
    case PK_GROUP_N: return aq_kernel<SRC, DST, PK_GROUP_N, OFF>;
    case PK_GROUP_M: return aq_kernel<SRC, DST, PK_GROUP_M, OFF>;
    }
    return nullptr;
}

template <int SRC, int DST>
KernelFn pick_off(int pk, bool off)
{
    return off ? pick_pk<SRC, DST, true>(pk) : pick_pk<SRC, DST, false>(pk);
}

template <int SRC>
KernelFn pick_dst(int dst, int pk, bool off)
{
    switch (dst) {
    case DST_BF16: return pick_off<SRC, DST_BF16>(pk, off);
    case DST_F16: return pick_off<SRC, DST_F16>(pk, off);
    case DST_F32: return pick_off<SRC, DST_F32>(pk, off);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_antiquantize(const AqPlan& p, hipStream_t stream)
{
    int pk = p.policy;  // DQ_PER_TENSOR .. DQ_PER_TOKEN map to the same numbers
    if (p.policy == DQ_PER_GROUP)
        pk = p.k_dim == 1 ? PK_GROUP_N : PK_GROUP_M;
    KernelFn fn = p.src_kind == SRC_I8 ? pick_dst<SRC_I8>(p.dst_kind, pk, p.offset != nullptr)
                                       : pick_dst<SRC_F8E4M3>(p.dst_kind, pk, p.offset != nullptr);
    if (!fn)
        return hipErrorInvalidValue;
    AqArgs a{};
    a.src = p.src;
    a.scale = p.scale;
    a.offset = p.offset;
    a.m = p.m;
    a.n = p.n;
    a.gs = p.group_size > 0 ? p.group_size : 1;
    a.n_groups = (p.n + a.gs - 1) / a.gs;
    a.dst = p.dst;
    a.strips = (p.n + 1023) / 1024;
    a.tiles = a.strips * ((p.m + kRB - 1) / kRB);
    a.nblocks = (a.tiles + 3) / 4;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(a.nblocks)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace dq
