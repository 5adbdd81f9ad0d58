// antiquantize.hip -- element-wise dequantization on gfx950
// (AntiQuantize, 功能说明: PER_TENSOR / PER_CHANNEL / PER_TOKEN / PER_GROUP,
// 表1 kDim, 表2 groupSize).
//
// Each wave owns one 1024-column strip and every G-th row of it (G = waves
// per strip), so at any moment all waves work inside one band of rows that
// sweeps down the matrix -- a compact DRAM footprint, which measured far
// faster than giving each wave a contiguous block of rows.  A wave keeps
// kPD of its rows in flight: before it converts row i it has already
// requested the next kPD-1, and right after converting row i it requests
// the one kPD steps ahead.  Lanes own E-element
// chunks, E = 8 for bf16/fp16 output (16 bytes) and E = 4 for fp32: chunk c
// of lane l covers columns strip*1024 + c*64*E + l*E, so every store
// instruction of the wave writes 1 KiB of contiguous output and every load
// instruction reads 64*E contiguous source bytes.  Source and destination
// are streamed with non-temporal accesses.  Parameters that vary along n
// are loaded once per wave (PER_CHANNEL) or once per group of rows
// (PER_GROUP with kDim = 0); a chunk never straddles a group because
// groupSize is a multiple of 32.  PER_TOKEN parameters are wave-uniform per
// row; PER_GROUP with kDim = 1 needs one parameter per chunk per row.
//
// Arithmetic (the page omits the formula; the library's reading):
//   dst = RN(RN(src + offset) * scale)   or   RN(src * scale)
// in binary32 (no contraction), then one round-to-nearest-even conversion
// to bf16 / fp16 (or none for fp32).

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

constexpr int kPD = 2;               // rows of loads in flight per wave
constexpr int64_t kTargetWaves = 16384;  // 256 CUs x 64 waves

enum AqPolicyKind : int { PK_TENSOR = 0, PK_CHANNEL = 1, PK_TOKEN = 2, PK_GROUP_N = 3, PK_GROUP_M = 4 };

struct AqArgs {
    const void* src;
    const float* scale;
    const float* offset;
    int64_t m, n;
    int64_t gs;        // group size (PER_GROUP)
    int64_t n_groups;  // ceil(n / gs) for kDim = 1
    void* dst;
    int64_t strips;         // ceil(n / 1024)
    int64_t row_step;       // G: waves per strip, the stride between a wave's rows
    int64_t waves;          // strips * G
    int64_t nblocks;
};

template <int DST>
struct Chunk {
    static constexpr int E = DST == DST_F32 ? 4 : 8;       // elements per chunk
    static constexpr int NCH = 1024 / (kWave * E);         // chunks per lane per row
    static constexpr int W = E / 4;                        // source dwords per chunk
};

// Four source bytes -> four floats (exact).
template <int SRC>
__device__ __forceinline__ void decode4(uint32_t w, float* v)
{
    if (SRC == SRC_I8) {
        v[0] = static_cast<float>(static_cast<int8_t>(w & 0xFFu));
        v[1] = static_cast<float>(static_cast<int8_t>((w >> 8) & 0xFFu));
        v[2] = static_cast<float>(static_cast<int8_t>((w >> 16) & 0xFFu));
        v[3] = static_cast<float>(static_cast<int8_t>(w >> 24));
    } else {
        // gfx950 converts OCP E4M3FN (NaN only at 0x7F / 0xFF, max 448).
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
        v[0] = lo[0];
        v[1] = lo[1];
        v[2] = hi[0];
        v[3] = hi[1];
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

// Store one chunk (16 bytes) of results.
template <int DST>
__device__ __forceinline__ void store_chunk(void* p, const float* t)
{
    if (DST == DST_F32) {
        st_stream16(p, make_uint4(__builtin_bit_cast(uint32_t, t[0]), __builtin_bit_cast(uint32_t, t[1]),
                                  __builtin_bit_cast(uint32_t, t[2]), __builtin_bit_cast(uint32_t, t[3])));
    } else if (DST == DST_BF16) {
        st_stream16(p, make_uint4(pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]),
                                  pack_bf16x2(t[4], t[5]), pack_bf16x2(t[6], t[7])));
    } else {
        st_stream16(p, make_uint4(pack_f16x2(t[0], t[1]), pack_f16x2(t[2], t[3]),
                                  pack_f16x2(t[4], t[5]), pack_f16x2(t[6], t[7])));
    }
}

template <int E>
__device__ __forceinline__ void load_params(const float* p, float* v)
{
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
        const float4 f = q[i];
        v[4 * i + 0] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}

template <int NCH, int W>
__device__ __forceinline__ void load_row(uint32_t (&raw)[NCH][W], const uint8_t* row, const int64_t (&jc)[NCH],
                                         const bool (&okc)[NCH])
{
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (okc[c]) {
            if (W == 2) {
                const uint2 w2 = ld_stream8(row + jc[c]);
                raw[c][0] = w2.x;
                raw[c][W - 1] = w2.y;
            } else {
                raw[c][0] = ld_stream4(row + jc[c]);
            }
        }
    }
}

template <int SRC, int DST, int PK, bool OFF>
__global__ __launch_bounds__(kBlock) void aq_kernel(AqArgs a)
{
    using C = Chunk<DST>;
    constexpr int E = C::E, NCH = C::NCH, W = C::W;
    constexpr bool kPerElem = PK == PK_CHANNEL || PK == PK_GROUP_M;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t wid = xcd_block(blockIdx.x, a.nblocks) * 4 + wave;
    if (wid >= a.waves)
        return;
    const int64_t strip = wid % a.strips;
    const int64_t G = a.row_step;
    const int64_t r0 = wid / a.strips;
    const int64_t r1 = a.m;
    if (r0 >= r1)
        return;
    int64_t jc[NCH];
    bool okc[NCH];
    int64_t gcol[NCH];  // PER_GROUP kDim = 1: the chunk's group
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        jc[c] = strip * 1024 + (c * kWave + lane) * E;
        okc[c] = jc[c] < a.n;  // n is a multiple of 16, so a chunk is whole or absent
        gcol[c] = PK == PK_GROUP_N ? jc[c] / a.gs : 0;
    }
    const uint8_t* src = static_cast<const uint8_t*>(a.src);
    uint8_t* dst = static_cast<uint8_t*>(a.dst);
    const int64_t out_elem = DST == DST_F32 ? 4 : 2;

    // Rows r0 .. r0 + kPD - 1 in flight before any arithmetic.
    uint32_t raw[kPD][NCH][W];
#pragma unroll
    for (int k = 0; k < kPD; ++k)
        if (r0 + k * G < r1)
            load_row<NCH, W>(raw[k], src + (r0 + k * G) * a.n, jc, okc);

    // Parameters fixed over many rows.
    float sv[NCH][E], ov[NCH][E];
    float s_u = 0.0f, o_u = 0.0f;
    int64_t g_lo = 0, g_hi = 0;  // PER_GROUP kDim = 0: rows of the group held in sv / ov
    auto load_vec_params = [&](int64_t row_base) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (okc[c]) {
                load_params<E>(a.scale + row_base + jc[c], sv[c]);
                if (OFF)
                    load_params<E>(a.offset + row_base + jc[c], ov[c]);
            }
        }
    };
    if (PK == PK_TENSOR) {
        s_u = a.scale[0];
        if (OFF)
            o_u = a.offset[0];
    } else if (PK == PK_CHANNEL) {
        load_vec_params(0);
    } else if (PK == PK_GROUP_M) {
        const int64_t g = r0 / a.gs;
        load_vec_params(g * a.n);
        g_lo = g * a.gs;
        g_hi = g_lo + a.gs;
    }

    for (int64_t r = r0; r < r1; r += kPD * G) {
#pragma unroll
        for (int k = 0; k < kPD; ++k) {
            const int64_t i = r + k * G;
            if (i >= r1)
                continue;
            if (PK == PK_GROUP_M && (i < g_lo || i >= g_hi)) {
                const int64_t g = i / a.gs;
                load_vec_params(g * a.n);
                g_lo = g * a.gs;
                g_hi = g_lo + a.gs;
            }
            float s1 = s_u, o1 = o_u;
            if (PK == PK_TOKEN) {
                s1 = a.scale[i];
                if (OFF)
                    o1 = a.offset[i];
            }
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (!okc[c])
                    continue;
                if (PK == PK_GROUP_N) {
                    const int64_t p = i * a.n_groups + gcol[c];
                    s1 = a.scale[p];
                    if (OFF)
                        o1 = a.offset[p];
                }
                float v[E];
#pragma unroll
                for (int w = 0; w < W; ++w)
                    decode4<SRC>(raw[k][c][w], v + 4 * w);
                float t[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float s = kPerElem ? sv[c][e] : s1;
                    if (OFF) {
                        const float o = kPerElem ? ov[c][e] : o1;
                        const float u = v[e] + o;
                        t[e] = u * s;
                    } else {
                        t[e] = v[e] * s;
                    }
                }
                store_chunk<DST>(dst + (i * a.n + jc[c]) * out_elem, t);
            }
            if (i + kPD * G < r1)
                load_row<NCH, W>(raw[k], src + (i + kPD * G) * a.n, jc, okc);
        }
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
    int64_t G = (kTargetWaves + a.strips - 1) / a.strips;  // waves per strip
    if (G > p.m)
        G = p.m;
    a.row_step = G;
    a.waves = a.strips * G;
    a.nblocks = (a.waves + 3) / 4;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(a.nblocks)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace dq
