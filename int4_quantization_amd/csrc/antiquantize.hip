// antiquantize.hip -- element-wise dequantization on gfx950
// (AntiQuantize, 功能说明: PER_TENSOR / PER_CHANNEL / PER_TOKEN / PER_GROUP,
// 表1 kDim, 表2 groupSize).
//
// A flat grid of short-lived threads: each converts one chunk of E
// consecutive elements of a row (E = 8 for bf16/fp16 output, 4 for fp32),
// so a lane reads 8 (or 4) source bytes and writes 16 output bytes, and
// every load and store instruction of a wave covers contiguous memory.
// That shape -- one narrow load and one 16-byte store per thread, many
// small workgroups -- measured fastest for this one-read, two-write
// traffic; every extra load or store a thread keeps in flight cost
// several percent.  Policies whose parameters vary along n (PER_CHANNEL,
// PER_GROUP with kDim = 0) instead give a thread R consecutive rows of one
// chunk, so the thread's parameter vectors are loaded once for R rows;
// PER_TOKEN and PER_GROUP with kDim = 1 load one parameter pair per chunk,
// PER_TENSOR one for the whole launch.  Sources: int8, fp8 E4M3FN and E5M2
// (the b8 cases of 表3), and fp4 E2M1 two codes per byte with e8m0 scales
// (the float4 case); parameters fp32, fp16, bf16 or e8m0, widened exactly.  Row and column come from one
// multiply-shift division by the chunks per row (exact for indices below
// 2^31; larger inputs are split over several launches).  Threads past the
// end repeat the last chunk, so every access is unconditional.  Source and
// destination are streamed with non-temporal accesses.
//
// Arithmetic (the page omits the formula; the library's reading):
//   dst = RN(RN(src + offset) * scale)   or   RN(src * scale)
// in binary32 (no contraction), then one round-to-nearest-even conversion
// to bf16 / fp16 (or none for fp32).

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

enum AqPolicyKind : int { PK_TENSOR = 0, PK_CHANNEL = 1, PK_TOKEN = 2, PK_GROUP_N = 3, PK_GROUP_M = 4 };

constexpr int kAqRowsPerThread = 8;  // PER_CHANNEL / PER_GROUP kDim = 0 (divides every groupSize)
constexpr int kAqGroupNUnits = 2;    // work units per thread with groups along n

// Work units per thread: two for groups along n (see aq_kernel), else one.
constexpr int aq_units_per_thread(int pk)
{
    return pk == PK_GROUP_N ? kAqGroupNUnits : 1;
}

struct AqArgs {
    const void* src;
    const void* scale;
    const void* offset;
    int64_t m, n;
    int64_t row0;       // first row of this launch
    int64_t rows;       // rows of this launch
    int64_t gs;         // group size (PER_GROUP)
    int64_t n_groups;   // ceil(n / gs) for kDim = 1
    void* dst;
    uint32_t cpr;       // chunks per row (n / E)
    uint32_t units;     // work units of this launch (threads that do work)
    DivMagic by_cpr;    // division by cpr
    DivMagic by_gsc;    // division by gs / E (chunks per group, kDim = 1)
    DivMagic by_gs;     // division by gs (rows per group, kDim = 0)
    uint32_t tiles_c;      // per channel in 2-D tiles: column tiles of kAqTileChunks chunks (0: flat order)
    DivMagic by_tiles_c;   // division by tiles_c
};

// Per channel with a row of whole column tiles: a workgroup takes
// kAqTileChunks chunks of kAqTileRowBlocks row blocks (64 x 4, 32 rows),
// wave w the tile's chunks 16 w .. 16 w + 15 in its 4 row blocks.  Each wave
// then loads the parameters of 16 chunks, not 64, and still reads whole
// 128-byte source lines and writes 256-byte output segments per row.
constexpr int kAqTileChunks = 64, kAqTileRowBlocks = 4;

template <int SRC, int DST>
struct Chunk {
    static constexpr int E = DST == DST_F32 ? 4 : 8;                 // elements per chunk
    static constexpr int SB = SRC == SRC_F4E2M1 ? E / 2 : E;         // source bytes per chunk
    static constexpr int W = SB / 4;                                 // source dwords per chunk
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
    } else if (SRC == SRC_F8E4M3) {
        // gfx950 converts OCP E4M3FN (NaN only at 0x7F / 0xFF, max 448).
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
        v[0] = lo[0];
        v[1] = lo[1];
        v[2] = hi[0];
        v[3] = hi[1];
    } else {
        // OCP E5M2 (bf8 in the ISA's naming).
        const auto lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
        v[0] = lo[0];
        v[1] = lo[1];
        v[2] = hi[0];
        v[3] = hi[1];
    }
}

// Eight fp4 E2M1 codes (one dword, element 2k in the low nibble of byte k)
// -> eight floats, exact: the hardware conversion with a scale of 1.
__device__ __forceinline__ void decode8_fp4(uint32_t w, float* v)
{
    const auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = b0[0];
    v[1] = b0[1];
    v[2] = b1[0];
    v[3] = b1[1];
    v[4] = b2[0];
    v[5] = b2[1];
    v[6] = b3[0];
    v[7] = b3[1];
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

// Parameters (scale, offset) widened exactly to fp32; the kind is a
// template argument, so the kernel has no branch around these loads.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b)
{
    // 2^(b - 127): the exponent field itself, 2^-127 as a subnormal, 0xFF NaN.
    const uint32_t bits = b == 0xFFu ? 0x7FC00000u : b == 0u ? 0x00400000u : b << 23;
    return __builtin_bit_cast(float, bits);
}

template <int P>
__device__ __forceinline__ float param1(const void* p, int64_t idx)
{
    if constexpr (P == PARAM_F32) {
        return static_cast<const float*>(p)[idx];
    } else if constexpr (P == PARAM_E8M0) {
        return e8m0_to_f32(static_cast<const uint8_t*>(p)[idx]);
    } else {
        const uint16_t h = static_cast<const uint16_t*>(p)[idx];
        return P == PARAM_F16 ? widen1<0>(h) : widen1<1>(h);
    }
}

// E consecutive parameters starting at idx (a multiple of E), one or two
// vector loads.
template <int E, int P>
__device__ __forceinline__ void param_vec(const void* p, int64_t idx, float* v)
{
    if constexpr (P == PARAM_F32) {
        const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            const float4 f = q[i];
            v[4 * i + 0] = f.x;
            v[4 * i + 1] = f.y;
            v[4 * i + 2] = f.z;
            v[4 * i + 3] = f.w;
        }
    } else if constexpr (P == PARAM_E8M0) {
        const uint8_t* q = static_cast<const uint8_t*>(p) + idx;
        uint32_t w[E / 4];
        if (E == 8) {
            const uint2 u = *reinterpret_cast<const uint2*>(q);
            w[0] = u.x;
            w[E / 4 - 1] = u.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(q);
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[e] = e8m0_to_f32((w[e / 4] >> (8 * (e % 4))) & 0xFFu);
    } else {
        const uint16_t* q = static_cast<const uint16_t*>(p) + idx;
        uint32_t w[E / 2];
        if (E == 8) {
            const uint4 u = *reinterpret_cast<const uint4*>(q);
            w[0] = u.x;
            w[1] = u.y;
            w[E / 2 - 2] = u.z;
            w[E / 2 - 1] = u.w;
        } else {
            const uint2 u = *reinterpret_cast<const uint2*>(q);
            w[0] = u.x;
            w[E / 2 - 1] = u.y;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint16_t h = static_cast<uint16_t>((w[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
            v[e] = P == PARAM_F16 ? widen1<0>(h) : widen1<1>(h);
        }
    }
}

// Wave-uniform fp32 parameters through the scalar memory path: the index
// (and so the address) is the same in every lane, so one scalar load serves
// the wave instead of a vector load per lane, which leaves the vector memory
// pipeline to the source and destination streams.  The address space cast
// makes the load a scalar one; it needs a 4-byte aligned pointer.
typedef const __attribute__((address_space(4))) uint32_t const_u32;

__device__ __forceinline__ float param1_scalar_f32(const void* p, int64_t idx)
{
    return __builtin_bit_cast(float, ((const_u32*)p)[idx]);
}

template <int W>
__device__ __forceinline__ void load_chunk(uint32_t (&raw)[W], const uint8_t* p)
{
    if (W == 2) {
        const uint2 w2 = ld_stream8(p);
        raw[0] = w2.x;
        raw[W - 1] = w2.y;
    } else {
        raw[0] = ld_stream4(p);
    }
}

template <int SRC, int DST, bool OFF>
__device__ __forceinline__ void convert_store(const uint32_t (&raw)[Chunk<SRC, DST>::W], const float* sv,
                                              const float* ov, void* out)
{
    constexpr int E = Chunk<SRC, DST>::E, W = Chunk<SRC, DST>::W;
    float v[E];
    if constexpr (SRC == SRC_F4E2M1) {
        decode8_fp4(raw[0], v);
    } else {
#pragma unroll
        for (int w = 0; w < W; ++w)
            decode4<SRC>(raw[w], v + 4 * w);
    }
    float t[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (OFF) {
            const float u = v[e] + ov[e];
            t[e] = u * sv[e];
        } else {
            t[e] = v[e] * sv[e];
        }
    }
    store_chunk<DST>(out, t);
}

// UNI: every wave lies inside one row (chunks per row a multiple of 64), so
// PER_TOKEN parameters are wave-uniform and are read with scalar loads
// (measured 2.3% faster on int8 [16384, 8192]).  PER_GROUP parameters are
// not: a wave's four groups of 128 are its own, so scalar loads of them all
// miss the scalar cache (measured 20% slower), and they stay vector loads.
template <int SRC, int DST, int PK, bool OFF, int P, bool UNI>
__global__ __launch_bounds__(kBlock) void aq_kernel(AqArgs a)
{
    using C = Chunk<SRC, DST>;
    constexpr int E = C::E, W = C::W, SB = C::SB;
    constexpr bool kPerElem = PK == PK_CHANNEL || PK == PK_GROUP_M;
    constexpr int R = kPerElem ? kAqRowsPerThread : 1;
    const int64_t out_elem = DST == DST_F32 ? 4 : 2;
    const uint8_t* src = static_cast<const uint8_t*>(a.src);
    uint8_t* dst = static_cast<uint8_t*>(a.dst);

    // Work unit u = (row block, chunk); a thread past the end repeats the
    // last unit (same bytes).  A thread takes CPT units kBlock apart, so a
    // workgroup covers kBlock * CPT consecutive units: with groups along n,
    // 4096 elements, whose parameters (32 groups of 128 at 4 bytes) fill
    // whole 128-byte lines that no other workgroup reads.
    constexpr int CPT = aq_units_per_thread(PK);
    const int64_t src_row = a.n / E * SB;  // source bytes per row
    uint32_t rb[CPT], jc[CPT];
    int64_t i0[CPT];
    uint32_t raw[CPT][R][W];
    // Source loads first, then the parameters: all are in flight together.
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        uint32_t u = blockIdx.x * (kBlock * CPT) + c * kBlock + threadIdx.x;
        if (PK == PK_CHANNEL && a.tiles_c) {  // uniform
            static_assert(kBlock == 4 * kWave && kAqTileChunks == 4 * 16 && kAqTileRowBlocks * 16 == kWave,
                          "four waves of 16 chunks x 4 row blocks");
            const uint32_t tr = div_by(blockIdx.x, a.by_tiles_c), tc = blockIdx.x - tr * a.tiles_c;
            const uint32_t wv = threadIdx.x / kWave, ln = threadIdx.x % kWave;
            u = (tr * kAqTileRowBlocks + ln / 16) * a.cpr + tc * kAqTileChunks + wv * 16 + ln % 16;
        }
        u = u < a.units ? u : a.units - 1;
        rb[c] = div_by(u, a.by_cpr);
        jc[c] = u - rb[c] * a.cpr;  // chunk within the row
        i0[c] = a.row0 + static_cast<int64_t>(rb[c]) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t i = i0[c] + r;
            i = i < a.row0 + a.rows ? i : a.row0 + a.rows - 1;  // past the end: repeat the last row
            load_chunk<W>(raw[c][r], src + i * src_row + static_cast<int64_t>(jc[c]) * SB);
        }
    }

    float sv[CPT][E], ov[CPT][E];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int64_t j = static_cast<int64_t>(jc[c]) * E;
        if constexpr (UNI && PK == PK_TOKEN) {
            const int64_t p = a.row0 + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(rb[c]));
            const float s1 = param1_scalar_f32(a.scale, p);
            const float o1 = OFF ? param1_scalar_f32(a.offset, p) : 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sv[c][e] = s1;
                ov[c][e] = o1;
            }
        } else if constexpr (PK == PK_TENSOR || PK == PK_TOKEN || PK == PK_GROUP_N) {
            int64_t p = 0;
            if (PK == PK_TOKEN)
                p = i0[c];
            if (PK == PK_GROUP_N)
                p = i0[c] * a.n_groups + div_by(jc[c], a.by_gsc);
            const float s1 = param1<P>(a.scale, p);
            const float o1 = OFF ? param1<P>(a.offset, p) : 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sv[c][e] = s1;
                ov[c][e] = o1;
            }
        } else {
            // The R rows share the group: R divides groupSize and the row
            // blocks start at multiples of R.
            const int64_t base =
                PK == PK_GROUP_M ? static_cast<int64_t>(div_by(static_cast<uint32_t>(i0[c]), a.by_gs)) * a.n : 0;
            param_vec<E, P>(a.scale, base + j, sv[c]);
            if (OFF)
                param_vec<E, P>(a.offset, base + j, ov[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int64_t j = static_cast<int64_t>(jc[c]) * E;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t i = i0[c] + r;
            i = i < a.row0 + a.rows ? i : a.row0 + a.rows - 1;
            convert_store<SRC, DST, OFF>(raw[c][r], sv[c], ov[c], dst + (i * a.n + j) * out_elem);
        }
    }
}

using KernelFn = void (*)(AqArgs);

template <int SRC, int DST, bool OFF, int P>
KernelFn pick_pk(int pk, bool uni)
{
    switch (pk) {
    case PK_TENSOR: return aq_kernel<SRC, DST, PK_TENSOR, OFF, P, false>;
    case PK_CHANNEL: return aq_kernel<SRC, DST, PK_CHANNEL, OFF, P, false>;
    case PK_TOKEN:
        if constexpr (P == PARAM_F32)
            if (uni)
                return aq_kernel<SRC, DST, PK_TOKEN, OFF, P, true>;
        return aq_kernel<SRC, DST, PK_TOKEN, OFF, P, false>;
    case PK_GROUP_N: return aq_kernel<SRC, DST, PK_GROUP_N, OFF, P, false>;
    case PK_GROUP_M: return aq_kernel<SRC, DST, PK_GROUP_M, OFF, P, false>;
    }
    return nullptr;
}

template <int SRC, int DST, int P>
KernelFn pick_off(int pk, bool off, bool uni)
{
    return off ? pick_pk<SRC, DST, true, P>(pk, uni) : pick_pk<SRC, DST, false, P>(pk, uni);
}

template <int SRC, int P>
KernelFn pick_dst(int dst, int pk, bool off, bool uni)
{
    switch (dst) {
    case DST_BF16: return pick_off<SRC, DST_BF16, P>(pk, off, uni);
    case DST_F16: return pick_off<SRC, DST_F16, P>(pk, off, uni);
    case DST_F32: return pick_off<SRC, DST_F32, P>(pk, off, uni);
    }
    return nullptr;
}

template <int SRC>
KernelFn pick_param(int param, int dst, int pk, bool off, bool uni)
{
    switch (param) {
    case PARAM_F32: return pick_dst<SRC, PARAM_F32>(dst, pk, off, uni);
    case PARAM_F16: return pick_dst<SRC, PARAM_F16>(dst, pk, off, uni);
    case PARAM_BF16: return pick_dst<SRC, PARAM_BF16>(dst, pk, off, uni);
    }
    return nullptr;
}

// The float4 case: PER_GROUP only, e8m0 scales, no offset, bf16 or fp16
// output.
KernelFn pick_fp4(int dst, int pk)
{
    const bool n_dir = pk == PK_GROUP_N;
    if (pk != PK_GROUP_N && pk != PK_GROUP_M)
        return nullptr;
    if (dst == DST_BF16)
        return n_dir ? aq_kernel<SRC_F4E2M1, DST_BF16, PK_GROUP_N, false, PARAM_E8M0, false>
                     : aq_kernel<SRC_F4E2M1, DST_BF16, PK_GROUP_M, false, PARAM_E8M0, false>;
    if (dst == DST_F16)
        return n_dir ? aq_kernel<SRC_F4E2M1, DST_F16, PK_GROUP_N, false, PARAM_E8M0, false>
                     : aq_kernel<SRC_F4E2M1, DST_F16, PK_GROUP_M, false, PARAM_E8M0, false>;
    return nullptr;
}

KernelFn pick_src(const AqPlan& p, int pk, bool uni)
{
    const bool off = p.offset != nullptr;
    switch (p.src_kind) {
    case SRC_I8: return pick_param<SRC_I8>(p.param_kind, p.dst_kind, pk, off, uni);
    case SRC_F8E4M3: return pick_param<SRC_F8E4M3>(p.param_kind, p.dst_kind, pk, off, uni);
    case SRC_F8E5M2: return pick_param<SRC_F8E5M2>(p.param_kind, p.dst_kind, pk, off, uni);
    case SRC_F4E2M1: return off || p.param_kind != PARAM_E8M0 ? nullptr : pick_fp4(p.dst_kind, pk);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_antiquantize(const AqPlan& p, hipStream_t stream)
{
    int pk = p.policy;  // DQ_PER_TENSOR .. DQ_PER_TOKEN map to the same numbers
    if (p.policy == DQ_PER_GROUP)
        pk = p.k_dim == 1 ? PK_GROUP_N : PK_GROUP_M;
    const int64_t E = p.dst_kind == DST_F32 ? 4 : 8;
    // Scalar PER_TOKEN parameter loads: fp32 parameters, 4-byte aligned,
    // and every wave inside one row.
    const bool rows_of_waves = p.n % (E * kWave) == 0;
    const bool f32_aligned = p.param_kind == PARAM_F32 &&
                             ((reinterpret_cast<uintptr_t>(p.scale) | reinterpret_cast<uintptr_t>(p.offset)) & 3) == 0;
    const bool uni = rows_of_waves && f32_aligned && pk == PK_TOKEN;
    KernelFn fn = pick_src(p, pk, uni);
    if (!fn)
        return hipErrorInvalidValue;
    const int64_t R = (pk == PK_CHANNEL || pk == PK_GROUP_M) ? kAqRowsPerThread : 1;
    AqArgs a{};
    a.src = p.src;
    a.scale = p.scale;
    a.offset = p.offset;
    a.m = p.m;
    a.n = p.n;
    a.gs = p.group_size > 0 ? p.group_size : 1;
    a.n_groups = (p.n + a.gs - 1) / a.gs;
    a.dst = p.dst;
    const int64_t cpr = p.n / E;  // n is a multiple of E (32-byte rows)
    if (cpr < 1 || cpr >= (int64_t{1} << 31))
        return hipErrorInvalidValue;
    a.cpr = static_cast<uint32_t>(cpr);
    a.by_cpr = div_magic(static_cast<uint64_t>(cpr));
    a.by_gsc = div_magic(static_cast<uint64_t>(a.gs >= E ? a.gs / E : 1));
    a.by_gs = div_magic(static_cast<uint64_t>(a.gs));
    // Row ranges of at most 2^31 - 1 work units, a multiple of R rows each
    // (so the PER_GROUP kDim = 0 row blocks stay aligned to R).
    const int64_t max_blocks_rows = ((int64_t{1} << 31) - 1) / cpr;  // row blocks per launch
    const int64_t max_rows = (max_blocks_rows > (int64_t{1} << 24) ? (int64_t{1} << 24) : max_blocks_rows) * R;
    for (int64_t row0 = 0; row0 < p.m; row0 += max_rows) {
        a.row0 = row0;
        a.rows = p.m - row0 < max_rows ? p.m - row0 : max_rows;
        const int64_t units = (a.rows + R - 1) / R * cpr;
        a.units = static_cast<uint32_t>(units);
        const int64_t per_block = kBlock * aq_units_per_thread(pk);
        int64_t blocks = (units + per_block - 1) / per_block;
        a.tiles_c = 0;
        if (pk == PK_CHANNEL && cpr % kAqTileChunks == 0) {
            const int64_t row_blocks = (a.rows + R - 1) / R;
            a.tiles_c = static_cast<uint32_t>(cpr / kAqTileChunks);
            a.by_tiles_c = div_magic(a.tiles_c);
            blocks = (row_blocks + kAqTileRowBlocks - 1) / kAqTileRowBlocks * a.tiles_c;
        }
        void* args[] = {&a};
        const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(fn),
                                               dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), args, 0, stream);
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace dq
