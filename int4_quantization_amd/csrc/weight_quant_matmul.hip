// weight_quant_matmul.hip -- x1 @ dequant(x2) + bias + x3 on gfx950: int8 or
// int4 weights fake-quantized per tensor, per channel or per group down k,
// then multiplied on the matrix cores.
//
// aclnnWeightQuantMatmulAllReduce (API function, constraints) fake-quantizes
// the weight x2, multiplies, and all-reduces over ranks; on one GPU the
// all-reduce is the identity.  Its formula is missing from the page; this
// library reads it with the AntiQuantize arithmetic (kDim = 0):
//   W[k, n]   = RN_T(RN(RN(x2 + offset) * scale))    (binary32; no offset: RN(x2 * scale))
//   out[m, n] = RN_T(sum_k x1[m, k] * W[k, n] + bias[n] + x3[m, n])
// where T is x1's dtype (the constraints give the parameters, bias, x3 and
// the output that dtype) and the sum is accumulated in binary32.  Products
// of two bf16 or two fp16 values are exact in binary32, so W is bit-exact
// and only the order of the binary32 additions differs from an exact sum.
//
// Matrix-core kernels (weights stored [n, k], i.e. x2 transposed, k
// contiguous):
//   - v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies row (or column) l % 16
//     and eight k values per instruction, and receives rows 4 (l / 16) ..
//     + 3 of column l % 16.
//   - Dequantization follows the formula step by step in binary32 (signed
//     byte or nibble -> binary32, + offset, * scale, round to T), so W is
//     exact.  A run of 32 k never straddles a parameter group (the group
//     size is a multiple of 32).
//   - Rows past m repeat the last row (their results are not stored);
//     columns past n repeat the last column (likewise).  k runs in whole
//     groups of 32 (int8) or 64 (int4) elements.
//   - wq_decode_kernel (at most 16 rows) walks k in supersteps of 128.
//     Since a dot product does not depend on the order of k, lane group
//     g = l / 16 takes the 32 consecutive k of [32 g, 32 g + 32) and splits
//     them over the superstep's four instructions, and x1 uses the same
//     assignment: each lane's weight load is one contiguous 32-byte (int8)
//     or 16-byte (int4) run of its column, and the dequantized weights go
//     from registers straight into the matrix cores.
//   - wq_gemm_kernel (more rows) stages 128 x 128 tiles in LDS.
//   Both are described further where they are defined.
// wq_generic_kernel: any layout and alignment, one thread per output
// element, binary32 accumulation in k order.  It is the path for weights
// stored [k, n].

#include "dq_device.h"
#include "dq_ext_internal.h"

namespace dq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWqSuper = kWqSuperK;  // k per superstep: 4 lane groups x 32

// Buffer loads: a 128-bit resource (base, size in bytes) and a 32-bit
// per-lane offset, so address arithmetic stays 32-bit and constant steps
// fold into the instruction's offset field.  Reads past the size return 0.
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufNonTemporal = 2;  // glc/slc/nt bits of the aux operand: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
template <int AUX>
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    return make_uint4(static_cast<uint32_t>(v.x), static_cast<uint32_t>(v.y), static_cast<uint32_t>(v.z),
                      static_cast<uint32_t>(v.w));
}
__device__ __forceinline__ uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

struct WqArgs {
    const uint16_t* x1;    // [m, k] T
    const uint8_t* x2;     // int8 [n, k] or int4 [n, k / 2] (fast); [k, n] or [k, n / 2] (generic)
    const uint16_t* scale;
    const uint16_t* offset;  // nullptr: none
    const uint16_t* bias;    // nullptr: none
    const uint16_t* x3;      // nullptr: none
    uint16_t* out;           // [m, n] T
    int64_t m, k, n;
    int64_t group_size;      // per group only
    int64_t groups;          // ceil(k / group_size), per group only
    int64_t k_chunk;         // k per split (a multiple of the batch)
    float* partial;          // splits > 1: binary32 partial sums [splits, m, n]
    DivMagic by_gs;          // division by group_size (k indices below 2^31)
};

template <int XT>
__device__ __forceinline__ float t_to_f32(uint16_t h) { return widen1<XT>(h); }

// Round a binary32 to T (nearest even), as raw bits.  The empty asm keeps
// the binary32 value: without it hipcc folds "binary32 multiply or add, then
// convert to fp16" into v_fma_mix*, which rounds only once.
template <int XT>
__device__ __forceinline__ uint16_t f32_to_t(float v)
{
    asm("" : "+v"(v));
    if constexpr (XT == X_BF16) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    } else {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
    }
}

// Parameter index of weight column c for the group holding k index kk.
template <int POL>
__device__ __forceinline__ int64_t param_index(const WqArgs& a, int64_t c, int64_t kk, bool trans)
{
    if constexpr (POL == DQ_PER_TENSOR)
        return 0;
    else if constexpr (POL == DQ_PER_CHANNEL)
        return c;
    else
        return trans ? c * a.groups + kk / a.group_size : (kk / a.group_size) * a.n + c;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two binary32 values rounded to T (nearest even) in one packed conversion
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).  For fp16 the empty asm keeps the
// binary32 inputs: otherwise hipcc may fold "binary32 multiply, then
// convert to fp16" into v_fma_mix*, which rounds only once.
template <int XT>
__device__ __forceinline__ uint32_t pack2_t(float a, float b)
{
    const f32x2 v = {a, b};
    if constexpr (XT == X_BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    } else {
        asm("" : "+v"(a), "+v"(b));
        const f32x2 w = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(w, f16x2));
    }
}

// Eight binary32 values rounded to T and packed as one MFMA operand.
template <int XT>
__device__ __forceinline__ uint4 pack8_t(const float (&w)[8])
{
    return make_uint4(pack2_t<XT>(w[0], w[1]), pack2_t<XT>(w[2], w[3]), pack2_t<XT>(w[4], w[5]),
                      pack2_t<XT>(w[6], w[7]));
}

template <int XT>
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, const f32x4& c)
{
    if constexpr (XT == X_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

// The integer codes of a lane's 32 consecutive k of one column, as
// binary32, each converted from a sign-extended byte in one instruction
// (v_cvt_f32_i32 with an SDWA byte select).  int8: the codes themselves.
// int4: each nibble is first moved to the high half of a byte, so the byte
// reads 16 * code; the caller folds the factor 16 back exactly.
// Eight of a lane's 32 codes (sub-step s of its run) as binary32: the code,
// or 16 * code for int4 (the nibble moved to the high half of a byte).
template <int WT>
__device__ __forceinline__ void decode8(const uint4& lo, const uint4& hi, int s, float (&v)[8])
{
    if constexpr (WT == WQ_I8) {
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = static_cast<float>(static_cast<int8_t>(w[2 * s + i / 4] >> (8 * (i % 4))));
    } else {
        const uint32_t w[4] = {lo.x, lo.y, lo.z, lo.w};
        const uint32_t even = (w[s] << 4) & 0xF0F0F0F0u, odd = w[s] & 0xF0F0F0F0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = static_cast<float>(static_cast<int8_t>(even >> (8 * j)));
            v[2 * j + 1] = static_cast<float>(static_cast<int8_t>(odd >> (8 * j)));
        }
    }
}

// One weight, from the decoded value d (the code, or 16 * code for int4):
//   offset: RN(RN(code + o) * s)        no offset: RN(code * s)
// For int4 without offset the scale arrives as s / 16, an exact power-of-two
// scaling of a bf16 / fp16 value (binary32 keeps its bits down to 2^-149),
// so d * (s / 16) is the same real product.  With offset the code is
// recovered exactly as d / 16 first.
template <int WT, bool OFF>
__device__ __forceinline__ float dequant1(float d, float s, float o)
{
    if constexpr (OFF) {
        const float code = WT == WQ_I4 ? d * 0.0625f : d;
        const float u = code + o;
        return u * s;
    } else {
        return d * s;
    }
}

// ---------------------------------------------------------------------------
// Decode-shaped kernel: at most 16 rows of x1, so the weights dominate the
// traffic.  A wave owns 16 RN columns; a workgroup (four waves) stages the
// x1 k-slice of each batch (U supersteps) in LDS once for its four waves,
// double-buffered, and each wave keeps the next batch's weight and
// parameter loads in flight while it dequantizes and multiplies the
// current one.  k is split across workgroups (blockIdx.z) as planned on the
// host.
// ---------------------------------------------------------------------------
// PAIR: per-group parameters with groups of 128 (one per superstep) and an
// even group count, so the two groups of a batch are adjacent in a column's
// parameter row and one 4-byte load fetches both (the loads of the per-group
// parameters cost as much time as the weight stream when made one by one).
template <int XT, int WT, int POL, bool OFF, int RN, int U, bool PAIR>
__global__ __launch_bounds__(kWqDecodeWaves * kWave) void wq_decode_kernel(const WqArgs a)
{
    static_assert(!PAIR || (POL == DQ_PER_GROUP && U == 2), "paired parameters: two supersteps of 128 per batch");
    constexpr int NT = kWqDecodeWaves * kWave;
    constexpr int BK = U * kWqSuper;       // k per batch
    constexpr int ROWB = BK * 2 + 32;      // LDS bytes per staged x1 row (a 32-byte pad, see below)
    constexpr int XV = BK / 8;             // 16-byte x1 vectors per row and batch
    constexpr int XP = 16 * XV / NT;       // staged vectors per thread and batch
    static_assert(XP * NT == 16 * XV, "a batch of 16 rows divides over the workgroup");
    // The operand read of superstep u and sub-step s2 takes, in lane group g,
    // the 8 k of chunk 16 u + 4 g + s2.  The chunks are stored in slot
    // 16 u + 4 s2 + g (the two 2-bit fields swapped), so the 4 lane groups
    // read 4 adjacent 16-byte slots of 16 rows: at a row stride of 8 modulo
    // 16 dwords that is free of bank conflicts on gfx950.  Slot and chunk
    // map to each other by the same swap.
    auto swap_chunk = [](int c) { return (c & ~15) | ((c & 3) << 2) | ((c >> 2) & 3); };
    constexpr int64_t kBytes32 = WT == WQ_I8 ? 32 : 16;  // weight bytes of 32 k
    constexpr int WV = WT == WQ_I8 ? 2 : 1;              // 16-byte weight loads per 32 k
    __shared__ __align__(16) uint8_t xs[2][16 * ROWB];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int li = lane % 16, g = lane / 16;
    const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * kWqDecodeWaves + wave) * (16 * RN);
    const int64_t k_beg = static_cast<int64_t>(blockIdx.z) * a.k_chunk;
    const int64_t k_end = k_beg + a.k_chunk < a.k ? k_beg + a.k_chunk : a.k;
    const int nb = static_cast<int>((k_end - k_beg + BK - 1) / BK);

    // Weight rows of at most 65535 x 65535 codes fit 32-bit byte offsets.
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(a.x2, static_cast<uint32_t>(a.n * (a.k / 32) * kBytes32));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x1, static_cast<uint32_t>(a.m * a.k * 2));
    uint32_t wcol[RN];  // byte offset of this lane's column and lane group
    int64_t col[RN];
#pragma unroll
    for (int t = 0; t < RN; ++t) {
        const int64_t c = n0 + 16 * t + li;
        col[t] = c < a.n ? c : a.n - 1;
        wcol[t] = static_cast<uint32_t>(col[t] * (a.k / 32) * kBytes32);
    }
    float s_chan[RN], o_chan[RN];
#pragma unroll
    for (int t = 0; t < RN; ++t) {
        s_chan[t] = 0.0f;
        o_chan[t] = 0.0f;
    }
    if constexpr (POL != DQ_PER_GROUP) {
#pragma unroll
        for (int t = 0; t < RN; ++t) {
            const int64_t p = param_index<POL>(a, col[t], 0, true);
            s_chan[t] = t_to_f32<XT>(a.scale[p]);
            o_chan[t] = OFF ? t_to_f32<XT>(a.offset[p]) : 0.0f;
        }
    }
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.scale, static_cast<uint32_t>(a.n * a.groups * 2));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(OFF ? a.offset : a.scale, static_cast<uint32_t>(a.n * a.groups * 2));

    // Loads of batch b (clamped to the last batch: a repeat is harmless).
    // x1: slot q = p * NT + tid of the 16 x XV grid, holding chunk
    // swap_chunk(slot); rows past m and k past the split are zeros.
    auto load_x = [&](int b, uint4 (&xr)[XP]) {
        const int bb = b < nb ? b : nb - 1;
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int q = p * NT + tid, row = q / XV, kv = swap_chunk(q % XV);
            const uint32_t kk = static_cast<uint32_t>(k_beg + static_cast<int64_t>(bb) * BK) + kv * 8;
            const bool ok = row < a.m && kk < k_end;
            const uint32_t rr = static_cast<uint32_t>(row < a.m ? row : a.m - 1);
            const uint32_t kc = ok ? kk : static_cast<uint32_t>(k_beg);
            const uint4 v = buf_load16<0>(xrs, (rr * static_cast<uint32_t>(a.k) + kc) * 2);
            xr[p] = ok ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf, const uint4 (&xr)[XP]) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int q = p * NT + tid, row = q / XV;
            *reinterpret_cast<uint4*>(&xs[buf][row * ROWB + (q % XV) * 16]) = xr[p];
        }
    };
    // Weights (and per-group parameters) of batch b for this lane: 32 k per
    // superstep, at k = batch start + 128 u + 32 g.
    auto load_w = [&](int b, uint4 (&w)[U][RN][WV], float (&sg)[U][RN], float (&og)[U][RN]) {
        const int bb = b < nb ? b : nb - 1;
        const uint32_t kb = static_cast<uint32_t>(k_beg + static_cast<int64_t>(bb) * BK);
        if constexpr (PAIR) {
#pragma unroll
            for (int t = 0; t < RN; ++t) {
                const uint32_t pi = static_cast<uint32_t>(col[t] * a.groups) + kb / kWqSuper;  // even
                const uint32_t sv = __builtin_amdgcn_raw_buffer_load_b32(srs, pi * 2, 0, 0);
                sg[0][t] = t_to_f32<XT>(static_cast<uint16_t>(sv));
                sg[1][t] = t_to_f32<XT>(static_cast<uint16_t>(sv >> 16));
                if constexpr (OFF) {
                    const uint32_t ov = __builtin_amdgcn_raw_buffer_load_b32(ors, pi * 2, 0, 0);
                    og[0][t] = t_to_f32<XT>(static_cast<uint16_t>(ov));
                    og[1][t] = t_to_f32<XT>(static_cast<uint16_t>(ov >> 16));
                } else {
                    og[0][t] = og[1][t] = 0.0f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t kg = kb + u * kWqSuper + 32 * g;
            const uint32_t kc = kg < k_end ? kg : static_cast<uint32_t>(k_beg);
#pragma unroll
            for (int t = 0; t < RN; ++t) {
                const uint32_t off = wcol[t] + (kc / 32) * static_cast<uint32_t>(kBytes32);
                w[u][t][0] = buf_load16<kBufNonTemporal>(wrs, off);
                if constexpr (WV == 2)
                    w[u][t][WV - 1] = buf_load16<kBufNonTemporal>(wrs, off + 16);
                if constexpr (POL == DQ_PER_GROUP && !PAIR) {
                    const uint32_t pi = static_cast<uint32_t>(col[t] * a.groups) + div_by(kc, a.by_gs);
                    sg[u][t] = t_to_f32<XT>(buf_load2(srs, pi * 2));
                    og[u][t] = OFF ? t_to_f32<XT>(buf_load2(ors, pi * 2)) : 0.0f;
                }
            }
        }
    };

    f32x4 acc[RN];
#pragma unroll
    for (int t = 0; t < RN; ++t)
        acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int buf, const uint4 (&w)[U][RN][WV], const float (&sg)[U][RN], const float (&og)[U][RN]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint4 av[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                av[s2] = *reinterpret_cast<const uint4*>(&xs[buf][li * ROWB + (16 * u + 4 * s2 + g) * 16]);
#pragma unroll
            for (int t = 0; t < RN; ++t) {
                float sc = s_chan[t], of = o_chan[t];
                if constexpr (POL == DQ_PER_GROUP) {
                    sc = sg[u][t];
                    of = og[u][t];
                }
                uint4 bv[4];
                if constexpr (WT == WQ_I4 && OFF) {
                    // v = 16 code: RN(v + 16 o) = 16 RN(code + o) and s / 16 is
                    // exact, so RN(RN(v + 16 o) * (s / 16)) is the formula,
                    // unless 16 o overflows (|o| near the binary32 limit).
                    // The test is made wave-uniform: a per-lane condition
                    // would be if-converted, computing every weight both ways.
                    const float o16 = of * 16.0f, s16 = sc * 0.0625f;
                    const bool huge = __any(__builtin_isinf(o16));
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        float v[8], wv[8];
                        decode8<WT>(w[u][t][0], w[u][t][WV - 1], s2, v);
                        if (__builtin_expect(huge, 0)) {
#pragma unroll 1
                            for (int j = 0; j < 8; ++j)
                                wv[j] = dequant1<WT, true>(v[j], sc, of);
                        } else {
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                wv[j] = (v[j] + o16) * s16;
                        }
                        bv[s2] = pack8_t<XT>(wv);
                    }
                } else {
                    const float sc_eff = WT == WQ_I4 ? sc * 0.0625f : sc;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        float v[8], wv[8];
                        decode8<WT>(w[u][t][0], w[u][t][WV - 1], s2, v);
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            wv[j] = dequant1<WQ_I8, OFF>(v[j], sc_eff, of);
                        bv[s2] = pack8_t<XT>(wv);
                    }
                }
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    acc[t] = mfma16<XT>(av[s2], bv[s2], acc[t]);
            }
        }
    };

    // Two register sets and two LDS buffers alternate: batch b + 1 is loaded
    // while batch b is computed.  nb is uniform (no batch when k is empty).
    if (nb > 0) {
        uint4 wA[U][RN][WV], wB[U][RN][WV];
        float sA[U][RN], oA[U][RN], sB[U][RN], oB[U][RN];
        uint4 xr[XP];
        load_x(0, xr);
        load_w(0, wA, sA, oA);
        store_x(0, xr);
        __syncthreads();
        for (int b = 0; b < nb; b += 2) {
            load_x(b + 1, xr);
            load_w(b + 1, wB, sB, oB);
            compute(0, wA, sA, oA);
            store_x(1, xr);
            __syncthreads();
            if (b + 1 >= nb)
                break;
            load_x(b + 2, xr);
            load_w(b + 2, wA, sA, oA);
            compute(1, wB, sB, oB);
            store_x(0, xr);
            __syncthreads();
        }
    }

    // Epilogue: lane holds rows 4 g .. 4 g + 3 of column li.
#pragma unroll
    for (int t = 0; t < RN; ++t) {
        const int64_t c = n0 + 16 * t + li;
        if (c >= a.n)
            continue;
        const float bias = a.bias && !a.partial ? t_to_f32<XT>(a.bias[c]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = 4 * g + i;
            if (row >= a.m)
                continue;
            if (a.partial) {
                a.partial[(static_cast<int64_t>(blockIdx.z) * a.m + row) * a.n + c] = acc[t][i];
            } else {
                float v = acc[t][i] + bias;
                if (a.x3)
                    v += t_to_f32<XT>(a.x3[row * a.n + c]);
                a.out[row * a.n + c] = f32_to_t<XT>(v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Prefill-shaped kernel: a 128 x 128 output tile per workgroup, four waves
// in a 2 x 2 grid, each 64 x 64 (4 x 4 blocks of 16 x 16).  Per k-step of
// 128 the x1 tile and the dequantized weight tile are staged in LDS, so every
// weight is dequantized once per 128 rows and every x1 element read once
// per 128 columns; the next step's global loads are in flight during the
// current step's matrix-core work.  (Measured: 256-row tiles lose more to
// occupancy than they save in dequantization; k-steps of 128 beat 64; eight
// waves split into four that dequantize the next step and four that run the
// matrix cores were no faster, as the second LDS buffer halves occupancy.)
//
// LDS layout of the prefill tiles.  Rows (x1 rows, weight columns) are
// padded by 32 bytes: on gfx950 the 16-byte operand reads of 16 rows by
// 4 lane groups are free of bank conflicts at that stride and not at a
// 16-byte pad.  16-byte stores are serviced 8 lanes at a time over 32
// banks, so in every 8-lane store each of the 4 weight columns it touches
// must receive two chunks whose slots differ in bit 0: the lanes of a
// column are assigned in pairs (wq_bmap), and the 8-element k-chunks of a
// row are stored in a permuted order (wq_phys_chunk).  x1 rows take the same
// permutation, so the matrix cores still pair equal k; a dot product's
// k order is free.
constexpr int kLdsPad = 16;  // elements

// Physical slot of logical k-chunk c in a BK-wide row.
template <int WT, int BK>
__device__ __forceinline__ constexpr int wq_phys_chunk(int c)
{
    constexpr int CPL = WT == WQ_I8 ? 2 : 4;  // chunks per 16-byte weight vector
    constexpr int LPC = BK / 8 / CPL;         // weight vectors per column row
    return (c % CPL) * LPC + c / CPL;
}

// Logical k-chunk held by physical slot p (the inverse of wq_phys_chunk);
// x1 lanes walk the slots in order, so 8 lanes fill 8 consecutive slots.
template <int WT, int BK>
__device__ __forceinline__ constexpr int wq_logical_chunk(int p)
{
    constexpr int CPL = WT == WQ_I8 ? 2 : 4;
    constexpr int LPC = BK / 8 / CPL;
    return (p % LPC) * CPL + p / LPC;
}

// Weight vector q of a tile -> column cl and vector kv within the column.
template <int WT, int BK>
__device__ __forceinline__ void wq_bmap(int q, int& cl, int& kv)
{
    constexpr int LPC = BK / (WT == WQ_I8 ? 16 : 32);
    static_assert(LPC >= 2 && LPC % 2 == 0, "two vectors per column and pass");
    const int a = q / 8, b = q % 8;
    cl = 4 * (a / (LPC / 2)) + b / 2;
    kv = 2 * (a % (LPC / 2)) + b % 2;
}

constexpr int kGemmBM = kWqGemmRows, kGemmBN = kWqGemmCols, kGemmBK = kWqGemmK;
static_assert(kWqSuperK % kGemmBK == 0, "k splits fall on k-step boundaries");
constexpr int kGemmThreads = kGemmBM / 64 * 2 * kWave;  // waves in a (BM / 64) x 2 grid

// PW (per-group parameters, groups of one k-step, kWqParamWindow-group
// aligned splits): once per kWqParamWindow steps, half of the threads load
// a window of consecutive scales of one column with one 16-byte load and the
// other half the offsets, into an LDS table; otherwise every weight vector
// loads its own 2-byte parameters each step, each such load touching one
// cache line per column (15-18% of the kernel on int4 g128 shapes).
template <int XT, int WT, int POL, bool OFF, bool PW>
__global__ __launch_bounds__(kGemmThreads) void wq_gemm_kernel(const WqArgs a)
{
    constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK, LR = kGemmBK + kLdsPad, NT = kGemmThreads;
    constexpr int AV = BM * (BK / 8) / NT;                         // 16-byte x1 vectors per thread
    constexpr int KPV = WT == WQ_I8 ? 16 : 32;                      // k per 16-byte weight vector
    constexpr int BQ = BN * (BK / KPV);                             // weight vectors per tile
    constexpr int BV = BQ >= NT ? BQ / NT : 1;                      // ... per thread (waves past BQ idle)
    static_assert(AV * NT == BM * BK / 8 && (BQ >= NT ? BV * NT == BQ : NT % BQ == 0 && BQ % kWave == 0),
                  "tile divides over threads");
    constexpr int WN = BN / 2, TN = WN / 16, ER = WN + 8;         // wave columns, their 16-blocks, epilogue row
    static_assert(BN % 32 == 0 && BM == 128, "2 x 2 waves of 64 rows x BN / 2 columns");
    constexpr int kStage = (BM + BN) * LR, kEpi = NT / kWave * 64 * ER;
    __shared__ __align__(16) uint16_t smem[kStage > kEpi ? kStage : kEpi];
    uint16_t* const As = smem;            // [BM][LR]: x1 rows
    uint16_t* const Bs = smem + BM * LR;  // [BN][LR]: dequantized weight columns
    constexpr int GW = kWqParamWindow;
    static_assert(!PW || (POL == DQ_PER_GROUP && NT >= 2 * BN), "a parameter window per column and tensor");
    __shared__ __align__(16) uint16_t pws[PW && OFF ? 2 : 1][PW ? BN : 1][PW ? GW : 1];  // [tensor][column][group]

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int li = lane % 16, g = lane / 16;
    const int wm = wave / 2, wn = wave % 2;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
    const int64_t k_beg = static_cast<int64_t>(blockIdx.z) * a.k_chunk;
    const int64_t k_end = k_beg + a.k_chunk < a.k ? k_beg + a.k_chunk : a.k;
    const int nk = static_cast<int>((k_end - k_beg + BK - 1) / BK);
    constexpr int64_t kBytes32 = WT == WQ_I8 ? 32 : 16;

    // Global loads of step kt into registers: x1 vectors (zeros past k_end)
    // and weight vectors (clamped in k: their x1 partner is zero).
    auto load = [&](int kt, uint4 (&ar)[AV], uint4 (&br)[BV], float (&bs)[BV], float (&bo)[BV]) {
        const int64_t kb = k_beg + static_cast<int64_t>(kt) * BK;
#pragma unroll
        for (int p = 0; p < AV; ++p) {
            const int q = p * NT + tid, row = q / (BK / 8), kv = wq_logical_chunk<WT, BK>(q % (BK / 8));
            const int64_t r = m0 + row < a.m ? m0 + row : a.m - 1;
            const int64_t kk = kb + kv * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(a.x1 + r * a.k + (kk < k_end ? kk : k_beg));
            ar[p] = kk < k_end ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < BV; ++p) {
            const int q = p * NT + tid;
            int cl, kv;
            wq_bmap<WT, BK>(q % BQ, cl, kv);
            const int64_t c = n0 + cl < a.n ? n0 + cl : a.n - 1;
            int64_t kk = kb + static_cast<int64_t>(kv) * KPV;
            kk = kk < k_end ? kk : k_beg;
            // Cached, unlike the decode kernel that reads each weight once:
            // every 128-row tile re-reads these (the non-temporal hint cost
            // 14% on 4096 x 8192 x 8192).
            const u32x4 v = *reinterpret_cast<const u32x4*>(a.x2 + c * (a.k / 32) * kBytes32 + kk * kBytes32 / 32);
            br[p] = make_uint4(v.x, v.y, v.z, v.w);
            if constexpr (POL == DQ_PER_GROUP && !PW) {
                const int64_t pi = c * a.groups + div_by(static_cast<uint32_t>(kk), a.by_gs);
                bs[p] = t_to_f32<XT>(a.scale[pi]);
                bo[p] = OFF ? t_to_f32<XT>(a.offset[pi]) : 0.0f;
            } else if constexpr (POL != DQ_PER_GROUP) {
                // Reloaded each step (cached): keeping them in registers
                // across the loop measured 7% slower.
                const int64_t pi = POL == DQ_PER_TENSOR ? 0 : c;
                bs[p] = t_to_f32<XT>(a.scale[pi]);
                bo[p] = OFF ? t_to_f32<XT>(a.offset[pi]) : 0.0f;
            }
        }
    };
    // The parameter window of steps kt .. kt + GW - 1 (kt a multiple of GW):
    // thread j < BN takes column j's scales, BN + j its offsets.
    uint4 pwr = make_uint4(0, 0, 0, 0);
    auto load_pw = [&](int kt) {
        if (PW && tid < (OFF ? 2 : 1) * BN) {
            const int j = tid % BN;
            const int64_t c = n0 + j < a.n ? n0 + j : a.n - 1;
            const int64_t g0 = k_beg / BK + kt;  // groups are one step long
            const uint16_t* src = (tid < BN ? a.scale : a.offset) + c * a.groups + g0;
            const u32x4 v = *reinterpret_cast<const u32x4*>(src);
            pwr = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto store_pw = [&]() {
        if (PW && tid < (OFF ? 2 : 1) * BN)
            *reinterpret_cast<uint4*>(&pws[tid / BN][tid % BN][0]) = pwr;
    };
    // Registers -> LDS: x1 as is; weights dequantized (exact binary32 steps,
    // one rounding to T) into the [column][k] layout the operands read.
    auto store = [&](int kt, const uint4 (&ar)[AV], const uint4 (&br)[BV], const float (&bs)[BV],
                     const float (&bo)[BV]) {
#pragma unroll
        for (int p = 0; p < AV; ++p) {
            const int q = p * NT + tid, row = q / (BK / 8);
            *reinterpret_cast<uint4*>(&As[row * LR + 8 * (q % (BK / 8))]) = ar[p];
        }
#pragma unroll
        for (int p = 0; p < BV; ++p) {
            const int q = p * NT + tid;
            if (q >= BQ)  // uniform per wave
                break;
            int cl, kv;
            wq_bmap<WT, BK>(q, cl, kv);
            float s0 = bs[p], of = bo[p];
            if constexpr (PW) {
                s0 = t_to_f32<XT>(pws[0][cl][kt % GW]);
                of = OFF ? t_to_f32<XT>(pws[OFF ? 1 : 0][cl][kt % GW]) : 0.0f;
            }
            const float sc = WT == WQ_I4 && !OFF ? s0 * 0.0625f : s0;
#pragma unroll
            for (int s2 = 0; s2 < KPV / 8; ++s2) {
                float v[8], w[8];
                decode8<WT>(br[p], br[p], s2, v);  // the vector's codes 8 s2 .. 8 s2 + 7
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if constexpr (WT == WQ_I4 && OFF)
                        w[j] = dequant1<WT, true>(v[j], sc, of);
                    else
                        w[j] = dequant1<WQ_I8, OFF>(v[j], sc, of);
                }
                *reinterpret_cast<uint4*>(&Bs[cl * LR + 8 * wq_phys_chunk<WT, BK>(kv * (KPV / 8) + s2)]) = pack8_t<XT>(w);
            }
        }
    };

    f32x4 acc[4][TN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < TN; ++t)
            acc[r][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if (nk > 0) {
        uint4 ar[AV], br[BV];
        float bs[BV], bo[BV];
        load(0, ar, br, bs, bo);
        load_pw(0);
        for (int kt = 0; kt < nk; ++kt) {
            __syncthreads();  // the previous step's operand reads are done
            if (PW && kt % GW == 0) {  // a new parameter window (uniform)
                store_pw();
                __syncthreads();
            }
            store(kt, ar, br, bs, bo);
            __syncthreads();
            load(kt + 1 < nk ? kt + 1 : kt, ar, br, bs, bo);  // in flight during the matrix-core work
            if (PW && (kt + 1) % GW == 0 && kt + 1 < nk)
                load_pw(kt + 1);
#pragma unroll
            for (int s2 = 0; s2 < BK / 32; ++s2) {
                uint4 av[4], bv[TN];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    av[r] = *reinterpret_cast<const uint4*>(&As[(wm * 64 + 16 * r + li) * LR + 32 * s2 + 8 * g]);
#pragma unroll
                for (int t = 0; t < TN; ++t)
                    bv[t] = *reinterpret_cast<const uint4*>(&Bs[(wn * WN + 16 * t + li) * LR + 32 * s2 + 8 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < TN; ++t)
                        acc[r][t] = mfma16<XT>(av[r], bv[t], acc[r][t]);
            }
        }
    }

    if (a.partial) {  // split k: binary32 partial sums, finished by wq_reduce_kernel
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int64_t c = n0 + wn * WN + 16 * t + li;
            if (c >= a.n)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t row = m0 + wm * 64 + 16 * r + 4 * g + i;
                    if (row < a.m)
                        a.partial[(static_cast<int64_t>(blockIdx.z) * a.m + row) * a.n + c] = acc[r][t][i];
                }
        }
        return;
    }

    // Epilogue through LDS: each wave writes its 64 x WN sums (+ bias) as T
    // into a row-major tile of 64 rows of WN + 8 in the staging memory, then
    // stores whole 16-byte row pieces (+ x3).
    __syncthreads();
    uint16_t* tile = smem + wave * (64 * ER);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int64_t c = n0 + wn * WN + 16 * t + li;
        const float b = a.bias && c < a.n ? t_to_f32<XT>(a.bias[c]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * r + 4 * g + i, cc = 16 * t + li;
                float v = acc[r][t][i] + b;
                if (a.x3) {
                    const int64_t row = m0 + wm * 64 + rr;
                    if (row < a.m && c < a.n)
                        v += t_to_f32<XT>(a.x3[row * a.n + c]);
                }
                tile[rr * ER + cc] = f32_to_t<XT>(v);
            }
    }
    __syncthreads();
    // 64 rows x WN / 8 pieces of 8 elements per wave tile: WN / 8 pieces per lane.
#pragma unroll
    for (int p = 0; p < WN / 8; ++p) {
        const int q = p * kWave + lane, rr = q / (WN / 8), pc = q % (WN / 8);
        const int64_t row = m0 + wm * 64 + rr;
        const int64_t c0 = n0 + wn * WN + pc * 8;
        if (row >= a.m)
            continue;
        const uint4 v = *reinterpret_cast<const uint4*>(&tile[rr * ER + pc * 8]);
        uint16_t* dst = a.out + row * a.n + c0;
        if (c0 + 8 <= a.n && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint16_t e[8] = {static_cast<uint16_t>(v.x), static_cast<uint16_t>(v.x >> 16),
                                   static_cast<uint16_t>(v.y), static_cast<uint16_t>(v.y >> 16),
                                   static_cast<uint16_t>(v.z), static_cast<uint16_t>(v.z >> 16),
                                   static_cast<uint16_t>(v.w), static_cast<uint16_t>(v.w >> 16)};
            for (int j = 0; j < 8; ++j)
                if (c0 + j < a.n)
                    dst[j] = e[j];
        }
    }
}

template <int XT, int WT>
__global__ __launch_bounds__(kBlock) void wq_generic_kernel(const WqArgs a, int pol, bool trans)
{
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (idx >= a.m * a.n)
        return;
    const int64_t row = idx / a.n, c = idx - row * a.n;
    float acc = 0.0f;
    float s = 0.0f, o = 0.0f;
    if (pol != DQ_PER_GROUP) {
        const int64_t p = pol == DQ_PER_TENSOR ? 0 : c;
        s = t_to_f32<XT>(a.scale[p]);
        o = a.offset ? t_to_f32<XT>(a.offset[p]) : 0.0f;
    }
    for (int64_t kk = 0; kk < a.k; ++kk) {
        if (pol == DQ_PER_GROUP && kk % a.group_size == 0) {
            const int64_t p = trans ? c * a.groups + kk / a.group_size : (kk / a.group_size) * a.n + c;
            s = t_to_f32<XT>(a.scale[p]);
            o = a.offset ? t_to_f32<XT>(a.offset[p]) : 0.0f;
        }
        const int64_t e = trans ? c * a.k + kk : kk * a.n + c;
        float v;
        if constexpr (WT == WQ_I8) {
            v = static_cast<float>(reinterpret_cast<const int8_t*>(a.x2)[e]);
        } else {
            const uint32_t byte = a.x2[e / 2];
            const int32_t nib = static_cast<int32_t>((e & 1) ? byte >> 4 : byte & 0xFu);
            v = static_cast<float>(nib >= 8 ? nib - 16 : nib);
        }
        const float w = a.offset ? dequant1<WQ_I8, true>(v, s, o) : dequant1<WQ_I8, false>(v, s, o);
        const float wt = t_to_f32<XT>(f32_to_t<XT>(w));
        acc += t_to_f32<XT>(a.x1[row * a.k + kk]) * wt;
    }
    if (a.bias)
        acc += t_to_f32<XT>(a.bias[c]);
    if (a.x3)
        acc += t_to_f32<XT>(a.x3[row * a.n + c]);
    a.out[idx] = f32_to_t<XT>(acc);
}

// out = RN_T(((partial[0] + partial[1]) + ...) + bias + x3), splits in order.
template <int XT>
__global__ __launch_bounds__(kBlock) void wq_reduce_kernel(const WqArgs a, int splits)
{
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    const int64_t total = a.m * a.n;
    if (idx >= total)
        return;
    float v = a.partial[idx];
    for (int z = 1; z < splits; ++z)
        v += a.partial[static_cast<int64_t>(z) * total + idx];
    if (a.bias)
        v += t_to_f32<XT>(a.bias[idx % a.n]);
    if (a.x3)
        v += t_to_f32<XT>(a.x3[idx]);
    a.out[idx] = f32_to_t<XT>(v);
}

template <int XT, int WT, int POL, bool OFF, int RN, int U>
hipError_t launch_decode(const WqArgs& a, int splits, hipStream_t stream)
{
    const int64_t cols = static_cast<int64_t>(kWqDecodeWaves) * 16 * RN;
    const int64_t gx = (a.n + cols - 1) / cols;
    const dim3 grid(static_cast<uint32_t>(gx), 1, static_cast<uint32_t>(splits));
    // Batch starts (k_chunk is a multiple of the batch) fall on even groups.
    if constexpr (POL == DQ_PER_GROUP && U == 2) {
        if (a.group_size == kWqSuper && a.groups % 2 == 0 && a.k_chunk % (U * kWqSuper) == 0)
            hipLaunchKernelGGL((wq_decode_kernel<XT, WT, POL, OFF, RN, U, true>), grid, dim3(kWqDecodeWaves * kWave),
                               0, stream, a);
        else
            hipLaunchKernelGGL((wq_decode_kernel<XT, WT, POL, OFF, RN, U, false>), grid,
                               dim3(kWqDecodeWaves * kWave), 0, stream, a);
    } else {
        hipLaunchKernelGGL((wq_decode_kernel<XT, WT, POL, OFF, RN, U, false>), grid, dim3(kWqDecodeWaves * kWave), 0,
                           stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || splits == 1)
        return err;
    const int64_t blocks = (a.m * a.n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL((wq_reduce_kernel<XT>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream, a, splits);
    return hipGetLastError();
}

// Whether the LDS-tiled kernel can take per-group parameters in windows:
// groups of one k-step, whole windows per column and per split, and 16-byte
// aligned parameter rows.
template <int POL, bool OFF>
bool gemm_param_window(const WqArgs& a)
{
    if (POL != DQ_PER_GROUP)
        return false;
    const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return a.group_size == kGemmBK && a.groups % kWqParamWindow == 0 && a.k_chunk % (kWqParamWindow * kGemmBK) == 0 &&
           al16(a.scale) && (!OFF || al16(a.offset));
}

template <int XT, int WT, int POL, bool OFF>
hipError_t launch_gemm(const WqArgs& a, int splits, hipStream_t stream)
{
    const int64_t gx = (a.n + kGemmBN - 1) / kGemmBN;
    const int64_t gy_total = (a.m + kGemmBM - 1) / kGemmBM;
    constexpr int64_t kMaxY = 65535;
    if (splits > 1 && gy_total > kMaxY)
        return hipErrorInvalidConfiguration;  // split k is planned for few tiles only
    for (int64_t y0 = 0; y0 < gy_total; y0 += kMaxY) {
        WqArgs c = a;
        c.x1 = a.x1 + y0 * kGemmBM * a.k;
        c.out = a.out + y0 * kGemmBM * a.n;
        c.x3 = a.x3 ? a.x3 + y0 * kGemmBM * a.n : nullptr;
        c.m = a.m - y0 * kGemmBM < kMaxY * kGemmBM ? a.m - y0 * kGemmBM : kMaxY * kGemmBM;
        const int64_t gy = (c.m + kGemmBM - 1) / kGemmBM;
        const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy), static_cast<uint32_t>(splits));
        if constexpr (POL == DQ_PER_GROUP) {
            if (gemm_param_window<POL, OFF>(a))
                hipLaunchKernelGGL((wq_gemm_kernel<XT, WT, POL, OFF, true>), grid, dim3(kGemmThreads), 0, stream, c);
            else
                hipLaunchKernelGGL((wq_gemm_kernel<XT, WT, POL, OFF, false>), grid, dim3(kGemmThreads), 0, stream, c);
        } else {
            hipLaunchKernelGGL((wq_gemm_kernel<XT, WT, POL, OFF, false>), grid, dim3(kGemmThreads), 0, stream, c);
        }
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    if (splits > 1) {
        const int64_t blocks = (a.m * a.n + kBlock - 1) / kBlock;
        hipLaunchKernelGGL((wq_reduce_kernel<XT>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream, a,
                           splits);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int XT, int WT, int POL, bool OFF>
hipError_t pick_tile(const WqPlan& p, const WqArgs& a, hipStream_t stream)
{
    if (p.tile == WQ_TILE_DECODE)
        return launch_decode<XT, WT, POL, OFF, kWqDecodeCols, wq_batch(WQ_TILE_DECODE)>(a, p.splits, stream);
    return launch_gemm<XT, WT, POL, OFF>(a, p.splits, stream);
}

template <int XT, int WT, int POL>
hipError_t pick_off(const WqPlan& p, const WqArgs& a, hipStream_t stream)
{
    return a.offset ? pick_tile<XT, WT, POL, true>(p, a, stream) : pick_tile<XT, WT, POL, false>(p, a, stream);
}

template <int XT, int WT>
hipError_t launch_wt(const WqPlan& p, const WqArgs& a, hipStream_t stream)
{
    if (p.variant == WQ_VAR_GENERIC) {
        const int64_t total = a.m * a.n;
        const int64_t blocks = (total + kBlock - 1) / kBlock;
        if (blocks > kMaxGridBlocks)
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((wq_generic_kernel<XT, WT>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream, a,
                           p.policy, p.transpose_x2);
        return hipGetLastError();
    }
    switch (p.policy) {
    case DQ_PER_TENSOR: return pick_off<XT, WT, DQ_PER_TENSOR>(p, a, stream);
    case DQ_PER_CHANNEL: return pick_off<XT, WT, DQ_PER_CHANNEL>(p, a, stream);
    default: return pick_off<XT, WT, DQ_PER_GROUP>(p, a, stream);
    }
}

}  // namespace

hipError_t launch_weight_quant_matmul(const WqPlan& p, void* workspace, hipStream_t stream)
{
    if (p.m == 0 || p.n == 0)
        return hipSuccess;
    WqArgs a;
    a.x1 = static_cast<const uint16_t*>(p.x1);
    a.x2 = static_cast<const uint8_t*>(p.x2);
    a.scale = static_cast<const uint16_t*>(p.scale);
    a.offset = static_cast<const uint16_t*>(p.offset);
    a.bias = static_cast<const uint16_t*>(p.bias);
    a.x3 = static_cast<const uint16_t*>(p.x3);
    a.out = static_cast<uint16_t*>(p.out);
    a.m = p.m;
    a.k = p.k;
    a.n = p.n;
    a.group_size = p.group_size > 0 ? p.group_size : 1;
    a.groups = p.group_size > 0 ? (p.k + p.group_size - 1) / p.group_size : 1;
    a.k_chunk = p.k_chunk;
    a.partial = p.splits > 1 ? static_cast<float*>(workspace) : nullptr;
    a.by_gs = div_magic(static_cast<uint64_t>(a.group_size));
    if (p.x_type == X_BF16)
        return p.w_type == WQ_I8 ? launch_wt<X_BF16, WQ_I8>(p, a, stream) : launch_wt<X_BF16, WQ_I4>(p, a, stream);
    return p.w_type == WQ_I8 ? launch_wt<X_F16, WQ_I8>(p, a, stream) : launch_wt<X_F16, WQ_I4>(p, a, stream);
}

}  // namespace dq
