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
//     exact.  The decode kernel, where that arithmetic bounds the time,
//     takes the offset and scale in one FMA where wq_fma.h shows it exact
//     (nearly always) and the step-by-step form otherwise.  A run of 32 k
//     never straddles a parameter group (the group size is a multiple of
//     32).
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

#include <atomic>
#include <type_traits>

#include "dq_device.h"
#include "dq_ext_internal.h"
#include "wq_fma.h"

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
// N = 1, 2 or 4 consecutive dwords with one load (off a multiple of 4 N).
template <int N>
__device__ __forceinline__ void buf_load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t (&w)[N])
{
    if constexpr (N == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (N == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = static_cast<uint32_t>(v[0]);
        w[1] = static_cast<uint32_t>(v[1]);
    } else {
        static_assert(N == 4, "one load of 4, 8 or 16 bytes");
        const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        w[0] = static_cast<uint32_t>(v.x);
        w[1] = static_cast<uint32_t>(v.y);
        w[2] = static_cast<uint32_t>(v.z);
        w[3] = static_cast<uint32_t>(v.w);
    }
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

// The one-FMA form of the dequantization with offset and when it is exact
// (wq_fma.h), for this kernel's code width and T.
template <int WT, int XT>
__device__ __forceinline__ bool fma_exact(float o, float s, float os)
{
    return wq_fma_exact(o, s, os, wq_fma_offset_floor(WT == WQ_I4, XT == X_BF16));
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
// PAIR: per-group parameters with groups of 128 (one per superstep) and a
// group count that is a multiple of U, so the U groups of a batch are
// adjacent in a column's parameter row and one load of 2 U bytes fetches
// them all (the loads of the per-group parameters cost as much time as the
// weight stream when made one by one).
template <int XT, int WT, int POL, bool OFF, int RN, int U, bool PAIR>
__global__ __launch_bounds__(kWqDecodeWaves * kWave) void wq_decode_kernel(const WqArgs a)
{
    static_assert(!PAIR || (POL == DQ_PER_GROUP && (U == 2 || U == 4 || U == 8)),
                  "grouped parameters: 2, 4 or 8 supersteps of 128 per batch, one load of 4, 8 or 16 bytes");
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
    bool chan_fma = false;  // per-tensor or per-channel: every column's parameters pass fma_exact
    if constexpr (POL != DQ_PER_GROUP) {
        bool ok = true;
#pragma unroll
        for (int t = 0; t < RN; ++t) {
            const int64_t p = param_index<POL>(a, col[t], 0, true);
            s_chan[t] = t_to_f32<XT>(a.scale[p]);
            o_chan[t] = OFF ? t_to_f32<XT>(a.offset[p]) : 0.0f;
            ok = ok && fma_exact<WT, XT>(o_chan[t], s_chan[t], o_chan[t] * s_chan[t]);
        }
        chan_fma = __all(ok);
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
                const uint32_t pi = static_cast<uint32_t>(col[t] * a.groups) + kb / kWqSuper;  // a multiple of U
                uint32_t sv[U / 2], ov[U / 2];
                buf_load_words<U / 2>(srs, pi * 2, sv);
                if constexpr (OFF)
                    buf_load_words<U / 2>(ors, pi * 2, ov);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    sg[u][t] = t_to_f32<XT>(static_cast<uint16_t>(sv[u / 2] >> (16 * (u % 2))));
                    og[u][t] = OFF ? t_to_f32<XT>(static_cast<uint16_t>(ov[u / 2] >> (16 * (u % 2)))) : 0.0f;
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
                // The test is wave-uniform, so the slower exact paths below
                // are a scalar branch taken only when some lane needs them.
                bool use_fma = false;
                float os = 0.0f;
                if constexpr (OFF) {
                    os = of * sc;
                    use_fma = POL == DQ_PER_GROUP ? __all(fma_exact<WT, XT>(of, sc, os)) : chan_fma;
                }
                if (use_fma) {
                    // int4 decodes to 16 code, and s / 16 is exact.
                    const float s_eff = WT == WQ_I4 ? sc * 0.0625f : sc;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        float v[8], wv[8];
                        decode8<WT>(w[u][t][0], w[u][t][WV - 1], s2, v);
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            wv[j] = __builtin_fmaf(v[j], s_eff, os);
                        bv[s2] = pack8_t<XT>(wv);
                    }
                } else if constexpr (WT == WQ_I4 && OFF) {
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
    // while batch b is computed (two or three batches ahead measured slower).
    // nb is uniform (no batch when k is empty).
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
// Balanced decode kernel (at most 16 rows, int4 weights in groups of 128 k):
// one workgroup of eight waves per compute unit.  The workgroup owns CB
// column blocks of 16 (the host picks CB = n / (16 * 256), so the 256
// workgroups fill the 256 compute units once), and wave w takes the k-range
// [w k / 8, (w + 1) k / 8) of all CB blocks.  Every SIMD then carries two
// waves of equal work, where the per-wave layout above leaves some SIMDs
// with two waves and others with one (n / 16 blocks are not a multiple of
// the SIMD count).  The eight partial sums of each output meet in LDS at the
// end and are added in wave order.
//
// Per batch of two supersteps (256 k) a wave stages its own x1 slice in LDS
// with direct-to-LDS loads, double-buffered, and keeps each block's next
// weights in flight from the moment the block's registers are free (both
// supersteps of a block at once: they share each column's 128-byte line).  The
// per-group parameters come into LDS eight groups (four batches) at a time,
// one 16-byte load per column and kind: loads of one dword per column and
// batch measured 5 us slower at 16 x 8192 x 28672.  Each x1 operand read serves CB blocks.  The operand
// and parameter reads from LDS are written in assembly with their wait: the
// compiler, seeing LDS reads after direct-to-LDS loads, would otherwise wait
// for every outstanding load there; an explicit wait on the vector memory
// counter orders them instead.  Their outputs are early-clobber: a read's
// data can land while later reads of the same block still need the address
// register, so no output may share a register with an input.
// ---------------------------------------------------------------------------
constexpr int kWqBalWaves = 8;

template <int XT, bool OFF, int CB>
__global__ __launch_bounds__(kWqBalWaves * kWave, 1) void wq_bal_kernel(const WqArgs a)
{
    constexpr int WT = WQ_I4, U = 2;
    constexpr int BK = U * kWqSuper;  // k per batch
    constexpr int CH = BK / 8;        // 16-byte chunks per x1 row and batch
    constexpr int SL = 16 * CH;       // x1 slots per wave buffer
    constexpr int XI = SL / kWave;    // direct-to-LDS loads of x1 per wave and batch
    constexpr int PC = 2 * kWave;     // parameter columns per kind (CB * 16, padded)
    constexpr int PB = 4;             // batches per parameter chunk (8 groups, 16 bytes a column)
    static_assert(CB >= 1 && CB <= kWqBalMaxBlocks && 16 * CB <= PC && XI * kWave == SL && CH == 32,
                  "geometry of the balanced decode kernel");
    // x1 slots [wave][buffer][slot] (128 KB); parameter chunks [wave][scale,
    // offset][column] (32 KB): eight groups as T bits, dword j holding batch
    // j's two (low half the first).  Each parameter load writes 64 lanes, so
    // rows hold 128 columns.
    __shared__ __align__(16) uint4 xs[kWqBalWaves][2][SL];
    __shared__ __align__(16) uint4 ps[kWqBalWaves][2][PC];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int li = lane % 16, g = lane / 16;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * CB);
    const uint32_t kw = static_cast<uint32_t>(a.k / kWqBalWaves);  // k per wave
    const uint32_t k0 = static_cast<uint32_t>(wave) * kw;
    const int nb = static_cast<int>(kw / BK);

    // The host keeps the weights, x1 and the parameters below 2^31 bytes.
    // Offsets past a resource's end read zeros with no memory access: x1
    // rows past m, parameter columns past the workgroup's, and the staging
    // of the batch after a wave's last.
    constexpr uint32_t kPast = 0xFFFFFFF0u;
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(a.x2, static_cast<uint32_t>(a.n * (a.k / 2)));
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x1, static_cast<uint32_t>(a.m * a.k * 2));
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(a.scale, static_cast<uint32_t>(a.n * a.groups * 2));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(OFF ? a.offset : a.scale, static_cast<uint32_t>(a.n * a.groups * 2));
    uint32_t wcol[CB];  // byte offset of this lane's run in each block's column
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        wcol[cb] = static_cast<uint32_t>((n0 + 16 * cb + li) * (a.k / 2)) + 16u * g;

    // x1 of batch b into LDS buffer buf: load p, lane l fills slot 64 p + l,
    // row r = 2 p + l / 32, with chunk (l % 32) ^ (r % 16) of the row (8 k
    // each), so the operand reads below (16 rows, one chunk each) touch 16
    // distinct 16-byte slots modulo 256 bytes in every group of 16 lanes
    // (gfx950 serves 16-byte reads 16 lanes at a time over 64 banks).
    auto stage_x = [&](int b, int buf) {
        const bool in = b < nb;
#pragma unroll
        for (int p = 0; p < XI; ++p) {
            const int r = 2 * p + lane / 32;
            const int c = (lane % 32) ^ (r % 16);
            const uint32_t off = (static_cast<uint32_t>(r) * static_cast<uint32_t>(a.k) + k0 +
                                  static_cast<uint32_t>(b) * BK + 8u * static_cast<uint32_t>(c)) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, &xs[wave][buf][64 * p], 16, in ? off : kPast, 0, 0, 0);
        }
    };
    // Parameter chunk q (batches PB q .. PB q + PB - 1): lane l of load i
    // takes column 64 i + l of the workgroup, 16 bytes of its groups.
    auto stage_p = [&](int q) {
        const uint32_t gb = (k0 + static_cast<uint32_t>(q) * (PB * BK)) / kWqSuper;
#pragma unroll
        for (int kind = 0; kind < (OFF ? 2 : 1); ++kind)
#pragma unroll
            for (int i = 0; i < PC / kWave; ++i) {
                const int c = kWave * i + lane;
                const uint32_t off = c < 16 * CB ? static_cast<uint32_t>((n0 + c) * a.groups + gb) * 2u : kPast;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kind ? ors : srs, &ps[wave][kind][kWave * i], 16, off, 0, 0,
                                                         0);
            }
    };
    auto load_w = [&](int b, int u, int cb, uint4 (&w)[U][CB]) {
        const uint32_t kb = k0 + static_cast<uint32_t>(b) * BK;
        w[u][cb] = buf_load16<kBufNonTemporal>(wrs, b < nb ? wcol[cb] + kb / 2 + 64u * u : kPast);
    };

    // Vector memory operations retire in order: batch b's staging (and a
    // parameter chunk's) is followed by its weight loads (U CB), issued while
    // batch b - 1 is computed, so the staging (and all before it) is complete
    // once that many or fewer are outstanding.
    constexpr int kAfter = U * CB;
    static_assert(kAfter < 64, "vmcnt range");
    auto wait_vm = [&](auto n_outstanding) {
        constexpr int n = decltype(n_outstanding)::value;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
        asm volatile("" ::: "memory");
    };

    // Waves w and w + 4 share a SIMD and run the same instruction stream;
    // giving the first the higher issue priority lets it run ahead while the
    // second fills the SIMD's idle cycles, instead of both waiting for
    // memory at the same points.
    if (wave < 4)
        __builtin_amdgcn_s_setprio(2);
    f32x4 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        acc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    uint4 w[U][CB];
    stage_p(0);
    stage_x(0, 0);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int u = 0; u < U; ++u)
            load_w(0, u, cb, w);
    const uint32_t xs_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&xs[wave][0][0]));
    const uint32_t ps_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ps[wave][0][0]));
    // Scale and offset dwords (T bits) of the 7 block slots at LDS address
    // pa: block cb at pa + 256 cb, offsets at pa + 2048 (slots past CB read
    // padding columns, unused).
    auto read_params = [&](uint32_t pa, uint32_t (&sp)[kWqBalMaxBlocks], uint32_t (&op)[kWqBalMaxBlocks]) {
        asm volatile(
            "ds_read_b32 %0, %14 offset:0\n\t"
            "ds_read_b32 %1, %14 offset:256\n\t"
            "ds_read_b32 %2, %14 offset:512\n\t"
            "ds_read_b32 %3, %14 offset:768\n\t"
            "ds_read_b32 %4, %14 offset:1024\n\t"
            "ds_read_b32 %5, %14 offset:1280\n\t"
            "ds_read_b32 %6, %14 offset:1536\n\t"
            "ds_read_b32 %7, %14 offset:2048\n\t"
            "ds_read_b32 %8, %14 offset:2304\n\t"
            "ds_read_b32 %9, %14 offset:2560\n\t"
            "ds_read_b32 %10, %14 offset:2816\n\t"
            "ds_read_b32 %11, %14 offset:3072\n\t"
            "ds_read_b32 %12, %14 offset:3328\n\t"
            "ds_read_b32 %13, %14 offset:3584\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(sp[0]), "=&v"(sp[1]), "=&v"(sp[2]), "=&v"(sp[3]), "=&v"(sp[4]), "=&v"(sp[5]), "=&v"(sp[6]),
              "=&v"(op[0]), "=&v"(op[1]), "=&v"(op[2]), "=&v"(op[3]), "=&v"(op[4]), "=&v"(op[5]), "=&v"(op[6])
            : "v"(pa)
            : "memory");
    };
    uint64_t okm[kWqBalMaxBlocks][U] = {};
    for (int b = 0; b < nb; ++b) {
        const int buf = b & 1;
        wait_vm(std::integral_constant<int, kAfter>{});
        stage_x(b + 1, buf ^ 1);
        // Once per parameter chunk, with an offset: whether the one-FMA form
        // holds (wq_fma.h) for every block, superstep and batch of the chunk,
        // lane group g checking batch PB q + g of column li, so bit 16 g + li
        // of okm[cb][u] covers that column's group (a quarter of the checks a
        // per-batch test of every lane makes).
        if constexpr (OFF) {
            if (b % PB == 0) {
                uint32_t cs[kWqBalMaxBlocks], co[kWqBalMaxBlocks];
                read_params(ps_base + static_cast<uint32_t>(li * 16 + g * 4), cs, co);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const float sc = t_to_f32<XT>(static_cast<uint16_t>(cs[cb] >> (16 * u)));
                        const float of = t_to_f32<XT>(static_cast<uint16_t>(co[cb] >> (16 * u)));
                        okm[cb][u] = __ballot(fma_exact<WT, XT>(of, sc, of * sc));
                    }
            }
        }
        // This batch's parameters: dword b % PB of each column's chunk.
        uint32_t sp[kWqBalMaxBlocks], op[kWqBalMaxBlocks];
        read_params(ps_base + static_cast<uint32_t>(li * 16 + (b % PB) * 4), sp, op);
        // The chunk's last batch has read it: the next chunk comes in now, ahead
        // of the next batch's weights (the wait above covers it then).
        if (b % PB == PB - 1 && b + 1 < nb)
            stage_p((b + 1) / PB);
        // x1 operands of the batch: superstep u, lane group g and sub-step s2
        // take chunk 16 u + 4 g + s2 of row li (the k assignment of the
        // decode kernel above); both supersteps in one round trip.
        static_assert(U == 2, "operand reads written for two supersteps");
        uint4 av[U][4];
        uint32_t ad[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const int c = 16 * u + 4 * g + s2;
                ad[u][s2] = xs_base + static_cast<uint32_t>((buf * SL + li * CH + (c ^ li)) * 16);
            }
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %9\n\t"
            "ds_read_b128 %2, %10\n\t"
            "ds_read_b128 %3, %11\n\t"
            "ds_read_b128 %4, %12\n\t"
            "ds_read_b128 %5, %13\n\t"
            "ds_read_b128 %6, %14\n\t"
            "ds_read_b128 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(av[0][0]), "=&v"(av[0][1]), "=&v"(av[0][2]), "=&v"(av[0][3]), "=&v"(av[1][0]), "=&v"(av[1][1]),
              "=&v"(av[1][2]), "=&v"(av[1][3])
            : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[0][2]), "v"(ad[0][3]), "v"(ad[1][0]), "v"(ad[1][1]),
              "v"(ad[1][2]), "v"(ad[1][3])
            : "memory");
        // Block by block, both supersteps of a block before the next block, so
        // a block's registers free (and its next runs go out) at (cb + 1) / CB
        // of the batch, almost a whole batch before they are used.
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float sc = t_to_f32<XT>(static_cast<uint16_t>(sp[cb] >> (16 * u)));
                const float of = OFF ? t_to_f32<XT>(static_cast<uint16_t>(op[cb] >> (16 * u))) : 0.0f;
                uint4 bv[4];
                bool use_fma = false;
                float os = 0.0f;
                if constexpr (OFF) {
                    os = of * sc;
                    use_fma = ((okm[cb][u] >> (16 * (b % PB))) & 0xFFFFull) == 0xFFFFull;
                }
                if (!OFF || use_fma) {
                    // int4 decodes to 16 code and s / 16 is exact; with an
                    // offset, RN(16 code * (s / 16) + RN(o s)) is the formula
                    // where fma_exact holds (wq_fma.h).
                    const float s_eff = sc * 0.0625f;
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        float v[8], wv[8];
                        decode8<WT>(w[u][cb], w[u][cb], s2, v);
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            wv[j] = OFF ? __builtin_fmaf(v[j], s_eff, os) : v[j] * s_eff;
                        bv[s2] = pack8_t<XT>(wv);
                    }
                } else {
                    // As in the decode kernel: RN(RN(16 code + 16 o) * (s / 16))
                    // unless 16 o overflows, then the formula step by step.
                    const float o16 = of * 16.0f, s16 = sc * 0.0625f;
                    const bool huge = __any(__builtin_isinf(o16));
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        float v[8], wv[8];
                        decode8<WT>(w[u][cb], w[u][cb], s2, v);
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
                }
                // The block's registers are free: the next batch's runs go
                // out, both supersteps together, since they are the two
                // halves of one 128-byte line per column (issued apart, the
                // line was often fetched twice: 1.64 times the algorithmic
                // bytes at 16 x 8192 x 28672).
                if (u == U - 1)
#pragma unroll
                    for (int uu = 0; uu < U; ++uu)
                        load_w(b + 1, uu, cb, w);
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    acc[cb] = mfma16<XT>(av[u][s2], bv[s2], acc[cb]);
            }
        }
    }

    // Partial sums of the eight waves meet in LDS over the x1 buffers, once
    // every direct-to-LDS load (the empty staging after the last batch
    // included) has landed and every wave has finished reading.
    wait_vm(std::integral_constant<int, 0>{});
    __syncthreads();
    static_assert(sizeof(f32x4) * kWqBalWaves * kWqBalMaxBlocks * kWave <= sizeof(xs), "partial sums fit");
    f32x4* const red = reinterpret_cast<f32x4*>(&xs[0][0][0]);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        red[(wave * CB + cb) * kWave + lane] = acc[cb];
    __syncthreads();
    if (tid < CB * kWave) {
        const int cb = tid / kWave, l = tid % kWave;
        f32x4 s = red[cb * kWave + l];
#pragma unroll
        for (int w8 = 1; w8 < kWqBalWaves; ++w8)
            s += red[(w8 * CB + cb) * kWave + l];
        // Lane l holds rows 4 (l / 16) .. + 3 of column l % 16 of the block.
        const int64_t c = n0 + 16 * cb + l % 16;
        const float bias = a.bias ? t_to_f32<XT>(a.bias[c]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = 4 * (l / 16) + i;
            if (row >= a.m)
                continue;
            float v = s[i] + bias;
            if (a.x3)
                v += t_to_f32<XT>(a.x3[row * a.n + c]);
            a.out[row * a.n + c] = f32_to_t<XT>(v);
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

// ---------------------------------------------------------------------------
// Wide prefill kernel: a 256 x 256 output tile per workgroup of four waves.
// Wave w owns the 64 columns 64 w .. 64 w + 63 over all 256 rows (8 x 2
// blocks of 32 x 32 on v_mfma_f32_32x32x16, 256 binary32 sums per lane in
// the accumulation registers), so each weight is loaded and dequantized by
// exactly one wave, straight from global memory into the matrix-core
// operand registers, and only x1 goes through LDS (double-buffered, one
// barrier per k-step of 64).  Per k-step a wave runs 64 matrix-core
// instructions (2048 cycles) against 32 KB of x1 operand reads per wave and
// 32 KB of staging stores per workgroup: LDS time is about three quarters
// of the matrix-core time, where the 128 x 128 tile above needs twice it.
// (With 16 x 16 blocks the same tile left the compiler copying accumulators
// between register files every step; 32 x 32 blocks keep them in place.)
//
// Operand layout of v_mfma_f32_32x32x16: lane l supplies row (or column)
// l % 32 and 8 k values; it receives rows 8 j + 4 (l / 32) + i (j, i < 4) of
// column l % 32.  k order inside a step: lane half h = l / 32 holds the 32
// consecutive k of [32 h, 32 h + 32), slice s (of 4) taking the 8 k from
// 32 h + 8 s, for x1 and for the weights alike, so a lane's weights of a
// step are one contiguous run of its column (32 bytes of int8, 16 of int4).
// x1 rows sit in LDS as 8 chunks of 8 k per row, chunk c of row r in slot
// c ^ (r % 8): the staging stores (8 lanes on one row) and the operand
// reads (8 lanes on 8 rows, one chunk) each touch 8 distinct 16-byte slots
// of a 128-byte window, free of bank conflicts without padding.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int XT>
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c)
{
    if constexpr (XT == X_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                       0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

template <int WT>
struct WideRaw;
template <>
struct WideRaw<WQ_I8> {
    uint4 lo, hi;  // 32 codes
};
template <>
struct WideRaw<WQ_I4> {
    uint4 lo;  // 32 codes
};

template <int XT, int WT, int POL, bool OFF>
__global__ __launch_bounds__(kWave * 4, 1) void wq_wide_kernel(const WqArgs a)
{
    constexpr int BM = kWqWideRows, BN = kWqWideCols, BK = kWqWideK, NT = kWave * 4;
    constexpr int RB = BM / 32;             // row blocks (all rows, every wave)
    constexpr int CB = BN / 4 / 32;         // column blocks per wave
    constexpr int SL = BK / 16;             // k slices per step
    constexpr int AV = BM * (BK / 8) / NT;  // 16-byte x1 vectors staged per thread and step
    constexpr int WSTEP = WT == WQ_I8 ? BK : BK / 2;  // weight bytes per column and step
    constexpr int ER = 64;                  // epilogue tile row (binary32)
    constexpr int kBuf = BM * (BK / 8);  // 16-byte chunks per x1 buffer
    static_assert(AV * NT == BM * BK / 8 && AV == 8, "x1 tile divides over threads");
    static_assert(RB == 8 && CB == 2 && SL == 4, "32 row-block iterations per step, 2 column blocks per wave");
    static_assert(4 * 32 * ER * 4 <= kBuf * 16, "the epilogue tiles fit one x1 buffer");
    // Two x1 buffers as two arrays, so the compiler can tell a buffer being
    // filled by direct-to-LDS loads from the one being read.  The epilogue
    // reuses the first.
    __shared__ __align__(16) uint4 As0[kBuf], As1[kBuf];
    auto abuf = [&](int b) -> uint4* { return b ? As1 : As0; };
    unsigned char* const smem = reinterpret_cast<unsigned char*>(As0);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int li = lane % 32, h = lane / 32;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
    const int64_t k_beg = static_cast<int64_t>(blockIdx.z) * a.k_chunk;
    const int64_t k_end = k_beg + a.k_chunk < a.k ? k_beg + a.k_chunk : a.k;
    const int nk = static_cast<int>((k_end - k_beg) / BK);  // the host plans whole pairs of steps

    // Buffer resources over this tile's x1 rows and weight columns (the host
    // keeps 256 rows of x1 and 256 weight columns below 2^31 bytes): loads
    // past the last row or column return zeros, whose results are not stored.
    const int64_t kw = WT == WQ_I8 ? a.k : a.k / 2;  // weight bytes per column
    const int64_t rows_left = a.m - m0 < BM ? a.m - m0 : BM, cols_left = a.n - n0 < BN ? a.n - n0 : BN;
    const __amdgpu_buffer_rsrc_t xrs =
        make_rsrc(a.x1 + m0 * a.k + k_beg, static_cast<uint32_t>((rows_left * a.k - k_beg) * 2));
    const __amdgpu_buffer_rsrc_t wrs =
        make_rsrc(a.x2 + n0 * kw + (k_beg / BK) * WSTEP, static_cast<uint32_t>(cols_left * kw - (k_beg / BK) * WSTEP));
    // x1 vector p of thread tid: row tid / 8 + 32 p, chunk tid % 8.
    const uint32_t a_off = static_cast<uint32_t>((tid / 8) * a.k * 2 + (tid % 8) * 16);
    const uint32_t a_pstride = static_cast<uint32_t>(32 * a.k * 2);
    const int a_slot = (tid / 16) % 8;  // (row / 2) % 8 of every staged row of this thread
    // This lane's weight runs: column block cb is column 64 wave + 32 cb + li of the tile.
    const uint32_t w_off = static_cast<uint32_t>((64 * wave + li) * kw + h * (WSTEP / 2));
    const uint32_t w_cbstride = static_cast<uint32_t>(32 * kw);
    // Parameter row offsets of this lane's columns (the host keeps n * groups
    // below 2^31).
    uint32_t prow[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t c = n0 + 64 * wave + 32 * cb + li;
        prow[cb] = static_cast<uint32_t>((c < a.n ? c : a.n - 1) * (POL == DQ_PER_GROUP ? a.groups : 1));
    }

    auto load_a = [&](int kt, uint4 (&ar)[AV]) {
#pragma unroll
        for (int p = 0; p < AV; ++p)
            ar[p] = buf_load16<0>(xrs, a_off + p * a_pstride + static_cast<uint32_t>(kt) * (BK * 2));
    };
    auto store_a1 = [&](int buf, int p, const uint4 (&ar)[AV]) {
        const int row = tid / 8 + 32 * p;
        abuf(buf)[row * 8 + ((tid % 8) ^ a_slot)] = ar[p];
    };
    // x1 of step kt straight into LDS buffer buf (direct-to-LDS buffer
    // loads, no registers): wave w's load p fills rows 64 w + 8 p .. + 7 (one
    // KB, lane l at 16 l), so lane l takes row r = 64 w + 8 p + l / 8 and
    // slot l % 8, i.e. chunk (l % 8) ^ ((r / 2) % 8) of that row.
    auto dma_a = [&](int kt, uint4* dst) {
#pragma unroll
        for (int p = 0; p < AV; ++p) {
            const int r = 64 * wave + 8 * p + lane / 8;
            const int c = (lane % 8) ^ ((r / 2) % 8);
            const uint32_t off = static_cast<uint32_t>(r) * static_cast<uint32_t>(a.k * 2) + c * 16 +
                                 static_cast<uint32_t>(kt) * (BK * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst + (64 * wave + 8 * p) * 8, 16, off, 0, 0, 0);
        }
    };
    // Wait until at most n vector-memory operations of this wave are
    // outstanding (they retire in order), then meet the workgroup barrier.
    // The direct-to-LDS loads of a buffer are complete once the loads issued
    // after them number n or fewer.  The empty asm statements keep the
    // compiler from moving LDS accesses across.
    auto wait_barrier = [&](auto n_outstanding) {
        constexpr int n = decltype(n_outstanding)::value;
        static_assert(n >= 0 && n < 64, "vmcnt range");
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto load_w = [&](int kt, WideRaw<WT> (&wr)[CB]) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint32_t off = w_off + cb * w_cbstride + static_cast<uint32_t>(kt) * WSTEP;
            wr[cb].lo = buf_load16<0>(wrs, off);
            if constexpr (WT == WQ_I8)
                wr[cb].hi = buf_load16<0>(wrs, off + 16);
        }
    };
    // Per-group parameters of step kt (groups are whole steps long), kept as
    // their T bits until the dequantization that uses them, so the loads are
    // not waited for where they are issued.
    auto load_p = [&](int kt, uint32_t (&sp)[CB], uint32_t (&op)[CB]) {
        const uint32_t grp = div_by(static_cast<uint32_t>(k_beg + static_cast<int64_t>(kt) * BK), a.by_gs);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint32_t pi = prow[cb] + grp;
            sp[cb] = a.scale[pi];
            op[cb] = OFF ? a.offset[pi] : 0u;
        }
    };

    // Parameters (T bits) of the steps held in the two weight sets (per
    // group), or of every step (per tensor, per channel: set 0 only).
    constexpr int PS = POL == DQ_PER_GROUP ? 2 : 1;
    uint32_t sp[PS][CB], op[PS][CB];
    if constexpr (POL != DQ_PER_GROUP) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint32_t pi = POL == DQ_PER_TENSOR ? 0u : prow[cb];
            sp[0][cb] = a.scale[pi];
            op[0][cb] = OFF ? a.offset[pi] : 0u;
        }
    }

    f32x16 acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            acc[rb][cb] = f32x16{};

    // Eight weights (slice sl of column block cb) of a raw set as one operand.
    auto dequant = [&](const WideRaw<WT> (&raw_set)[CB], const uint32_t (&spv)[CB], const uint32_t (&opv)[CB],
                       int cb, int sl) -> uint4 {
        const float s0 = t_to_f32<XT>(static_cast<uint16_t>(spv[cb]));
        const float of = OFF ? t_to_f32<XT>(static_cast<uint16_t>(opv[cb])) : 0.0f;
        const float sc = WT == WQ_I4 && !OFF ? s0 * 0.0625f : s0;
        float v[8], w[8];
        if constexpr (WT == WQ_I8)
            decode8<WT>(raw_set[cb].lo, raw_set[cb].hi, sl, v);
        else
            decode8<WT>(raw_set[cb].lo, raw_set[cb].lo, sl, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (OFF) {
                // RN(code + o): the decoded value times 1/16 (int4) is the code exactly.
                const float u = __builtin_fmaf(v[j], WT == WQ_I4 ? 0.0625f : 1.0f, of);
                w[j] = u * s0;
            } else {
                w[j] = v[j] * sc;
            }
        }
        return pack8_t<XT>(w);
    };

    WideRaw<WT> wr[2][CB];
    uint4 bop[SL][CB];
    if constexpr (kWqWideDma) {
        // Step kt reads LDS buffer B = kt % 2, as 32 row-block iterations of
        // two matrix-core instructions each (slice s in iterations 8 s .. 8 s
        // + 7), with the x1 operand reads three iterations ahead.  On entry
        // bop[0..2] hold step kt's slices 0-2 as operands, wr[B] step kt's raw
        // weights and wr[B ^ 1] step kt + 1's.  Spread over the iterations:
        //   0      direct-to-LDS loads of step kt + 1's x1 into the other
        //          buffer (last read in step kt - 1);
        //   1, 5   dequantize step kt's slice 3 into bop[3];
        //   8      load step kt + 2's weights into wr[B] (consumed by now);
        //   9-31   dequantize step kt + 1's slices 0, 1, 2 into bop[0..2],
        //          each after this step's use of that slice.
        // The step ends waiting for step kt + 1's x1 (only step kt + 2's
        // weight loads may remain) and meeting the barrier.
        constexpr int kWl = CB * (WT == WQ_I8 ? 2 : 1) + (POL == DQ_PER_GROUP ? CB * (OFF ? 2 : 1) : 0);
        auto step = [&](int kt, auto bsel) {
            constexpr int B = decltype(bsel)::value;
            const uint4* Ab = B ? As1 : As0;
            auto aread = [&](int it) {
                const int s = it / RB, rb = it % RB;
                return Ab[(32 * rb + li) * 8 + ((4 * h + s) ^ ((li / 2) % 8))];
            };
            uint4 av[3] = {aread(0), aread(1), aread(2)};
#pragma unroll
            for (int it = 0; it < SL * RB; ++it) {
                const int s = it / RB, rb = it % RB;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    acc[rb][cb] = mfma32<XT>(av[it % 3], bop[s][cb], acc[rb][cb]);
                if (it + 3 < SL * RB)
                    av[it % 3] = aread(it + 3);
                if (it == 0)
                    dma_a(kt + 1, B ? As0 : As1);
                if (it == 1 || it == 5)  // this step's slice 3
                    bop[3][it / 4] = dequant(wr[B], sp[B % PS], op[B % PS], it / 4, 3);
                if (it == AV) {
                    load_w(kt + 2, wr[B]);
                    if constexpr (POL == DQ_PER_GROUP)
                        load_p(kt + 2 < nk ? kt + 2 : nk - 1, sp[B % PS], op[B % PS]);
                }
                if (it >= RB && it % 4 == 1) {  // next step's slice it / 8 - 1, after this step used it
                    const int sn = it / RB - 1, cb = (it / 4) % 2;
                    bop[sn][cb] = dequant(wr[B ^ 1], sp[(B ^ 1) % PS], op[(B ^ 1) % PS], cb, sn);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_barrier(std::integral_constant<int, kWl>{});
        };

        // Steps come in pairs (the host plans k chunks of whole pairs).
        if (nk > 0) {
            dma_a(0, As0);
            load_w(0, wr[0]);
            load_w(1, wr[1]);
            if constexpr (POL == DQ_PER_GROUP) {
                load_p(0, sp[0], op[0]);
                load_p(1, sp[PS - 1], op[PS - 1]);
            }
#pragma unroll
            for (int sl = 0; sl < SL - 1; ++sl)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
                    bop[sl][cb] = dequant(wr[0], sp[0], op[0], cb, sl);
            wait_barrier(std::integral_constant<int, 0>{});
            for (int kt = 0; kt < nk; kt += 2) {
                step(kt, std::integral_constant<int, 0>{});
                step(kt + 1, std::integral_constant<int, 1>{});
            }
            // The loop's last loads (past the end) may still be writing LDS.
            wait_barrier(std::integral_constant<int, 0>{});
        }
    } else {
    // Step kt on LDS buffer B = kt % 2, as 32 row-block iterations of two
    // matrix-core instructions each (slice s in iterations 8 s .. 8 s + 7),
    // with the x1 operand reads three iterations ahead.  On entry bop[0..2]
    // hold step kt's slices 0-2 as operands, wr[B] step kt's raw weights,
    // wr[B ^ 1] step kt + 1's, ar[B] step kt + 1's x1 and ar[B ^ 1] step
    // kt + 2's.  Spread over the iterations:
    //   0-7    stage ar[B] in the other LDS buffer; dequantize step kt's
    //          slice 3 into bop[3] (free since the last step's slice 3);
    //   8      load step kt + 3's x1 into ar[B] and step kt + 2's weights
    //          into wr[B] (consumed by now);
    //   8-31   dequantize step kt + 1's slices 0, 1, 2 into bop[0..2], each
    //          after this step's use of that slice.
    // x1 is thus loaded two steps and weights one step before their use.
    // The code is straight-line: past the last step the loads read zeros
    // (past the buffer resources' ends) and the staged x1 and operands are
    // never used.  Scheduling barriers keep each iteration's work in place,
    // so the operand reads do not all move to the top.
    uint4 ar[2][AV];
    auto step = [&](int kt, auto bsel) {
        constexpr int B = decltype(bsel)::value;
        const uint4* Ab = B ? As1 : As0;
        auto aread = [&](int it) {
            const int s = it / RB, rb = it % RB;
            return Ab[(32 * rb + li) * 8 + ((4 * h + s) ^ ((li / 2) % 8))];
        };
        uint4 av[3] = {aread(0), aread(1), aread(2)};
#pragma unroll
        for (int it = 0; it < SL * RB; ++it) {
            const int s = it / RB, rb = it % RB;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[rb][cb] = mfma32<XT>(av[it % 3], bop[s][cb], acc[rb][cb]);
            if (it + 3 < SL * RB)
                av[it % 3] = aread(it + 3);
            if (it < AV)
                store_a1(B ^ 1, it, ar[B]);
            if (it == 1 || it == 5)  // this step's slice 3
                bop[3][it / 4] = dequant(wr[B], sp[B % PS], op[B % PS], it / 4, 3);
            if (it == AV) {
                load_a(kt + 3, ar[B]);
                load_w(kt + 2, wr[B]);
                if constexpr (POL == DQ_PER_GROUP)
                    load_p(kt + 2 < nk ? kt + 2 : nk - 1, sp[B % PS], op[B % PS]);
            }
            if (it >= RB && it % 4 == 1) {  // next step's slice it / 8 - 1, after this step used it
                const int sn = it / RB - 1, cb = (it / 4) % 2;
                bop[sn][cb] = dequant(wr[B ^ 1], sp[(B ^ 1) % PS], op[(B ^ 1) % PS], cb, sn);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };

    // Steps come in pairs (the host plans k chunks of whole pairs).
    if (nk > 0) {
        load_a(0, ar[1]);
        load_w(0, wr[0]);
        load_w(1, wr[1]);
        if constexpr (POL == DQ_PER_GROUP) {
            load_p(0, sp[0], op[0]);
            load_p(1, sp[PS - 1], op[PS - 1]);
        }
        load_a(1, ar[0]);
#pragma unroll
        for (int p = 0; p < AV; ++p)
            store_a1(0, p, ar[1]);
        load_a(2, ar[1]);
#pragma unroll
        for (int sl = 0; sl < SL - 1; ++sl)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                bop[sl][cb] = dequant(wr[0], sp[0], op[0], cb, sl);
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            step(kt, std::integral_constant<int, 0>{});
            step(kt + 1, std::integral_constant<int, 1>{});
        }
    }

    }

    // Epilogue in 8 passes of 32 rows (one row block): each wave writes its
    // 32 x 64 sums (+ bias) as binary32 into a padded row-major tile, then
    // every lane takes 8 consecutive columns of a row: + x3, one rounding to
    // T, one 16-byte store (or the binary32 partial sums of a k split).
    float bias[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const int64_t c = n0 + 64 * wave + 32 * cb + li;
        bias[cb] = a.bias && !a.partial ? t_to_f32<XT>(a.bias[c < a.n ? c : a.n - 1]) : 0.0f;
    }
    float* const tile = reinterpret_cast<float*>(smem) + wave * (32 * ER);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        __syncthreads();  // the previous pass's (or the main loop's) LDS reads are done
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tile[(8 * j + 4 * h + i) * ER + 32 * cb + li] = acc[rb][cb][4 * j + i] + bias[cb];
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int q = p * kWave + lane, rr = q / 8, cc = (q % 8) * 8;
            const int64_t row = m0 + 32 * rb + rr;
            const int64_t c0 = n0 + 64 * wave + cc;
            if (row >= a.m || c0 >= a.n)
                continue;
            const float4 lo = *reinterpret_cast<const float4*>(&tile[rr * ER + cc]);
            const float4 hi = *reinterpret_cast<const float4*>(&tile[rr * ER + cc + 4]);
            float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            const bool full = c0 + 8 <= a.n;
            if (a.partial) {
                float* dst = a.partial + (static_cast<int64_t>(blockIdx.z) * a.m + row) * a.n + c0;
                for (int j = 0; j < 8; ++j)
                    if (full || c0 + j < a.n)
                        dst[j] = v[j];
                continue;
            }
            uint16_t* dst = a.out + row * a.n + c0;
            const bool vec = full && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
            if (a.x3) {
                const uint16_t* x3p = a.x3 + row * a.n + c0;
                if (vec && (reinterpret_cast<uintptr_t>(x3p) & 15) == 0) {
                    const uint4 x = *reinterpret_cast<const uint4*>(x3p);
                    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[j] += t_to_f32<XT>(static_cast<uint16_t>(xw[j / 2] >> (16 * (j % 2))));
                } else {
                    for (int j = 0; j < 8; ++j)
                        if (c0 + j < a.n)
                            v[j] += t_to_f32<XT>(x3p[j]);
                }
            }
            if (vec) {
                const uint4 o = make_uint4(pack2_t<XT>(v[0], v[1]), pack2_t<XT>(v[2], v[3]),
                                           pack2_t<XT>(v[4], v[5]), pack2_t<XT>(v[6], v[7]));
                *reinterpret_cast<uint4*>(dst) = o;
            } else {
                for (int j = 0; j < 8; ++j)
                    if (c0 + j < a.n)
                        dst[j] = f32_to_t<XT>(v[j]);
            }
        }
    }
}

template <int XT, int WT, int POL, bool OFF>
hipError_t launch_wide(const WqArgs& a, int splits, hipStream_t stream)
{
    const int64_t gx = (a.n + kWqWideCols - 1) / kWqWideCols;
    const int64_t gy = (a.m + kWqWideRows - 1) / kWqWideRows;
    if (gy > 65535)
        return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy), static_cast<uint32_t>(splits));
    hipLaunchKernelGGL((wq_wide_kernel<XT, WT, POL, OFF>), grid, dim3(kWave * 4), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || splits == 1)
        return err;
    const int64_t blocks = (a.m * a.n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL((wq_reduce_kernel<XT>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream, a, splits);
    return hipGetLastError();
}

template <int XT, int WT, int POL, bool OFF, int RN, int U>
hipError_t launch_decode(const WqArgs& a, int splits, hipStream_t stream)
{
    const int64_t cols = static_cast<int64_t>(kWqDecodeWaves) * 16 * RN;
    const int64_t gx = (a.n + cols - 1) / cols;
    const dim3 grid(static_cast<uint32_t>(gx), 1, static_cast<uint32_t>(splits));
    // Batch starts (k_chunk is a multiple of the batch) fall on multiples
    // of U groups.
    if constexpr (POL == DQ_PER_GROUP && (U == 2 || U == 4 || U == 8)) {
        if (a.group_size == kWqSuper && a.groups % U == 0 && a.k_chunk % (U * kWqSuper) == 0)
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

template <int XT, bool OFF>
hipError_t launch_balanced(const WqArgs& a, hipStream_t stream)
{
    const int64_t cb = a.n / (16 * kWqBalWorkgroups);
    const dim3 grid(static_cast<uint32_t>(kWqBalWorkgroups)), block(kWqBalWaves * kWave);
    switch (cb) {
    case 1: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 4>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 5>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 6>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((wq_bal_kernel<XT, OFF, 7>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int XT, int WT, int POL, bool OFF>
hipError_t pick_tile(const WqPlan& p, const WqArgs& a, hipStream_t stream)
{
    if constexpr (WT == WQ_I4 && POL == DQ_PER_GROUP) {
        if (p.tile == WQ_TILE_BALANCED)
            return p.splits == 1 && a.group_size == kWqSuper && a.k % kWqBalKMultiple == 0 && a.m <= 16 &&
                           a.n % (16 * kWqBalWorkgroups) == 0
                       ? launch_balanced<XT, OFF>(a, stream)
                       : hipErrorInvalidValue;
    }
    if (p.tile == WQ_TILE_BALANCED)
        return hipErrorInvalidValue;
    if (p.tile == WQ_TILE_DECODE)
        return launch_decode<XT, WT, POL, OFF, kWqDecodeCols, wq_batch(WQ_TILE_DECODE, WT)>(a, p.splits, stream);
    if (p.tile == WQ_TILE_WIDE)
        return launch_wide<XT, WT, POL, OFF>(a, p.splits, stream);
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

// ---------------------------------------------------------------------------
// Split-k scratch of dq_weight_quant_matmul_noalloc: binary32 partial sums
// [splits, m, n] in a file-scope device array, one per GPU, held until the
// process ends.  Every split writes each valid partial sum before the reduce
// kernel reads it, so the array needs no clearing.  The array's name is a
// host-side stand-in: host code uses only the per-device address that
// hipGetSymbolAddress returns for it.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kWqScratchBytes];

hipError_t wq_scratch_address(void** ptr)
{
    static std::atomic<void*> cache[kWqScratchDevices];
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kWqScratchDevices)
        return hipErrorInvalidDevice;
    void* p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        if (!p)
            return hipErrorInvalidSymbol;
        cache[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

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
