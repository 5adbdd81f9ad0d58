// mx_quantize.hip -- mx block quantization on gfx950: every block of 32
// consecutive elements (along the last dimension, or down the first) shares
// one e8m0 scale.
//
// The mx formula of aclnnQuantBatchMatmulInplaceAdd (计算公式, mx量化)
// multiplies the code sums of each block of gsK = 32 elements along K by one
// FLOAT8_E8M0 scale per block and operand, the last block possibly short.
// This file produces such operands.  The pages print no producer; it follows
// the OCP Microscaling v1.0 conversion.  Per block:
//   shared = floor(log2 max|v|) - emax(element format), clamped to [-127, 127]
//   scale  = shared + 127 (an e8m0 byte)
//   code_i = the element value nearest to v_i / 2^shared, ties to even,
//            saturating at the largest finite magnitude, the sign kept on
//            zero results.
// A block holding a NaN or an infinity gets the NaN scale 0xFF and zero codes.
//
// Arithmetic.
//   - The largest magnitude is found on the 16-bit patterns.  With the sign
//     cleared, a larger pattern is a larger magnitude, and the NaN and
//     infinity patterns are the largest.  So the scale byte is integer work:
//     bf16's exponent field is binary32's, and fp16's comes from its exact
//     binary32 widening.
//   - v * 2^-shared is an exact binary32 product.  Only results far below
//     the smallest element subnormal lose bits, and they encode as a zero of
//     v's sign either way.
//   - Element rounding is the hardware's.  v_cvt_pk_fp8_f32 and
//     v_cvt_pk_bf8_f32 round to nearest even but do not saturate (overflow
//     gives NaN / infinity), so the product is first clamped to the largest
//     finite magnitude.  v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to
//     nearest even and saturates by itself.  Both keep subnormals and the
//     sign of zero.
//
// Kernels.
//   mx_row_kernel      axis 1, last dimension a multiple of 8.  A lane holds
//                      one 16-byte vector (8 elements) of a block, so a
//                      block is one lane quad.  The block maximum takes two
//                      DPP quad swaps.  Loads and stores are wave-contiguous.
//                      Each lane stores one scale byte per four vector slots,
//                      and the wave's scale stores cover 64 consecutive bytes.
//   mx_col_kernel      axis 0, last dimension a multiple of 8.  A lane holds
//                      8 adjacent columns, and each wave of a workgroup a
//                      slice of rows of one 32-row block: in-lane maxima per
//                      column, combined across the waves through LDS, and 8
//                      scale bytes per lane in one 8-byte store.
//   mx_generic_kernel  any shape or alignment: one thread per block (axis 1)
//                      or per block and column pair (axis 0), 2-byte loads.

#include "dq_device.h"
#include "dq_ext_internal.h"

namespace dq {
namespace {

constexpr int kMxBlock = 32;   // elements per scale block (gsK)
constexpr int kMxRowVecs = 4;  // vector slots per lane in mx_row_kernel
constexpr int kMxColRows = 4;  // rows per wave in mx_col_kernel (8 waves per 32-row block)
constexpr int64_t kMaxGridY = 65535;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int ELEM>
struct MxFmt;
template <>
struct MxFmt<MX_E4M3> {  // OCP FP8 E4M3FN: largest finite 448 = 1.75 * 2^8
    static constexpr uint32_t emax = 8;
    static constexpr float maxv = 448.0f;
};
template <>
struct MxFmt<MX_E5M2> {  // OCP FP8 E5M2: largest finite 57344 = 1.75 * 2^15
    static constexpr uint32_t emax = 15;
    static constexpr float maxv = 57344.0f;
};
template <>
struct MxFmt<MX_E2M1> {  // OCP MX FP4 E2M1: largest finite 6 = 1.5 * 2^2
    static constexpr uint32_t emax = 2;
    static constexpr float maxv = 6.0f;
};

// Magnitude patterns (sign bits cleared) of the two 16-bit elements of a word.
__device__ __forceinline__ uint32_t abs2(uint32_t w) { return w & 0x7FFF7FFFu; }

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Scale byte of a block from the largest magnitude pattern among its elements.
template <int XT, int ELEM>
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax16)
{
    constexpr uint32_t emax = MxFmt<ELEM>::emax;
    uint32_t e;  // biased binary32 exponent of max|v|: floor(log2 max|v|) + 127, 0 below 2^-126
    if constexpr (XT == X_BF16)
        e = amax16 >> 7;
    else
        e = __builtin_bit_cast(uint32_t, widen1<X_F16>(static_cast<uint16_t>(amax16))) >> 23;
    constexpr uint32_t inf = XT == X_BF16 ? 0x7F80u : 0x7C00u;
    return amax16 >= inf ? 0xFFu : (e > emax ? e - emax : 0u);
}

// 2^-shared for a scale byte c <= 252 (a normal binary32).  For the NaN
// scale the value is meaningless; those codes are masked.
__device__ __forceinline__ float mx_inv_scale(uint32_t c) { return __builtin_bit_cast(float, (254u - c) << 23); }

// Codes of eight scaled values (|t| < 2^(emax + 1)).  fp8: two words, element
// 0 in the lowest byte.  fp4: one word (.x), element 0 in the lowest nibble.
template <int ELEM>
__device__ __forceinline__ uint2 mx_codes8(const float (&t)[8])
{
    uint2 r;
    if constexpr (ELEM == MX_E2M1) {
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[0], t[1], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[2], t[3], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[4], t[5], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, t[6], t[7], 1.0f, 3);
        r.x = w;
        r.y = 0;
    } else {
        constexpr float m = MxFmt<ELEM>::maxv;
        float c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            c[i] = __builtin_amdgcn_fmed3f(t[i], -m, m);
        if constexpr (ELEM == MX_E4M3) {
            r.x = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
            r.x = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], r.x, true);
            r.y = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
            r.y = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], r.y, true);
        } else {
            r.x = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
            r.x = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], r.x, true);
            r.y = __builtin_amdgcn_cvt_pk_bf8_f32(c[4], c[5], 0, false);
            r.y = __builtin_amdgcn_cvt_pk_bf8_f32(c[6], c[7], r.y, true);
        }
    }
    return r;
}

// Code of one scaled value, in the low 8 (fp8) or 4 (fp4) bits.
template <int ELEM>
__device__ __forceinline__ uint32_t mx_code1(float t)
{
    if constexpr (ELEM == MX_E2M1) {
        return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t, t, 1.0f, 0) & 0xFu;
    } else {
        constexpr float m = MxFmt<ELEM>::maxv;
        const float c = __builtin_amdgcn_fmed3f(t, -m, m);
        if constexpr (ELEM == MX_E4M3)
            return __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
        else
            return __builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xFFu;
    }
}

__device__ __forceinline__ uint32_t quad_max(uint32_t m)
{
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), kDppQuadXor1, 0xF, 0xF, false)));
    m = max(m, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), kDppQuadXor2, 0xF, 0xF, false)));
    return m;
}

// ---------------------------------------------------------------------------
// Axis 1, vectors.  Units are the blocks of a chunk of rows, in row-major
// order; unit u is (row u / nblk, block u % nblk) and its scale byte sits at
// scale[u].  Lane (quad q, part p) of a wave holds, in vector slot v, part p
// of unit base + 16v + q.
// ---------------------------------------------------------------------------
struct MxRowArgs {
    const uint16_t* x;
    uint8_t* y;
    uint8_t* scale;
    uint32_t units;  // blocks in this chunk, <= 2^31 - 1
    uint32_t nblk;   // blocks per row
    uint32_t nvec;   // 16-byte vectors per row (n / 8)
    int64_t n;
    DivMagic by_nblk;
};

template <int XT, int ELEM, bool FLAT>
__global__ __launch_bounds__(kBlock) void mx_row_kernel(const MxRowArgs a)
{
    constexpr int V = kMxRowVecs;
    const uint32_t lane = threadIdx.x & (kWave - 1), part = lane & 3u, quad = lane >> 2;
    const uint32_t base = (blockIdx.x * (kBlock / kWave) + (threadIdx.x / kWave)) * (V * 16u);

    // Every load first, from clamped units (a clamped quad repeats the last
    // block and stores identical bytes).  In a short last block the lanes
    // past the row's end read the block's first vector and count as empty.
    uint4 raw[V];
    int64_t off[V];
    bool valid[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        uint32_t u = base + v * 16u + quad;
        u = u < a.units ? u : a.units - 1;
        if constexpr (FLAT) {
            off[v] = static_cast<int64_t>(u) * kMxBlock + part * 8;
            valid[v] = true;
        } else {
            const uint32_t row = div_by(u, a.by_nblk), j = u - row * a.nblk;
            const uint32_t k = j * 4 + part;
            valid[v] = k < a.nvec;
            off[v] = static_cast<int64_t>(row) * a.n + static_cast<int64_t>(valid[v] ? k : j * 4) * 8;
        }
        raw[v] = ld_stream16(a.x + off[v]);
    }

    uint32_t sbyte[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        uint32_t m = max_u16x2(max_u16x2(abs2(raw[v].x), abs2(raw[v].y)), max_u16x2(abs2(raw[v].z), abs2(raw[v].w)));
        m = max(m & 0xFFFFu, m >> 16);
        if constexpr (!FLAT)
            m = valid[v] ? m : 0u;
        m = quad_max(m);
        const uint32_t c = mx_scale_byte<XT, ELEM>(m);
        sbyte[v] = c;
        const float inv = mx_inv_scale(c);
        float t[8];
        widen8<XT>(raw[v], t);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] *= inv;
        uint2 codes = mx_codes8<ELEM>(t);
        const uint32_t keep = c == 0xFFu ? 0u : ~0u;
        codes.x &= keep;
        codes.y &= keep;
        if (FLAT || valid[v]) {
            // fp4: a plain 4-byte store (measured 2.5% faster than a
            // non-temporal one on bf16 [8192, 7168]).
            if constexpr (ELEM == MX_E2M1)
                *reinterpret_cast<uint32_t*>(a.y + off[v] / 2) = codes.x;
            else
                st_stream8(a.y + off[v], codes);
        }
    }

    // Lane (q, p) stores the scale bytes of slots p, p + 4, ...: each store
    // instruction of the wave covers 64 consecutive units.
    static_assert(V % 4 == 0, "one scale byte per lane per four vector slots");
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
        const uint32_t s = part == 0 ? sbyte[4 * h] : part == 1 ? sbyte[4 * h + 1]
                         : part == 2 ? sbyte[4 * h + 2] : sbyte[4 * h + 3];
        uint32_t u = base + (4 * h + part) * 16u + quad;
        u = u < a.units ? u : a.units - 1;
        __builtin_nontemporal_store(static_cast<uint8_t>(s), a.scale + u);
    }
}

// ---------------------------------------------------------------------------
// Axis 0, vectors.  A workgroup holds 64 adjacent column vectors (8 columns
// each) of one 32-row block; wave w holds rows w*R .. w*R + R - 1, so every
// load and store of a wave covers 1 KB (or its code bytes) of one row.  The
// waves combine their per-column maxima through LDS.  Rows past the end
// repeat the last row: the maximum is unchanged and the stores repeat
// identical bytes.
// ---------------------------------------------------------------------------
struct MxColArgs {
    const uint16_t* x;
    uint8_t* y;
    uint8_t* scale;
    int64_t rows;  // in this chunk
    int64_t n;
    uint32_t nvec;
};

template <int XT, int ELEM, int R>
__global__ __launch_bounds__(kMxBlock / R * kWave) void mx_col_kernel(const MxColArgs a)
{
    constexpr int W = kMxBlock / R;  // waves per workgroup
    __shared__ uint32_t part[W][4][kWave];
    const uint32_t lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const uint32_t cv0 = blockIdx.x * kWave + lane;
    const int64_t col = static_cast<int64_t>(cv0 < a.nvec ? cv0 : a.nvec - 1) * 8;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kMxBlock + w * R;
    uint4 raw[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t r = r0 + k < a.rows ? r0 + k : a.rows - 1;
        raw[k] = ld_stream16(a.x + r * a.n + col);
    }
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < R; ++k) {
        acc[0] = max_u16x2(acc[0], abs2(raw[k].x));
        acc[1] = max_u16x2(acc[1], abs2(raw[k].y));
        acc[2] = max_u16x2(acc[2], abs2(raw[k].z));
        acc[3] = max_u16x2(acc[3], abs2(raw[k].w));
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
        part[w][d][lane] = acc[d];
    __syncthreads();
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        acc[d] = part[0][d][lane];
#pragma unroll
        for (int q = 1; q < W; ++q)
            acc[d] = max_u16x2(acc[d], part[q][d][lane]);
    }
    uint32_t c[8];
    float inv[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        c[2 * d] = mx_scale_byte<XT, ELEM>(acc[d] & 0xFFFFu);
        c[2 * d + 1] = mx_scale_byte<XT, ELEM>(acc[d] >> 16);
    }
    uint2 keep;
    if constexpr (ELEM == MX_E2M1) {
        keep.x = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            keep.x |= (c[i] == 0xFFu ? 0u : 0xFu) << (4 * i);
        keep.y = 0;
    } else {
        keep.x = keep.y = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            keep.x |= (c[i] == 0xFFu ? 0u : 0xFFu) << (8 * i);
            keep.y |= (c[i + 4] == 0xFFu ? 0u : 0xFFu) << (8 * i);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        inv[i] = mx_inv_scale(c[i]);
    if (w == 0) {
        const uint2 sb = make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                                    c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
        st_stream8(a.scale + static_cast<int64_t>(blockIdx.y) * a.n + col, sb);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int64_t r = r0 + k < a.rows ? r0 + k : a.rows - 1;
        float t[8];
        widen8<XT>(raw[k], t);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] *= inv[i];
        uint2 codes = mx_codes8<ELEM>(t);
        codes.x &= keep.x;
        codes.y &= keep.y;
        if constexpr (ELEM == MX_E2M1)
            st_stream4(a.y + (r * a.n + col) / 2, codes.x);
        else
            st_stream8(a.y + r * a.n + col, codes);
    }
}

// ---------------------------------------------------------------------------
// Any shape and alignment.  Axis 1: thread u is block (u / nblk, u % nblk).
// Axis 0: thread u is (block row u / ncp, column pair u % ncp), so one thread
// writes both nibbles of an fp4 byte.
// ---------------------------------------------------------------------------
struct MxGenArgs {
    const uint16_t* x;
    uint8_t* y;
    uint8_t* scale;
    int64_t rows, n;
    int64_t nblk;   // axis 1: blocks per row; axis 0: blocks per column
    int64_t ncp;    // axis 0: column pairs, ceil(n / 2)
    int64_t units;  // threads with work
    int axis;
};

template <int XT, int ELEM>
__device__ void mx_generic_column(const MxGenArgs& a, int64_t jb, int64_t col, uint32_t* c, float* inv)
{
    const int64_t r0 = jb * kMxBlock, len = a.rows - r0 < kMxBlock ? a.rows - r0 : kMxBlock;
    uint32_t m = 0;
    for (int64_t k = 0; k < len; ++k)
        m = max(m, static_cast<uint32_t>(a.x[(r0 + k) * a.n + col] & 0x7FFFu));
    *c = mx_scale_byte<XT, ELEM>(m);
    *inv = mx_inv_scale(*c);
    a.scale[jb * a.n + col] = static_cast<uint8_t>(*c);
}

template <int XT, int ELEM>
__global__ __launch_bounds__(kBlock) void mx_generic_kernel(const MxGenArgs a)
{
    const int64_t u = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (u >= a.units)
        return;
    if (a.axis == 1) {
        const int64_t row = u / a.nblk, j = u - row * a.nblk;
        const int64_t c0 = j * kMxBlock, len = a.n - c0 < kMxBlock ? a.n - c0 : kMxBlock;
        const uint16_t* xr = a.x + row * a.n + c0;
        uint32_t m = 0;
        for (int64_t k = 0; k < len; ++k)
            m = max(m, static_cast<uint32_t>(xr[k] & 0x7FFFu));
        const uint32_t c = mx_scale_byte<XT, ELEM>(m);
        const float inv = mx_inv_scale(c);
        const uint32_t keep = c == 0xFFu ? 0u : 0xFFu;
        a.scale[u] = static_cast<uint8_t>(c);
        if constexpr (ELEM == MX_E2M1) {
            // c0 and n are even, so the block owns whole bytes.
            for (int64_t k = 0; k < len; k += 2) {
                const uint32_t lo = mx_code1<ELEM>(widen1<XT>(xr[k]) * inv);
                const uint32_t hi = mx_code1<ELEM>(widen1<XT>(xr[k + 1]) * inv);
                a.y[(row * a.n + c0 + k) / 2] = static_cast<uint8_t>((lo | hi << 4) & keep);
            }
        } else {
            for (int64_t k = 0; k < len; ++k)
                a.y[row * a.n + c0 + k] = static_cast<uint8_t>(mx_code1<ELEM>(widen1<XT>(xr[k]) * inv) & keep);
        }
    } else {
        const int64_t jb = u / a.ncp, cp = u - jb * a.ncp;
        const int64_t col0 = 2 * cp;
        const bool two = col0 + 1 < a.n;
        uint32_t c_lo = 0, c_hi = 0;
        float inv_lo = 0.0f, inv_hi = 0.0f;
        mx_generic_column<XT, ELEM>(a, jb, col0, &c_lo, &inv_lo);
        if (two)
            mx_generic_column<XT, ELEM>(a, jb, col0 + 1, &c_hi, &inv_hi);
        const uint32_t keep_lo = c_lo == 0xFFu ? 0u : 0xFFu, keep_hi = c_hi == 0xFFu ? 0u : 0xFFu;
        const int64_t r0 = jb * kMxBlock, len = a.rows - r0 < kMxBlock ? a.rows - r0 : kMxBlock;
        for (int64_t k = 0; k < len; ++k) {
            const int64_t r = r0 + k;
            const uint32_t lo = mx_code1<ELEM>(widen1<XT>(a.x[r * a.n + col0]) * inv_lo) & keep_lo;
            if constexpr (ELEM == MX_E2M1) {
                // fp4 needs an even n, so the pair is whole.
                const uint32_t hi = mx_code1<ELEM>(widen1<XT>(a.x[r * a.n + col0 + 1]) * inv_hi) & keep_hi;
                a.y[(r * a.n + col0) / 2] = static_cast<uint8_t>(lo | hi << 4);
            } else {
                a.y[r * a.n + col0] = static_cast<uint8_t>(lo);
                if (two)
                    a.y[r * a.n + col0 + 1] =
                        static_cast<uint8_t>(mx_code1<ELEM>(widen1<XT>(a.x[r * a.n + col0 + 1]) * inv_hi) & keep_hi);
            }
        }
    }
}

template <int XT, int ELEM>
hipError_t launch_typed(const MxPlan& p, hipStream_t stream)
{
    const uint16_t* x = static_cast<const uint16_t*>(p.x);
    uint8_t* y = static_cast<uint8_t*>(p.y);
    // Code bytes per element, times 2.
    const int64_t cb2 = ELEM == MX_E2M1 ? 1 : 2;
    if (p.variant == MX_VAR_ROW) {
        const int64_t nblk = (p.n + kMxBlock - 1) / kMxBlock;
        const int64_t per_block = static_cast<int64_t>(kBlock / kWave) * kMxRowVecs * 16;  // units per workgroup
        const int64_t rows_per_chunk = kMaxGridBlocks / nblk;  // units stay below 2^31
        const bool flat = p.n % kMxBlock == 0;
        for (int64_t r0 = 0; r0 < p.rows; r0 += rows_per_chunk) {
            const int64_t rc = p.rows - r0 < rows_per_chunk ? p.rows - r0 : rows_per_chunk;
            MxRowArgs a;
            a.x = x + r0 * p.n;
            a.y = y + r0 * p.n * cb2 / 2;
            a.scale = p.scale + r0 * nblk;
            a.units = static_cast<uint32_t>(rc * nblk);
            a.nblk = static_cast<uint32_t>(nblk);
            a.nvec = static_cast<uint32_t>(p.n / 8);
            a.n = p.n;
            a.by_nblk = div_magic(static_cast<uint64_t>(nblk));
            const int64_t blocks = (static_cast<int64_t>(a.units) + per_block - 1) / per_block;
            if (flat)
                hipLaunchKernelGGL((mx_row_kernel<XT, ELEM, true>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock),
                                   0, stream, a);
            else
                hipLaunchKernelGGL((mx_row_kernel<XT, ELEM, false>), dim3(static_cast<uint32_t>(blocks)),
                                   dim3(kBlock), 0, stream, a);
            const hipError_t err = hipGetLastError();
            if (err != hipSuccess)
                return err;
        }
        return hipSuccess;
    }
    if (p.variant == MX_VAR_COL) {
        const int64_t nvec = p.n / 8;
        const int64_t per_block = kWave;  // column vectors per workgroup
        const int64_t gx = (nvec + per_block - 1) / per_block;
        const int64_t nbr = (p.rows + kMxBlock - 1) / kMxBlock;
        for (int64_t j0 = 0; j0 < nbr; j0 += kMaxGridY) {
            const int64_t jc = nbr - j0 < kMaxGridY ? nbr - j0 : kMaxGridY;
            const int64_t r0 = j0 * kMxBlock;
            MxColArgs a;
            a.x = x + r0 * p.n;
            a.y = y + r0 * p.n * cb2 / 2;
            a.scale = p.scale + j0 * p.n;
            a.rows = p.rows - r0 < jc * kMxBlock ? p.rows - r0 : jc * kMxBlock;
            a.n = p.n;
            a.nvec = static_cast<uint32_t>(nvec);
            hipLaunchKernelGGL((mx_col_kernel<XT, ELEM, kMxColRows>), dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(jc)),
                               dim3(kMxBlock / kMxColRows * kWave), 0, stream, a);
            const hipError_t err = hipGetLastError();
            if (err != hipSuccess)
                return err;
        }
        return hipSuccess;
    }
    MxGenArgs a;
    a.x = x;
    a.y = y;
    a.scale = p.scale;
    a.rows = p.rows;
    a.n = p.n;
    a.axis = p.axis;
    if (p.axis == 1) {
        a.nblk = (p.n + kMxBlock - 1) / kMxBlock;
        a.ncp = 0;
        a.units = p.rows * a.nblk;
    } else {
        a.nblk = (p.rows + kMxBlock - 1) / kMxBlock;
        a.ncp = (p.n + 1) / 2;
        a.units = a.nblk * a.ncp;
    }
    const int64_t blocks = (a.units + kBlock - 1) / kBlock;
    if (blocks > kMaxGridBlocks)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((mx_generic_kernel<XT, ELEM>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

template <int XT>
hipError_t launch_elem(const MxPlan& p, hipStream_t stream)
{
    switch (p.elem) {
    case MX_E4M3: return launch_typed<XT, MX_E4M3>(p, stream);
    case MX_E5M2: return launch_typed<XT, MX_E5M2>(p, stream);
    default: return launch_typed<XT, MX_E2M1>(p, stream);
    }
}

}  // namespace

hipError_t launch_mx_quantize(const MxPlan& p, hipStream_t stream)
{
    if (p.rows == 0 || p.n == 0)
        return hipSuccess;
    return p.x_type == X_BF16 ? launch_elem<X_BF16>(p, stream) : launch_elem<X_F16>(p, stream);
}

}  // namespace dq
