/*
 * dquant_oracle.c -- plain, slow, single-threaded CPU oracle for per-token
 * dynamic quantization, its AdaLayerNorm fusion, AntiQuantize, mx block
 * quantization and the weight-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: it is used by tests/, by the smoke check and by the CPU
 * baseline leg of bench.py.  It shares no code, header, table or constant
 * with the HIP library; its element conversions (bf16, fp16, fp8-e4m3fn,
 * fp8-e5m2, fp4-e2m1, e8m0) are written here from the format definitions.
 *
 * Arithmetic rules (built with -O2 -ffp-contract=off -fno-fast-math, SSE
 * scalar float on x86-64, so FLT_EVAL_METHOD == 0):
 *   - every fp32 step is one IEEE-754 binary32 operation rounded to nearest
 *     even; nothing is fused, nothing is flushed to zero;
 *   - "round" in the formulas is round-half-to-even (nearbyintf under the
 *     default FE_TONEAREST mode);
 *   - a code that leaves the output range saturates to the range; NaN -> 0.
 *
 * Sources (the pages' titles and sections):
 *   [DQ]   aclnnDynamicQuantV2, "Description"/"Formula" (symmetric and
 *          asymmetric, with and without smoothScalesOptional; scale_opt /
 *          offset_opt per output type) and its constraints section (INT4:
 *          last dim even; INT32: last dim divisible by 8).
 *   [ADA]  aclnnAdaLayerNormQuant, "Formula" steps 1-5.
 *   [AQ]   AntiQuantize (Ascend C API), 功能说明 (function description:
 *          PER_TENSOR / PER_CHANNEL / PER_TOKEN / PER_GROUP shapes, kDim),
 *          表1 (AntiQuantizeConfig), 表2 (AntiQuantizeParams), 表3 (dtype
 *          combinations), 调用示例 (the worked example).
 *   [MX]   aclnnQuantBatchMatmulInplaceAdd, 计算公式 (mx量化: blocks of
 *          gsK = 32 along K, FLOAT8_E8M0 block scales), the consumer whose
 *          operands the mx block quantizer produces.
 *   [WQ]   aclnnWeightQuantMatmulAllReduce, API function and constraints
 *          (x2 fake-quantized per tensor / channel / group, then the
 *          matmul; parameter shapes; the empty-k case).
 *
 * Readings taken where the pages are silent or garbled are stated next to
 * the step that depends on them.
 *
 * Pinning: every function here is checked by tests/oracle_pins.py against
 * values fixed independently of this file (hand-worked rows, the pages'
 * worked example, closed forms, invariants, and numpy float32 / torch
 * evaluations of each formula), and tests/test_oracle_mutants.py shows that
 * planted mistakes fail those checks.  What no page value fixes is the sign
 * convention of the AntiQuantize offset: that is a reading (stated at
 * oracle_antiquantize), and its parity is unpinned by the pages.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element type codes of this oracle (its own numbering). */
enum {
    ORC_F32 = 0,
    ORC_F16 = 1,
    ORC_BF16 = 2,
    ORC_I8 = 3,
    ORC_I4 = 4,
    ORC_I32 = 5,
    ORC_F8E4M3 = 6,
    ORC_F64 = 7,
    ORC_F8E5M2 = 8,
    ORC_F4E2M1 = 9, /* two codes per byte, element 2k in the low nibble */
    ORC_E8M0 = 10
};

/* ------------------------------------------------------------------------ */
/* Element conversions, from the format definitions.                         */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_to_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* bfloat16 is the upper half of a binary32: widening appends 16 zero bits. */
float orc_bf16_to_f32(uint16_t h)
{
    return bits_to_f32((uint32_t)h << 16);
}

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        if (f != 0)
            return nanf("");
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return (float)(sign ? -v : v); /* exact: every binary16 is a binary32 */
}

/* OCP fp8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits, no
 * infinities; exponent 15 with fraction 7 is NaN; largest finite 448. */
float orc_e4m3fn_to_f32(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int f = b & 7;
    double v;
    if (e == 15 && f == 7)
        return nanf("");
    if (e == 0)
        v = ldexp((double)f, -9); /* (f/8) * 2^-6 */
    else
        v = ldexp((double)(8 + f), e - 10); /* (1 + f/8) * 2^(e-7) */
    return (float)(sign ? -v : v);
}

/* OCP fp8 E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits, IEEE-style
 * infinities (exponent 31, fraction 0) and NaNs (exponent 31, fraction
 * nonzero); largest finite 57344. */
float orc_e5m2_to_f32(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 2) & 0x1F;
    int f = b & 3;
    double v;
    if (e == 31)
        return f ? nanf("") : (sign ? -INFINITY : INFINITY);
    if (e == 0)
        v = ldexp((double)f, -16); /* (f/4) * 2^-14 */
    else
        v = ldexp((double)(4 + f), e - 17); /* (1 + f/4) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* OCP MX fp4 E2M1: 1 sign, 2 exponent (bias 1), 1 fraction bit, no
 * infinities or NaNs; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
float orc_e2m1_to_f32(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int f = nibble & 1;
    double v;
    if (e == 0)
        v = 0.5 * f; /* subnormal: (f/2) * 2^(1-1) */
    else
        v = ldexp((double)(2 + f), e - 2); /* (1 + f/2) * 2^(e-1) */
    return (float)(sign ? -v : v);
}

/* OCP MX E8M0 scale: an unsigned biased exponent, value 2^(b - 127); 0xFF
 * is NaN. */
float orc_e8m0_to_f32(uint8_t b)
{
    if (b == 0xFF)
        return nanf("");
    return (float)ldexp(1.0, (int)b - 127);
}

/* Round a binary32 to bfloat16, nearest-even.  Works on the bit pattern:
 * the kept upper 16 bits are incremented when the dropped lower 16 bits are
 * above half, or exactly half and the kept part is odd. */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u = f32_to_bits(x);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040); /* keep sign, force quiet */
    uint32_t upper = u >> 16;
    uint32_t lower = u & 0xFFFFu;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* a carry into the exponent is the correct result */
    return (uint16_t)upper;
}

/* Round a binary32 to binary16, nearest-even, from the definition: find
 * the quantum of the target binade, divide (exactly, by a power of two),
 * round the quotient to an integer with ties to even, rebuild the bits. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00);
    double a = fabs((double)x);
    if (isinf(x) || a >= 65520.0) /* 65520 is the tie between 65504 and 2^16 */
        return (uint16_t)(sign | 0x7C00);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);     /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;    /* a in [2^E, 2^(E+1)) */
    if (E < -14) {    /* subnormal range: quantum 2^-24 */
        double q = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the smallest normal */
    }
    double q = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E + 15 >= 31)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

static float load_as_f32(const void* p, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32:
        return ((const float*)p)[i];
    case ORC_F16:
        return orc_f16_to_f32(((const uint16_t*)p)[i]);
    case ORC_BF16:
        return orc_bf16_to_f32(((const uint16_t*)p)[i]);
    case ORC_I8:
        return (float)((const int8_t*)p)[i];
    case ORC_F8E4M3:
        return orc_e4m3fn_to_f32(((const uint8_t*)p)[i]);
    case ORC_F8E5M2:
        return orc_e5m2_to_f32(((const uint8_t*)p)[i]);
    case ORC_F4E2M1: {
        uint8_t byte = ((const uint8_t*)p)[i / 2];
        return orc_e2m1_to_f32((uint8_t)((i & 1) ? byte >> 4 : byte & 0xF));
    }
    case ORC_E8M0:
        return orc_e8m0_to_f32(((const uint8_t*)p)[i]);
    default:
        return nanf("");
    }
}

/* Vector forms of the conversions, for tests that pin them against library
 * routines. */
void orc_convert_to_f32(const void* src, int src_dtype, int64_t count, float* dst)
{
    for (int64_t i = 0; i < count; ++i)
        dst[i] = load_as_f32(src, src_dtype, i);
}

void orc_convert_from_f32(const float* src, int64_t count, int dst_dtype, uint16_t* dst)
{
    for (int64_t i = 0; i < count; ++i)
        dst[i] = dst_dtype == ORC_BF16 ? orc_f32_to_bf16(src[i]) : orc_f32_to_f16(src[i]);
}

/* ------------------------------------------------------------------------ */
/* Saturating round-half-to-even.                                            */
/* ------------------------------------------------------------------------ */

/* sat(rne(t)): NaN -> 0; otherwise round to the nearest integer with ties
 * to even, then clamp to [lo, hi] (so +inf -> hi and -inf -> lo). */
static int sat_rne(float t, int lo, int hi)
{
    if (isnan(t))
        return 0;
    float r = nearbyintf(t);
    if (r < (float)lo)
        return lo;
    if (r > (float)hi)
        return hi;
    return (int)r;
}

/* ------------------------------------------------------------------------ */
/* [DQ] aclnnDynamicQuantV2                                                  */
/* ------------------------------------------------------------------------ */

/* The expert that owns row r.  groupIndexOptional tells the experts apart
 * (Description).  Reading: it holds cumulative per-expert row ends, so
 * expert e owns rows [gi[e-1], gi[e]); the owner is the first e with
 * r < gi[e]; a row past the last end belongs to the last expert. */
static int64_t expert_of_row(int64_t r, const int32_t* gi, int64_t n_experts)
{
    for (int64_t e = 0; e < n_experts; ++e)
        if (r < (int64_t)gi[e])
            return e;
    return n_experts - 1;
}

/*
 * Per-row dynamic quantization (Formula, all four cases).
 *
 *   x          [rows, n] of x_dtype (F16 or BF16), row-major.
 *   smooth     NULL (no smoothScalesOptional), or fp32 [n] when
 *              group_index is NULL, or fp32 [n_experts, n] with group_index.
 *   group_index int32 [n_experts] or NULL.
 *   symmetric  1: scale = row_max(|in|) / D, y = round(in / scale).
 *              0: scale = (row_max(in) - row_min(in)) / scale_opt,
 *                 offset = offset_opt - row_max(in) / scale,
 *                 y = round(in / scale + offset).
 *   out_dtype  ORC_I8: (scale_opt, offset_opt) = (255, 127), codes in
 *              [-128, 127]; ORC_I4 / ORC_I32: (15, 7), codes in [-8, 7].
 *              Reading: the symmetric divisor D is offset_opt (127 for
 *              INT8, as printed; 7 for INT4/INT32, whose code range ends
 *              at 7).
 *   y          INT8: one byte per code.  INT4: two codes per byte, the
 *              even-indexed code in the low nibble (reading).  INT32: eight
 *              codes per little-endian word, code 8w+i in bits [4i, 4i+3]
 *              (reading), so the bytes equal the INT4 bytes.
 *   scale      fp32 [rows].  offset: fp32 [rows] (asymmetric only).
 *
 * Each formula step is one binary32 operation, evaluated left to right as
 * printed: scale = RN(RN(max - min) / scale_opt), q = RN(max / scale),
 * offset = RN(offset_opt - q), code = sat(rne(RN(RN(in / scale) + offset))).
 */
void oracle_dynamic_quant(const void* x, int x_dtype, int64_t rows, int64_t n,
                          const float* smooth, const int32_t* group_index,
                          int64_t n_experts, int symmetric, int out_dtype,
                          void* y, float* scale, float* offset)
{
    const float scale_opt = out_dtype == ORC_I8 ? 255.0f : 15.0f;
    const float offset_opt = out_dtype == ORC_I8 ? 127.0f : 7.0f;
    const int code_lo = out_dtype == ORC_I8 ? -128 : -8;
    const int code_hi = out_dtype == ORC_I8 ? 127 : 7;
    float* v = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    int* c = (int*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int));

    for (int64_t r = 0; r < rows; ++r) {
        /* input = x * smoothScalesOptional (element-wise, per expert) */
        const float* s = NULL;
        if (smooth) {
            int64_t e = group_index ? expert_of_row(r, group_index, n_experts) : 0;
            s = smooth + e * n;
        }
        for (int64_t j = 0; j < n; ++j) {
            float xv = load_as_f32(x, x_dtype, r * n + j);
            v[j] = s ? xv * s[j] : xv;
        }

        if (symmetric) {
            float amax = 0.0f;
            for (int64_t j = 0; j < n; ++j) {
                float a = fabsf(v[j]);
                if (a > amax)
                    amax = a;
            }
            float sc = amax / offset_opt;
            for (int64_t j = 0; j < n; ++j)
                c[j] = sat_rne(v[j] / sc, code_lo, code_hi);
            scale[r] = sc;
        } else {
            float hi = v[0], lo = v[0];
            for (int64_t j = 1; j < n; ++j) {
                if (v[j] > hi)
                    hi = v[j];
                if (v[j] < lo)
                    lo = v[j];
            }
            float range = hi - lo;
            float sc = range / scale_opt;
            float q_hi = hi / sc;
            float off = offset_opt - q_hi;
            for (int64_t j = 0; j < n; ++j) {
                float q = v[j] / sc;
                float t = q + off;
                c[j] = sat_rne(t, code_lo, code_hi);
            }
            scale[r] = sc;
            offset[r] = off;
        }

        if (out_dtype == ORC_I8) {
            int8_t* yr = (int8_t*)y + r * n;
            for (int64_t j = 0; j < n; ++j)
                yr[j] = (int8_t)c[j];
        } else if (out_dtype == ORC_I4) {
            uint8_t* yr = (uint8_t*)y + r * (n / 2);
            for (int64_t k = 0; k < n / 2; ++k)
                yr[k] = (uint8_t)((c[2 * k] & 0xF) | ((c[2 * k + 1] & 0xF) << 4));
        } else { /* ORC_I32 */
            uint32_t* yr = (uint32_t*)y + r * (n / 8);
            for (int64_t w = 0; w < n / 8; ++w) {
                uint32_t word = 0;
                for (int i = 0; i < 8; ++i)
                    word |= (uint32_t)(c[8 * w + i] & 0xF) << (4 * i);
                yr[w] = word;
            }
        }
    }
    free(v);
    free(c);
}

/* ------------------------------------------------------------------------ */
/* [ADA] aclnnAdaLayerNormQuant                                              */
/* ------------------------------------------------------------------------ */

/*
 * Formula steps 1-3, the plain definition, in binary64.
 *
 *   x       [B, S, H] of x_dtype; rows are (b, s) pairs, b = row / S.
 *   scale, shift: [B, H] of their dtype (a [B, 1, H] tensor has the same
 *           memory), broadcast over S.
 *   weight, bias: [H] or NULL (reading: absent weight is 1, absent bias 0).
 *   smooth  [H] or NULL (step 3 is skipped when absent).
 *   y       binary64 [B*S*H] out.
 *
 *   LayerNorm(x) = (x - E(x)) / sqrt(Var(x) + eps) * weight + bias
 *   y = LayerNorm(x) * (1 + scale) + shift;  y = y * smooth.
 * Reading: Var is the biased (divide by H) variance, as in LayerNorm; E and
 * Var are taken with the two-pass definition.
 */
void oracle_ada_layernorm_modulate(const void* x, int x_dtype, int64_t B, int64_t S, int64_t H,
                                   const void* scale, int scale_dtype,
                                   const void* shift, int shift_dtype,
                                   const void* weight, int weight_dtype,
                                   const void* bias, int bias_dtype,
                                   const void* smooth, int smooth_dtype,
                                   double eps, double* y)
{
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t s = 0; s < S; ++s) {
            int64_t row = b * S + s;
            double sum = 0.0;
            for (int64_t j = 0; j < H; ++j)
                sum += (double)load_as_f32(x, x_dtype, row * H + j);
            double mean = sum / (double)H;
            double ss = 0.0;
            for (int64_t j = 0; j < H; ++j) {
                double d = (double)load_as_f32(x, x_dtype, row * H + j) - mean;
                ss += d * d;
            }
            double var = ss / (double)H;
            double rstd = 1.0 / sqrt(var + eps);
            for (int64_t j = 0; j < H; ++j) {
                double xv = (double)load_as_f32(x, x_dtype, row * H + j);
                double w = weight ? (double)load_as_f32(weight, weight_dtype, j) : 1.0;
                double bb = bias ? (double)load_as_f32(bias, bias_dtype, j) : 0.0;
                double ln = (xv - mean) * rstd * w + bb;
                double sc = (double)load_as_f32(scale, scale_dtype, b * H + j);
                double sh = (double)load_as_f32(shift, shift_dtype, b * H + j);
                double yv = ln * (1.0 + sc) + sh;
                if (smooth)
                    yv = yv * (double)load_as_f32(smooth, smooth_dtype, j);
                y[row * H + j] = yv;
            }
        }
    }
}

/*
 * Formula steps 4-5 on top of steps 1-3:
 *   quantScale = row_max(|y|) / 127;  out = round(y / quantScale).
 * The pages fix no precision.  Reading: the quantization decision is taken
 * in binary32, the precision the device computes in: y is rounded once to
 * binary32, then quantScale = RN(max|y32| / 127) and
 * out = sat(rne(RN(y32 / quantScale))) in [-128, 127], as in the symmetric
 * INT8 DynamicQuant step.  y is returned through y64 (may be NULL).
 */
void oracle_ada_layernorm_quant(const void* x, int x_dtype, int64_t B, int64_t S, int64_t H,
                                const void* scale, int scale_dtype,
                                const void* shift, int shift_dtype,
                                const void* weight, int weight_dtype,
                                const void* bias, int bias_dtype,
                                const void* smooth, int smooth_dtype,
                                double eps, int8_t* out, float* quant_scale, double* y64)
{
    int64_t total = B * S * H;
    double* y = y64 ? y64 : (double*)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
    oracle_ada_layernorm_modulate(x, x_dtype, B, S, H, scale, scale_dtype, shift, shift_dtype,
                                  weight, weight_dtype, bias, bias_dtype, smooth, smooth_dtype,
                                  eps, y);
    for (int64_t row = 0; row < B * S; ++row) {
        const double* yr = y + row * H;
        float amax = 0.0f;
        for (int64_t j = 0; j < H; ++j) {
            float a = fabsf((float)yr[j]);
            if (a > amax)
                amax = a;
        }
        float qs = amax / 127.0f;
        for (int64_t j = 0; j < H; ++j)
            out[row * H + j] = (int8_t)sat_rne((float)yr[j] / qs, -128, 127);
        quant_scale[row] = qs;
    }
    if (!y64)
        free(y);
}

/* ------------------------------------------------------------------------ */
/* [AQ] AntiQuantize                                                         */
/* ------------------------------------------------------------------------ */

enum { ORC_PER_TENSOR = 0, ORC_PER_CHANNEL = 1, ORC_PER_TOKEN = 2, ORC_PER_GROUP = 3 };

/*
 * Element-wise fake-quantization (dequantization) of src [m, n] into
 * dst [m, n] (功能说明).  The parameter that element (i, j) uses depends on
 * the policy (表1 AntiQuantizeConfig.policy, .kDim):
 *   PER_TENSOR  scale/offset shape [1]          -> index 0
 *   PER_CHANNEL shape [1, n]                    -> index j
 *   PER_TOKEN   shape [m, 1]                    -> index i
 *   PER_GROUP   kDim = 1 (groups along n): shape [m, ceil(n/gs)] -> (i, j / gs)
 *               kDim = 0 (groups along m): shape [ceil(m/gs), n] -> (i / gs, j)
 * A last group that is shorter than groupSize uses its own parameter (the
 * shapes round the group count up).
 *
 * The formula after "the formulas are as follows" is missing from the page.
 * Reading: scale is the scaling factor and offset the offset applied to the
 * quantized input (表2), so dst = (src + offset) * scale, as two binary32
 * operations, RN(RN(v + o) * s); without offset (hasOffset = false)
 * dst = RN(v * s).  The binary32 result is rounded once to dst's type
 * (bf16 or fp16, nearest-even; F32 keeps it).
 *
 * src_dtype ORC_I8, ORC_F8E4M3 or ORC_F8E5M2 (the b8 cases of 表3);
 * scale/offset F32, F16 or BF16 (widened exactly); offset may be NULL.
 *
 * The float4 case of 表3 (PER_GROUP, fp4x2 source, fp8_e8m0 scale, no
 * offset -- 约束说明): src_dtype ORC_F4E2M1 (two codes per byte, element
 * 2k in the low nibble; n even), scale_dtype ORC_E8M0, offset NULL.  Its
 * formula is missing from the page too; reading: the e8m0 scale is the
 * power of two 2^(e - 127) that multiplies the decoded element, so
 * dst = RN(decode(src) * 2^(e - 127)) -- exact in binary32 except where it
 * overflows to infinity -- then rounded once to dst's type.  The same code
 * path computes it: v and s are the decoded values, t = RN(v * s).
 */
void oracle_antiquantize(const void* src, int src_dtype, int64_t m, int64_t n,
                         const void* scale, int scale_dtype,
                         const void* offset, int offset_dtype,
                         int policy, int kdim, int64_t group_size,
                         int dst_dtype, void* dst)
{
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            int64_t p;
            if (policy == ORC_PER_TENSOR)
                p = 0;
            else if (policy == ORC_PER_CHANNEL)
                p = j;
            else if (policy == ORC_PER_TOKEN)
                p = i;
            else if (kdim == 1)
                p = i * ((n + group_size - 1) / group_size) + j / group_size;
            else
                p = (i / group_size) * n + j;

            float v = load_as_f32(src, src_dtype, i * n + j);
            float s = load_as_f32(scale, scale_dtype, p);
            float t;
            if (offset) {
                float o = load_as_f32(offset, offset_dtype, p);
                float u = v + o;
                t = u * s;
            } else {
                t = v * s;
            }
            if (dst_dtype == ORC_F32)
                ((float*)dst)[i * n + j] = t;
            else if (dst_dtype == ORC_BF16)
                ((uint16_t*)dst)[i * n + j] = orc_f32_to_bf16(t);
            else
                ((uint16_t*)dst)[i * n + j] = orc_f32_to_f16(t);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* [MX] mx block quantization (producer of the mx operands)                  */
/* ------------------------------------------------------------------------ */

/* Parameters of an OCP element format: width in bits, fraction bits,
 * exponent bias, the largest finite magnitude, and emax = floor(log2(largest
 * finite)). */
struct orc_elem_fmt {
    int bits;
    int mbits;
    int bias;
    double maxv;
    int emax;
};

static struct orc_elem_fmt orc_fmt_of(int dtype)
{
    struct orc_elem_fmt f;
    if (dtype == ORC_F8E4M3) {
        f.bits = 8; f.mbits = 3; f.bias = 7; f.maxv = 448.0; f.emax = 8;     /* 1.75 * 2^8 */
    } else if (dtype == ORC_F8E5M2) {
        f.bits = 8; f.mbits = 2; f.bias = 15; f.maxv = 57344.0; f.emax = 15; /* 1.75 * 2^15 */
    } else {
        f.bits = 4; f.mbits = 1; f.bias = 1; f.maxv = 6.0; f.emax = 2;       /* 1.5 * 2^2 */
    }
    return f;
}

/* Encode a finite, non-negative magnitude a into the exponent and fraction
 * fields of an element format: nearest representable value with ties to the
 * even fraction, a result beyond the largest finite magnitude saturating to
 * it.  Every step is exact in double (a is a binary32 value scaled by a power
 * of two, and the quanta are powers of two). */
static unsigned orc_encode_magnitude(double a, struct orc_elem_fmt f)
{
    if (a == 0.0)
        return 0;
    int emin = 1 - f.bias; /* exponent of the smallest normal */
    int e;
    frexp(a, &e);
    int E = e - 1; /* a in [2^E, 2^(E+1)) */
    if (E < emin)
        E = emin; /* the subnormals share the smallest normal's quantum */
    double q = nearbyint(ldexp(a, f.mbits - E)); /* a in quanta of 2^(E - mbits) */
    double v = ldexp(q, E - f.mbits);            /* the rounded value */
    if (v > f.maxv)
        v = f.maxv;
    if (v < ldexp(1.0, emin)) /* subnormal (or zero): exponent field 0 */
        return (unsigned)ldexp(v, f.mbits - emin);
    frexp(v, &e);
    E = e - 1;
    unsigned frac = (unsigned)(ldexp(v, f.mbits - E) - ldexp(1.0, f.mbits));
    return ((unsigned)(E + f.bias) << f.mbits) | frac;
}

static void orc_store_code(void* y, int elem_dtype, int64_t i, unsigned code)
{
    if (elem_dtype == ORC_F4E2M1) {
        uint8_t* b = (uint8_t*)y + i / 2;
        if (i & 1)
            *b = (uint8_t)((*b & 0x0F) | (code << 4));
        else
            *b = (uint8_t)((*b & 0xF0) | (code & 0x0F));
    } else {
        ((uint8_t*)y)[i] = (uint8_t)code;
    }
}

/*
 * mx block quantization: the producer of the operands that the mx formula of
 * aclnnQuantBatchMatmulInplaceAdd (计算公式, mx量化) consumes.  That formula
 * multiplies, per block of gsK = 32 consecutive elements along the
 * contraction axis (kLoops = ceil(K / 32) blocks, the last one possibly
 * shorter), the element codes by one FLOAT8_E8M0 scale per block: scale1[m, j]
 * for x1 [M, K], scale2[j, n] for x2 [K, N].  The pages print no producer.
 * Reading (the OCP Microscaling Formats v1.0 conversion, section 6.3): per
 * block,
 *     shared = floor(log2(max |v|)) - emax(element format),
 *              clamped to the e8m0 range [-127, 127];
 *     scale code = shared + 127;
 *     code_i = nearest element value to v_i / 2^shared, ties to even,
 *              saturating at the largest finite element magnitude, the sign
 *              of v_i kept (also on a zero result).
 * An all-zero block has max |v| = 0: floor(log2 0) = -inf clamps to -127
 * (scale code 0) and every code is a zero of v's sign.  A block holding a NaN
 * or an infinity gets the NaN scale 0xFF and all-zero codes (reading: the
 * NaN scale makes the whole block NaN whatever its codes).
 *
 *   x          [rows, n] of x_dtype (F16 or BF16), row-major.
 *   elem_dtype ORC_F8E4M3, ORC_F8E5M2 or ORC_F4E2M1 (n even; two codes per
 *              byte along n, element 2k in the low nibble).
 *   axis       1: blocks run along n (the x1 layout), scale [rows, ceil(n/32)];
 *              0: blocks run along rows (the x2 layout), scale [ceil(rows/32), n].
 *   y          codes, [rows, n] bytes (fp8) or [rows, n/2] bytes (fp4).
 *   scale      e8m0 bytes.
 */
void oracle_mx_quantize(const void* x, int x_dtype, int64_t rows, int64_t n,
                        int elem_dtype, int axis, void* y, uint8_t* scale)
{
    const int64_t gs = 32;
    struct orc_elem_fmt f = orc_fmt_of(elem_dtype);
    /* A block is (outer index o, block index j) and holds elements k = 0..31
     * at (r, c) = axis 1 ? (o, j*32 + k) : (j*32 + k, o). */
    int64_t outer = axis == 1 ? rows : n;
    int64_t along = axis == 1 ? n : rows;
    int64_t blocks = (along + gs - 1) / gs;
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t j = 0; j < blocks; ++j) {
            int64_t len = along - j * gs < gs ? along - j * gs : gs;
            double amax = 0.0;
            int finite = 1;
            for (int64_t k = 0; k < len; ++k) {
                int64_t r = axis == 1 ? o : j * gs + k;
                int64_t c = axis == 1 ? j * gs + k : o;
                float v = load_as_f32(x, x_dtype, r * n + c);
                if (!isfinite(v))
                    finite = 0;
                else if (fabs((double)v) > amax)
                    amax = fabs((double)v);
            }
            int64_t si = axis == 1 ? o * blocks + j : j * n + o;
            int shared = -127;
            if (finite && amax > 0.0) {
                int e;
                frexp(amax, &e);
                shared = (e - 1) - f.emax; /* floor(log2 amax) - emax */
                if (shared < -127)
                    shared = -127;
                if (shared > 127)
                    shared = 127;
            }
            scale[si] = finite ? (uint8_t)(shared + 127) : 0xFF;
            for (int64_t k = 0; k < len; ++k) {
                int64_t r = axis == 1 ? o : j * gs + k;
                int64_t c = axis == 1 ? j * gs + k : o;
                unsigned code = 0;
                if (finite) {
                    double t = ldexp((double)load_as_f32(x, x_dtype, r * n + c), -shared);
                    unsigned sign = signbit(t) ? 1u << (f.bits - 1) : 0u;
                    code = sign | orc_encode_magnitude(fabs(t), f);
                }
                orc_store_code(y, elem_dtype, r * n + c, code);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* [WQ] weight-quantized matmul                                              */
/* ------------------------------------------------------------------------ */

/* Round a double to bfloat16 or binary16, nearest-even, from the definition
 * (the quantum of the target binade; no intermediate binary32 rounding). */
static uint16_t orc_f64_to_half(double x, int dtype)
{
    const int mbits = dtype == ORC_BF16 ? 7 : 10;
    const int ebits = dtype == ORC_BF16 ? 8 : 5;
    const int bias = (1 << (ebits - 1)) - 1;
    uint16_t sign = signbit(x) ? (uint16_t)(1u << 15) : 0;
    uint16_t inf = (uint16_t)(((1u << ebits) - 1) << mbits);
    if (isnan(x))
        return (uint16_t)(sign | inf | (1u << (mbits - 1)));
    double a = fabs(x);
    if (isinf(x))
        return (uint16_t)(sign | inf);
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);
    int E = e - 1;
    int emin = 1 - bias;
    if (E < emin)
        E = emin;
    double q = nearbyint(ldexp(a, mbits - E)); /* quanta of 2^(E - mbits) */
    if (q >= ldexp(1.0, mbits + 1)) {          /* carried into the next binade */
        q = ldexp(q, -1);
        E += 1;
    }
    if (E > bias) /* beyond the largest finite value */
        return (uint16_t)(sign | inf);
    if (q < ldexp(1.0, mbits)) /* subnormal */
        return (uint16_t)(sign | (uint16_t)q);
    return (uint16_t)(sign | (uint16_t)((E + bias) << mbits) | (uint16_t)(q - ldexp(1.0, mbits)));
}

/* Signed weight code x2[kk, nn] of an int8 or int4 weight held as [k, n]
 * (transpose_x2 == 0) or as [n, k] (transpose_x2 != 0).  int4 codes sit two
 * per byte along the stored last dimension, the even element in the low
 * nibble, and are sign-extended from 4 bits. */
static int weight_code(const void* x2, int w_dtype, int transpose_x2, int64_t k, int64_t n,
                       int64_t kk, int64_t nn)
{
    int64_t i = transpose_x2 ? nn * k + kk : kk * n + nn;
    if (w_dtype == ORC_I8)
        return ((const int8_t*)x2)[i];
    uint8_t byte = ((const uint8_t*)x2)[i / 2];
    int v = (i & 1) ? byte >> 4 : byte & 0xF;
    return v >= 8 ? v - 16 : v;
}

/*
 * The fake-quantized weight of aclnnWeightQuantMatmulAllReduce (API
 * function: x2 is fake-quantized, then multiplied), per tensor, per channel
 * or per group down k.  The formula is missing from the page; reading: the
 * AntiQuantize arithmetic with kDim = 0,
 *     W[kk, nn] = RN_T(RN(RN(x2 + offset) * scale))   (offset given)
 *     W[kk, nn] = RN_T(RN(x2 * scale))                 (no offset)
 * in binary32, rounded once to T, the dtype of x1 and the parameters (the
 * constraints make x1, antiquantScale, antiquantOffset, bias, x3 and the
 * output one dtype).  Parameter index by policy (shapes from the
 * constraints): per tensor [1]: 0; per channel [n]: nn; per group
 * [ceil(k/gs), n]: (kk / gs) * n + nn, or, with x2 transposed (the
 * parameters transposed with it), [n, ceil(k/gs)]: nn * ceil(k/gs) + kk / gs.
 *
 *   W   T bits, [k, n] row-major whatever x2's layout.
 */
void oracle_weight_dequant(const void* x2, int w_dtype, int64_t k, int64_t n, int transpose_x2,
                           const void* scale, const void* offset, int param_dtype, int policy,
                           int64_t group_size, uint16_t* W)
{
    int64_t groups = policy == ORC_PER_GROUP ? (k + group_size - 1) / group_size : 1;
    for (int64_t kk = 0; kk < k; ++kk) {
        for (int64_t nn = 0; nn < n; ++nn) {
            int64_t p;
            if (policy == ORC_PER_TENSOR)
                p = 0;
            else if (policy == ORC_PER_CHANNEL)
                p = nn;
            else
                p = transpose_x2 ? nn * groups + kk / group_size : (kk / group_size) * n + nn;
            float v = (float)weight_code(x2, w_dtype, transpose_x2, k, n, kk, nn);
            float s = load_as_f32(scale, param_dtype, p);
            float t;
            if (offset) {
                float u = v + load_as_f32(offset, param_dtype, p);
                t = u * s;
            } else {
                t = v * s;
            }
            W[kk * n + nn] = param_dtype == ORC_BF16 ? orc_f32_to_bf16(t) : orc_f32_to_f16(t);
        }
    }
}

/*
 * out = x1 @ W + bias + x3 for the W above (aclnnWeightQuantMatmulAllReduce
 * on one rank, where the AllReduce is the identity; the page's empty-k case
 * gives bias + x3).  Reading: one product of the exact inputs, the sum
 * accumulated in binary64 here (the device accumulates in binary32), bias
 * [n] and x3 [m, n] added, no intermediate rounding; the result is returned
 * unrounded in binary64 (rounding to T, and the device's accumulation error,
 * are the tests' tolerance).  Also returns sum_kk |x1 * W| per element, the
 * scale of the accumulation error bound.
 *
 *   x1        [m, k] of x_dtype (F16 / BF16).
 *   W         T bits [k, n] from oracle_weight_dequant.
 *   bias, x3  NULL or T [n] / [m, n].
 *   out, mag  binary64 [m, n].
 */
void oracle_weight_quant_matmul(const void* x1, int x_dtype, int64_t m, int64_t k, int64_t n,
                                const uint16_t* W, const void* bias, const void* x3,
                                double* out, double* mag)
{
    for (int64_t mm = 0; mm < m; ++mm) {
        for (int64_t nn = 0; nn < n; ++nn) {
            double acc = 0.0, am = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) {
                double a = (double)load_as_f32(x1, x_dtype, mm * k + kk);
                double w = (double)load_as_f32(W, x_dtype, kk * n + nn);
                acc += a * w; /* exact product (at most 22 significant bits) */
                am += fabs(a * w);
            }
            if (bias)
                acc += (double)load_as_f32(bias, x_dtype, nn);
            if (x3)
                acc += (double)load_as_f32(x3, x_dtype, mm * n + nn);
            out[mm * n + nn] = acc;
            if (mag)
                mag[mm * n + nn] = am;
        }
    }
}

/* Vector form of the double -> bf16 / fp16 rounding, for the tests. */
void orc_convert_f64_to_half(const double* src, int64_t count, int dst_dtype, uint16_t* dst)
{
    for (int64_t i = 0; i < count; ++i)
        dst[i] = orc_f64_to_half(src[i], dst_dtype);
}
