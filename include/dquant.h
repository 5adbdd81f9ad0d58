/*
 * dquant.h -- C ABI of libdquant: per-token dynamic quantization, its
 * AdaLayerNorm fusion, AntiQuantize, mx block quantization and the
 * weight-quantized matmul on AMD MI355X (gfx950).
 *
 * Calling convention (after the two-phase form of the aclnn host ops,
 * "Each operator has two calls": a get-workspace-size call that returns
 * the workspace size and an executor holding the computation, then the
 * execute call):
 *
 *   1. dq_<op>_get_workspace_size(...) validates every argument on the
 *      host, picks the kernel variant and launch geometry and returns an
 *      executor plus the workspace size in bytes.  It makes no HIP call and
 *      touches no device memory, so it is usable without a GPU.
 *   2. dq_<op>(workspace, workspace_size, executor, stream) enqueues the
 *      kernel(s) on `stream` and returns without synchronizing.
 *
 * Ownership
 *   - The caller owns every tensor buffer, the workspace and the stream.
 *     The library never allocates device memory and never synchronizes.
 *     Only the weight-quantized matmul ever asks for a workspace.
 *   - Tensors are dense, row-major (last dimension contiguous) device
 *     buffers described by dq_tensor; the library keeps only the pointers.
 *   - An executor is host memory owned by the library.  The execute call
 *     consumes it, whether it succeeds or fails; an executor that is never
 *     executed must be released with dq_executor_destroy.
 *
 * Errors
 *   Every call returns a dq_status.  On any status other than DQ_SUCCESS,
 *   dq_get_last_error() returns a message for the calling thread and no
 *   executor is returned.  Device faults and other asynchronous errors
 *   surface at the caller's next synchronization on the stream.
 *
 * Determinism: every op is bit-deterministic from run to run (fixed
 * reduction trees, no atomics).
 */
#ifndef DQUANT_H
#define DQUANT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dq_status {
    DQ_SUCCESS = 0,
    DQ_ERR_NULLPTR = 1,   /* a required pointer is NULL                       */
    DQ_ERR_DTYPE = 2,     /* unsupported dtype or dtype combination           */
    DQ_ERR_SHAPE = 3,     /* shapes disagree, or a dimension is out of range  */
    DQ_ERR_ALIGN = 4,     /* a size or address breaks an alignment rule       */
    DQ_ERR_PARAM = 5,     /* a scalar parameter is out of range               */
    DQ_ERR_OVERLAP = 6,   /* an output overlaps an input that forbids it      */
    DQ_ERR_WORKSPACE = 7, /* the workspace passed is smaller than required    */
    DQ_ERR_RUNTIME = 8    /* the HIP runtime rejected a launch                */
} dq_status;

typedef enum dq_dtype {
    DQ_F32 = 0,
    DQ_F16 = 1,
    DQ_BF16 = 2,
    DQ_I8 = 3,
    DQ_I4 = 4,     /* two 4-bit codes per byte, the even element in the low nibble */
    DQ_I32 = 5,    /* int32; as a DynamicQuant output: eight 4-bit codes per word  */
    DQ_F8E4M3 = 6, /* OCP fp8 E4M3FN (no infinities, max 448)                      */
    DQ_F8E5M2 = 7, /* OCP fp8 E5M2 (IEEE-style infinities and NaNs, max 57344)      */
    DQ_F4E2M1 = 8, /* OCP MX fp4 E2M1, two codes per byte, the even element in the
                    * low nibble (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives) */
    DQ_E8M0 = 9    /* OCP MX E8M0 scale: one byte, value 2^(b - 127), 0xFF is NaN  */
} dq_dtype;

#define DQ_MAX_DIMS 8

/* A dense row-major tensor in device memory.  dims[0..ndim-1] are element
 * counts; for DQ_I4 and DQ_F4E2M1 they count 4-bit codes (the buffer holds
 * half as many bytes along the last dimension).  A descriptor whose non-zero
 * dims multiply to more than 2^48 is rejected with DQ_ERR_SHAPE. */
typedef struct dq_tensor {
    void* data;
    int32_t dtype; /* a dq_dtype value; any other value is rejected (DQ_ERR_DTYPE) */
    int32_t ndim;
    int64_t dims[DQ_MAX_DIMS];
} dq_tensor;

typedef struct dq_executor dq_executor;

/* AntiQuantize quantization policy (AntiQuantize, 表1 AntiQuantizePolicy). */
typedef enum dq_antiquant_policy {
    DQ_PER_TENSOR = 0,
    DQ_PER_CHANNEL = 1,
    DQ_PER_TOKEN = 2,
    DQ_PER_GROUP = 3
} dq_antiquant_policy;

/* ------------------------------------------------------------------------
 * DynamicQuant -- aclnnDynamicQuantV2, Description and Formula.
 *
 * Per row r of x (the last dimension is the row; leading dimensions are
 * flattened into R rows of N elements):
 *   in = x * smooth[e(r)]            (when smooth_scales is given)
 *   symmetric:  scale = row_max(|in|) / D,  y = round(in / scale)
 *   asymmetric: scale = (row_max(in) - row_min(in)) / scale_opt,
 *               offset = offset_opt - row_max(in) / scale,
 *               y = round(in / scale + offset)
 * with (scale_opt, offset_opt) = (255, 127) for INT8 and (15, 7) for INT4
 * and INT32 output, D = offset_opt, round = half to even, codes saturated
 * to [-128, 127] or [-8, 7] (NaN -> 0).  Every step is one correctly
 * rounded binary32 operation in the order printed, so results are
 * bit-exact against a plain IEEE evaluation.
 *
 *   x             F16 or BF16, [..., N], N >= 1.  R = prod(leading dims)
 *                 may be 0 (the execute call is then a no-op).
 *   smooth_scales NULL, or F32 [N] (no group_index), or F32 [E, N] with
 *                 group_index.
 *   group_index   NULL, or I32 [E] (E >= 1) holding cumulative per-expert
 *                 row ends: expert e owns rows [gi[e-1], gi[e]); the owner
 *                 of row r is the first e with r < gi[e], and rows at or
 *                 past gi[E-1] belong to expert E-1.  (aclnnDynamicQuantV2,
 *                 Description: in the MoE case every expert has its own
 *                 smooth-scale row, and the group index tells which rows
 *                 use which.)  Requires smooth_scales.  Its device contents
 *                 are not validated.
 *   symmetric     nonzero: symmetric; 0: asymmetric.
 *   y             output.  DQ_I8 [..., N]; DQ_I4 [..., N] with N even
 *                 (N/2 bytes per row); DQ_I32 [..., N/8] with N % 8 == 0
 *                 (code 8w+i in bits [4i, 4i+3] of word w, so the bytes
 *                 equal the INT4 bytes).
 *   scale         output, F32, shape x.shape[:-1].
 *   offset        output, F32, shape x.shape[:-1]; required when
 *                 asymmetric, must be NULL when symmetric.
 *   workspace_size, executor: returned.  The workspace size is 0.
 * Errors: DQ_ERR_NULLPTR (missing x/y/scale/offset, NULL data),
 *   DQ_ERR_DTYPE, DQ_ERR_SHAPE (shape mismatch, N == 0, INT4 N odd, INT32
 *   N % 8 != 0, group_index without smooth_scales), DQ_ERR_PARAM (offset
 *   given for symmetric).
 * ------------------------------------------------------------------------ */
dq_status dq_dynamic_quant_get_workspace_size(const dq_tensor* x, const dq_tensor* smooth_scales,
                                              const dq_tensor* group_index, int symmetric,
                                              const dq_tensor* y, const dq_tensor* scale,
                                              const dq_tensor* offset, size_t* workspace_size,
                                              dq_executor** executor);
dq_status dq_dynamic_quant(void* workspace, size_t workspace_size, dq_executor* executor,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * AdaLayerNorm + DynamicQuant fusion -- aclnnAdaLayerNormQuant, Formula.
 *
 * For each row (b, s) of x [B, S, H]:
 *   LN = (x - E(x)) / sqrt(Var(x) + epsilon) * weight + bias  (biased Var)
 *   y  = LN * (1 + scale[b]) + shift[b];  y = y * smooth       (if given)
 *   quant_scale = row_max(|y|) / 127;  out = round(y / quant_scale)
 * Only symmetric INT8 quantization is fused (the page: "only DynamicQuant
 * is supported").  Statistics and modulation run in fp32 on the device;
 * the quantization step is the bit-exact symmetric step of DynamicQuant
 * applied to the fp32 y.
 *
 *   x             F16 or BF16 [B, S, H], H >= 1; B * S may be 0.
 *   scale, shift  same dtype as x, [B, 1, H] or [B, H].
 *   weight, bias  NULL or same dtype as x, [H] (absent: weight 1, bias 0).
 *   smooth_scales NULL or F32 [H].
 *   epsilon       > 0 and finite (used as fp32).
 *   out           I8 [B, S, H].   quant_scale: F32 [B, S].
 *   workspace size: 0.
 * Errors: DQ_ERR_NULLPTR, DQ_ERR_DTYPE, DQ_ERR_SHAPE, DQ_ERR_PARAM
 *   (epsilon <= 0 or not finite).
 * ------------------------------------------------------------------------ */
dq_status dq_ada_layernorm_quant_get_workspace_size(const dq_tensor* x, const dq_tensor* scale,
                                                    const dq_tensor* shift,
                                                    const dq_tensor* weight,
                                                    const dq_tensor* bias,
                                                    const dq_tensor* smooth_scales,
                                                    double epsilon, const dq_tensor* out,
                                                    const dq_tensor* quant_scale,
                                                    size_t* workspace_size,
                                                    dq_executor** executor);
dq_status dq_ada_layernorm_quant(void* workspace, size_t workspace_size, dq_executor* executor,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * AntiQuantize -- AntiQuantize (Ascend C API), 功能说明 / 表1-表3 / 约束说明.
 *
 * Element-wise dequantization of src [m, n] into dst [m, n]:
 *   dst[i, j] = (src[i, j] + offset[p]) * scale[p]     (offset given)
 *   dst[i, j] = src[i, j] * scale[p]                    (offset NULL,
 *                                                        hasOffset = false)
 * computed as two correctly rounded fp32 operations, then rounded once
 * (nearest even) to dst's type.  The parameter p by policy:
 *   DQ_PER_TENSOR   scale/offset [1]                         p = 0
 *   DQ_PER_CHANNEL  [1, n] (or [n])                          p = j
 *   DQ_PER_TOKEN    [m, 1] (or [m])                          p = i
 *   DQ_PER_GROUP    k_dim = 1: [m, ceil(n/gs)]               p = (i, j / gs)
 *                   k_dim = 0: [ceil(m/gs), n]               p = (i / gs, j)
 * The page leaves the formula itself out; the sign convention of the
 * offset is this library's reading (it is the value that undoes
 * DynamicQuant's "+ offset" when passed negated).
 *
 * The float4 case of 表3 (fp4x2 source, fp8_e8m0 scale, PER_GROUP only,
 * no offset -- 约束说明) reads its missing formula the same way:
 *   dst[i, j] = decode(src[i, j]) * 2^(scale[p] - 127)
 * as one correctly rounded fp32 multiply (exact unless it overflows to
 * infinity; scale 0xFF is NaN), then rounded once to dst's type.
 *
 *   src        I8, F8E4M3 or F8E5M2 (the b8 cases of 表3), or F4E2M1 (the
 *              float4 case), exactly 2-D [m, n] (the page: at most two
 *              dims); for F4E2M1 n counts 4-bit codes and must be even.
 *   scale      b8 sources: F32, F16 or BF16 (widened exactly), policy
 *              shape.  F4E2M1: E8M0.
 *   offset     NULL, or the scale's dtype and shape; NULL for F4E2M1.
 *   policy     a dq_antiquant_policy value (anything else: DQ_ERR_PARAM).
 *   k_dim      0 or 1, used by DQ_PER_GROUP only.
 *   group_size DQ_PER_GROUP: > 0 and a multiple of 32 (表2); ignored
 *              otherwise.
 *   dst        BF16 or F16 [m, n] (表3), or, for b8 sources, F32 [m, n]
 *              (the unrounded binary32 result, an extension of this
 *              library).
 *   n * sizeof(src) and n * sizeof(dst) must be multiples of 32 bytes and
 *   src/dst 16-byte aligned (约束说明: 32-byte aligned rows); PER_CHANNEL
 *   and PER_GROUP k_dim = 0 parameters 16-byte aligned (8 for E8M0); src
 *   and dst must not overlap.  m may be 0.  Workspace size: 0.
 * Errors: DQ_ERR_NULLPTR, DQ_ERR_DTYPE (including an F4E2M1 source with a
 *   non-E8M0 scale, an offset, or an F32 dst), DQ_ERR_SHAPE (ndim != 2,
 *   param shape, odd n for F4E2M1), DQ_ERR_ALIGN, DQ_ERR_PARAM (policy,
 *   k_dim, group_size, an F4E2M1 source with a policy other than
 *   PER_GROUP), DQ_ERR_OVERLAP.
 * ------------------------------------------------------------------------ */
dq_status dq_antiquantize_get_workspace_size(const dq_tensor* src, const dq_tensor* scale,
                                             const dq_tensor* offset, int32_t policy,
                                             int32_t k_dim, uint32_t group_size,
                                             const dq_tensor* dst, size_t* workspace_size,
                                             dq_executor** executor);
dq_status dq_antiquantize(void* workspace, size_t workspace_size, dq_executor* executor,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * mx block quantization -- the producer of the block-scaled operands that
 * the mx formula of aclnnQuantBatchMatmulInplaceAdd (计算公式, mx量化)
 * consumes: one FLOAT8_E8M0 scale per block of gsK = 32 consecutive
 * elements along the contraction axis, the last block possibly short.  The
 * pages print only that consumer; the conversion is the OCP Microscaling
 * v1.0 one.  Per block of elements v:
 *   shared = floor(log2(max |v|)) - emax, clamped to [-127, 127]
 *            (emax = 8 for F8E4M3, 15 for F8E5M2, 2 for F4E2M1)
 *   scale  = shared + 127                         (E8M0 byte)
 *   y_i    = the element value nearest to v_i / 2^shared, ties to even,
 *            saturated to the largest finite magnitude (448, 57344, 6),
 *            the sign of v_i kept also on a zero result.
 * An all-zero block gets scale 0 and zero codes; a block holding a NaN or
 * an infinity gets scale 0xFF (NaN) and all-zero codes.  Decoding
 * y_i * 2^(scale - 127) -- AntiQuantize's float4 case, or the mx formula --
 * gives back the nearest representable value of every element.
 *
 *   x      F16 or BF16, exactly 2-D [rows, n]; rows may be 0, n >= 1,
 *          n < 2^31.
 *   axis   1: blocks run along n (the x1 [M, K] layout of the mx formula):
 *             scale [rows, ceil(n/32)], scale[r, j] covers x[r, 32j .. 32j+31].
 *          0: blocks run down the rows (the x2 [K, N] layout): scale
 *             [ceil(rows/32), n], scale[j, c] covers x[32j .. 32j+31, c].
 *   y      F8E4M3 or F8E5M2 [rows, n] (one code per byte), or F4E2M1
 *          [rows, n] (n even; two codes per byte along n, the even element
 *          in the low nibble -- the layout AntiQuantize reads).
 *   scale  E8M0, the shape given by axis.
 *   No alignment is required.  The vector kernels are used when n % 8 == 0,
 *   x is 16-byte aligned and y 8-byte (fp8) or 4-byte (fp4) aligned, and,
 *   for axis 0, scale is 8-byte aligned; otherwise a generic kernel runs.
 *   y and scale must not overlap x or each other.  Workspace size: 0.
 * Errors: DQ_ERR_NULLPTR, DQ_ERR_DTYPE, DQ_ERR_SHAPE (ndim != 2, shapes,
 *   n == 0, n >= 2^31, odd n for F4E2M1), DQ_ERR_PARAM (axis not 0 or 1),
 *   DQ_ERR_OVERLAP.
 * ------------------------------------------------------------------------ */
dq_status dq_mx_quantize_get_workspace_size(const dq_tensor* x, int32_t axis, const dq_tensor* y,
                                            const dq_tensor* scale, size_t* workspace_size,
                                            dq_executor** executor);
dq_status dq_mx_quantize(void* workspace, size_t workspace_size, dq_executor* executor,
                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Weight-quantized matmul -- aclnnWeightQuantMatmulAllReduce on one GPU
 * (API function: the weight x2 is fake-quantized, then multiplied; the
 * all-reduce over ranks is the identity on one rank; constraints: shapes,
 * dtypes, parameter shapes, the empty-k case).  The page's formula is
 * missing; this library reads it with the AntiQuantize arithmetic:
 *   W[k, n]   = RN_T((x2[k, n] + offset[p]) * scale[p])   (two binary32
 *               operations, or one without offset, rounded once to T)
 *   out[m, n] = RN_T(sum_k x1[m, k] * W[k, n] + bias[n] + x3[m, n])
 * with the sum accumulated in binary32 (any order) and one final rounding;
 * T is x1's dtype.  With k == 0 the output is bias + x3 (the page's empty
 * case).  The result is within gamma_{k+2} * (sum_k |x1 W| + |bias| + |x3|)
 * + half an ulp of T of the exact value, gamma_j = j 2^-24 / (1 - j 2^-24).
 *
 *   x1            F16 or BF16, [m, k] or [b, s, k]; m = prod(leading dims)
 *                 may be 0.  k in [0, 65535].
 *   x2            I8, or I4 (two signed 4-bit codes per byte along the
 *                 stored last dimension, the even element in the low
 *                 nibble).  transpose_x2 == 0: [k, n] in memory;
 *                 transpose_x2 != 0: [n, k] in memory (x2 given as its
 *                 transpose, the nn.Linear layout).  n in [1, 65535].
 *   antiquant_scale   x1's dtype.  group_size == 0: [1] (per tensor) or
 *                 [n] / [1, n] (per channel).  group_size > 0 (a multiple
 *                 of 32): [ceil(k/gs), n], or [n, ceil(k/gs)] when
 *                 transpose_x2 (the parameters transposed with x2).
 *   antiquant_offset  NULL, or the scale's dtype and shape.
 *   bias          NULL or x1's dtype [n].
 *   x3            NULL or x1's dtype with out's shape.
 *   out           x1's dtype, x1.shape[:-1] + [n]; must not overlap an input.
 *   The matrix-core kernel runs when transpose_x2 is set, k % 32 == 0 (I8)
 *   or k % 64 == 0 (I4), and x1 and x2 are 16-byte aligned; otherwise a
 *   generic kernel (one thread per output element) computes the same
 *   arithmetic much more slowly.
 *   Workspace: 0 bytes, except when the output has too few tiles to fill
 *   the GPU (small m * n): then k is split across workgroups and the
 *   workspace holds the binary32 partial sums, splits * m * n * 4 bytes
 *   (16-byte aligned, owned by the caller, contents scratch).  The partial
 *   sums are added in split order, so results stay bit-reproducible.
 * Errors: DQ_ERR_NULLPTR, DQ_ERR_DTYPE, DQ_ERR_SHAPE (ranks, shapes, k or n
 *   out of range, odd stored last dimension for I4), DQ_ERR_PARAM
 *   (group_size negative or not a multiple of 32), DQ_ERR_OVERLAP;
 *   execute: DQ_ERR_WORKSPACE (workspace NULL or smaller than returned),
 *   DQ_ERR_ALIGN (workspace not 16-byte aligned).
 * ------------------------------------------------------------------------ */
dq_status dq_weight_quant_matmul_get_workspace_size(const dq_tensor* x1, const dq_tensor* x2,
                                                    int32_t transpose_x2,
                                                    const dq_tensor* antiquant_scale,
                                                    const dq_tensor* antiquant_offset,
                                                    int64_t group_size, const dq_tensor* bias,
                                                    const dq_tensor* x3, const dq_tensor* out,
                                                    size_t* workspace_size, dq_executor** executor);
dq_status dq_weight_quant_matmul(void* workspace, size_t workspace_size, dq_executor* executor,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Allocation-free weight-quantized matmul.
 *
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * validation, plan, kernels and results as the two-phase pair above, in one
 * call that allocates nothing, neither device memory nor host memory (no
 * executor).  Where the plan splits k, the binary32 partial sums go to a
 * scratch array the library owns, DQ_WQ_SCRATCH_BYTES (32 MiB) per GPU,
 * held on each GPU the call runs on until the process ends; it needs no
 * clearing (every split writes all of its partial sums).
 *
 *   Arguments as for dq_weight_quant_matmul_get_workspace_size, plus the
 *   stream, whose device must be the current device.
 *   Errors: those of dq_weight_quant_matmul_get_workspace_size;
 *   DQ_ERR_WORKSPACE when the partial sums would exceed DQ_WQ_SCRATCH_BYTES
 *   (splits * m * n * 4 bytes: decode shapes need at most about 2 MiB, and
 *   only prefill shapes with few output tiles come near the limit); use the
 *   two-phase pair with a caller workspace then.  DQ_ERR_PARAM when the
 *   stream belongs to another device; DQ_ERR_RUNTIME on a launch failure.
 *   Every call on one GPU shares that GPU's scratch array: calls that
 *   overlap on one GPU (concurrent streams, or graphs replayed
 *   concurrently) race on it and must be serialized by the caller.
 * ------------------------------------------------------------------------ */
#define DQ_WQ_SCRATCH_BYTES ((size_t)32 << 20)
dq_status dq_weight_quant_matmul_noalloc(const dq_tensor* x1, const dq_tensor* x2, int32_t transpose_x2,
                                         const dq_tensor* antiquant_scale,
                                         const dq_tensor* antiquant_offset, int64_t group_size,
                                         const dq_tensor* bias, const dq_tensor* x3, const dq_tensor* out,
                                         hipStream_t stream);

/* Release an executor that was never passed to an execute call.  NULL is a
 * no-op. */
void dq_executor_destroy(dq_executor* executor);

/* Message for the calling thread's last non-success status ("" if none).
 * The pointer stays valid until the thread's next libdquant call. */
const char* dq_get_last_error(void);

/* Measurement utility (not a quantization op): enqueue a plain device copy
 * of `bytes` bytes (a multiple of 16, both pointers 16-byte aligned, no
 * overlap) on `stream`.  Its bandwidth is the achievable-ceiling reference
 * for the memory-bound kernels above, and its HBM counters calibrate the
 * profiler's FETCH_SIZE / WRITE_SIZE readings. */
dq_status dq_copy_probe(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DQUANT_H */
