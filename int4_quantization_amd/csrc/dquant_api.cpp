// dquant_api.cpp -- the C ABI of libdquant: argument validation, kernel
// variant selection and executors (phase 1, host only, no HIP calls), and
// the execute calls that enqueue the kernels (phase 2).
//
// The two-phase shape follows the aclnn host ops (aclnnDynamicQuantV2,
// aclnnAdaLayerNormQuant: a get-workspace-size call that validates the
// parameters and returns an executor, then the execute call).

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "dq_ext_internal.h"

enum ExecOp : int {
    OP_DYNAMIC_QUANT = 1,
    OP_ADA_LAYERNORM_QUANT = 2,
    OP_ANTIQUANTIZE = 3,
    OP_MX_QUANTIZE = 4,
    OP_WEIGHT_QUANT_MATMUL = 5
};

struct dq_executor {
    int op;
    dq::DqPlan dq;
    dq::AdaPlan ada;
    dq::AqPlan aq;
    dq::MxPlan mx;
    dq::WqPlan wq;
};

namespace {

thread_local std::string g_last_error;

dq_status fail(dq_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

dq_status ok()
{
    g_last_error.clear();
    return DQ_SUCCESS;
}

const char* dtype_name(int32_t d)
{
    switch (d) {
    case DQ_F32: return "F32";
    case DQ_F16: return "F16";
    case DQ_BF16: return "BF16";
    case DQ_I8: return "I8";
    case DQ_I4: return "I4";
    case DQ_I32: return "I32";
    case DQ_F8E4M3: return "F8E4M3";
    case DQ_F8E5M2: return "F8E5M2";
    case DQ_F4E2M1: return "F4E2M1";
    case DQ_E8M0: return "E8M0";
    }
    return "unknown";
}

// Largest element count a tensor may describe (2^48, far beyond any HBM).
// Bounding the product of the non-zero dims keeps every element, byte and
// row count derived from a shape inside int64, for empty tensors too.
constexpr int64_t kMaxElems = int64_t(1) << 48;

// Checks ndim range, non-negative dims and the element-count bound; returns
// the element count.
bool shape_ok(const dq_tensor* t, int64_t* numel)
{
    if (t->ndim < 0 || t->ndim > DQ_MAX_DIMS)
        return false;
    int64_t nonzero = 1;
    bool empty = false;
    for (int i = 0; i < t->ndim; ++i) {
        const int64_t d = t->dims[i];
        if (d < 0)
            return false;
        if (d == 0) {
            empty = true;
            continue;
        }
        if (nonzero > kMaxElems / d)
            return false;
        nonzero *= d;
    }
    *numel = empty ? 0 : nonzero;
    return true;
}

// A tensor's data must be non-null whenever it holds elements.
dq_status check_tensor(const dq_tensor* t, const char* name, int64_t* numel)
{
    if (!t)
        return fail(DQ_ERR_NULLPTR, "%s is NULL", name);
    int64_t n = 0;
    if (!shape_ok(t, &n))
        return fail(DQ_ERR_SHAPE, "%s: ndim %d or a dimension is out of range", name, t->ndim);
    if (n > 0 && !t->data)
        return fail(DQ_ERR_NULLPTR, "%s->data is NULL", name);
    if (numel)
        *numel = n;
    return DQ_SUCCESS;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool same_dims(const dq_tensor* t, const int64_t* dims, int ndim)
{
    if (t->ndim != ndim)
        return false;
    for (int i = 0; i < ndim; ++i)
        if (t->dims[i] != dims[i])
            return false;
    return true;
}

// Shape [d0] or [1, d0] / [d0, 1] style checks used by AntiQuantize.
bool is_shape(const dq_tensor* t, std::initializer_list<int64_t> want)
{
    if (t->ndim != static_cast<int>(want.size()))
        return false;
    int i = 0;
    for (int64_t w : want)
        if (t->dims[i++] != w)
            return false;
    return true;
}

int64_t elem_bytes_x16(int32_t d)  // bytes per element times 2 (I4 is half a byte)
{
    switch (d) {
    case DQ_F32: case DQ_I32: return 8;
    case DQ_F16: case DQ_BF16: return 4;
    case DQ_I8: case DQ_F8E4M3: case DQ_F8E5M2: case DQ_E8M0: return 2;
    case DQ_I4: case DQ_F4E2M1: return 1;
    }
    return 0;
}

dq_executor* new_executor(int op)
{
    dq_executor* e = new (std::nothrow) dq_executor;
    if (e) {
        std::memset(e, 0, sizeof *e);
        e->op = op;
    }
    return e;
}

// Workgroups the weight-quantized matmul aims for when splitting k.
// Split-k targets (workgroups), measured: k is split only while the output
// tiles alone would leave the chip short of work, since every split costs a
// binary32 partial tile and a reduce launch.
constexpr int64_t kWqTargetBlocks = 384, kWqGemmTargetBlocks = 512;

int pick_vpl(int64_t per_lane, const int* choices, int count)
{
    for (int i = 0; i < count; ++i)
        if (choices[i] >= per_lane)
            return choices[i];
    return -1;
}

}  // namespace

extern "C" {

const char* dq_get_last_error(void) { return g_last_error.c_str(); }

void dq_executor_destroy(dq_executor* executor) { delete executor; }

// ---------------------------------------------------------------------------
// DynamicQuant
// ---------------------------------------------------------------------------
dq_status dq_dynamic_quant_get_workspace_size(const dq_tensor* x, const dq_tensor* smooth_scales,
                                              const dq_tensor* group_index, int symmetric,
                                              const dq_tensor* y, const dq_tensor* scale,
                                              const dq_tensor* offset, size_t* workspace_size,
                                              dq_executor** executor)
{
    if (!workspace_size || !executor)
        return fail(DQ_ERR_NULLPTR, "workspace_size and executor must not be NULL");
    *executor = nullptr;
    *workspace_size = 0;
    dq_status st;
    int64_t nx = 0, ny = 0, ns = 0;
    if ((st = check_tensor(x, "x", &nx)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(y, "y", &ny)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(scale, "scale", &ns)) != DQ_SUCCESS) return st;

    if (x->dtype != DQ_F16 && x->dtype != DQ_BF16)
        return fail(DQ_ERR_DTYPE, "x must be F16 or BF16, got %s", dtype_name(x->dtype));
    if (y->dtype != DQ_I8 && y->dtype != DQ_I4 && y->dtype != DQ_I32)
        return fail(DQ_ERR_DTYPE, "y must be I8, I4 or I32, got %s", dtype_name(y->dtype));
    if (scale->dtype != DQ_F32)
        return fail(DQ_ERR_DTYPE, "scale must be F32, got %s", dtype_name(scale->dtype));
    if (x->ndim < 1)
        return fail(DQ_ERR_SHAPE, "x must have at least one dimension");
    const int64_t n = x->dims[x->ndim - 1];
    if (n < 1)
        return fail(DQ_ERR_SHAPE, "the last dimension of x must be >= 1");
    const int64_t rows = nx / n;
    if (rows > dq::kMaxGridBlocks)
        return fail(DQ_ERR_SHAPE, "at most %lld rows are supported, got %lld", (long long)dq::kMaxGridBlocks,
                    (long long)rows);

    if (y->dtype == DQ_I8 || y->dtype == DQ_I4) {
        if (!same_dims(y, x->dims, x->ndim))
            return fail(DQ_ERR_SHAPE, "y must have the shape of x");
        if (y->dtype == DQ_I4 && n % 2 != 0)
            return fail(DQ_ERR_SHAPE, "INT4 output needs an even last dimension, got %lld",
                        (long long)n);
    } else {
        if (n % 8 != 0)
            return fail(DQ_ERR_SHAPE, "INT32 output needs the last dimension of x divisible by 8, got %lld",
                        (long long)n);
        int64_t want[DQ_MAX_DIMS];
        std::memcpy(want, x->dims, sizeof want);
        want[x->ndim - 1] = n / 8;
        if (!same_dims(y, want, x->ndim))
            return fail(DQ_ERR_SHAPE, "INT32 y must be x.shape[:-1] + [N/8]");
    }
    if (!same_dims(scale, x->dims, x->ndim - 1))
        return fail(DQ_ERR_SHAPE, "scale must have shape x.shape[:-1]");

    if (symmetric) {
        if (offset)
            return fail(DQ_ERR_PARAM, "offset must be NULL for symmetric quantization");
    } else {
        int64_t no = 0;
        if (!offset)
            return fail(DQ_ERR_NULLPTR, "asymmetric quantization needs an offset output");
        if ((st = check_tensor(offset, "offset", &no)) != DQ_SUCCESS) return st;
        if (offset->dtype != DQ_F32)
            return fail(DQ_ERR_DTYPE, "offset must be F32, got %s", dtype_name(offset->dtype));
        if (!same_dims(offset, x->dims, x->ndim - 1))
            return fail(DQ_ERR_SHAPE, "offset must have shape x.shape[:-1]");
    }

    int64_t n_experts = 0;
    if (group_index) {
        int64_t ng = 0;
        if (!smooth_scales)
            return fail(DQ_ERR_SHAPE, "group_index needs smooth_scales [E, N]");
        if ((st = check_tensor(group_index, "group_index", &ng)) != DQ_SUCCESS) return st;
        if (group_index->dtype != DQ_I32)
            return fail(DQ_ERR_DTYPE, "group_index must be I32, got %s", dtype_name(group_index->dtype));
        if (group_index->ndim != 1 || group_index->dims[0] < 1)
            return fail(DQ_ERR_SHAPE, "group_index must be [E] with E >= 1");
        if (!group_index->data)
            return fail(DQ_ERR_NULLPTR, "group_index->data is NULL");
        n_experts = group_index->dims[0];
    }
    if (smooth_scales) {
        int64_t nsm = 0;
        if ((st = check_tensor(smooth_scales, "smooth_scales", &nsm)) != DQ_SUCCESS) return st;
        if (smooth_scales->dtype != DQ_F32)
            return fail(DQ_ERR_DTYPE, "smooth_scales must be F32, got %s",
                        dtype_name(smooth_scales->dtype));
        if (group_index) {
            if (!is_shape(smooth_scales, {n_experts, n}))
                return fail(DQ_ERR_SHAPE, "smooth_scales must be [E, N] = [%lld, %lld]",
                            (long long)n_experts, (long long)n);
        } else if (!is_shape(smooth_scales, {n})) {
            return fail(DQ_ERR_SHAPE, "smooth_scales must be [N] = [%lld]", (long long)n);
        }
        if (!smooth_scales->data)
            return fail(DQ_ERR_NULLPTR, "smooth_scales->data is NULL");
    }

    dq_executor* e = new_executor(OP_DYNAMIC_QUANT);
    if (!e)
        return fail(DQ_ERR_RUNTIME, "out of host memory");
    dq::DqPlan& p = e->dq;
    p.x = x->data;
    p.smooth = smooth_scales ? static_cast<const float*>(smooth_scales->data) : nullptr;
    p.group_index = group_index ? static_cast<const int32_t*>(group_index->data) : nullptr;
    p.n_experts = n_experts;
    p.rows = rows;
    p.n = n;
    p.x_type = x->dtype == DQ_F16 ? dq::X_F16 : dq::X_BF16;
    p.out_kind = y->dtype == DQ_I8 ? dq::OUT_I8 : dq::OUT_I4;
    p.symmetric = symmetric != 0;
    p.y = y->data;
    p.scale = static_cast<float*>(scale->data);
    p.offset = symmetric ? nullptr : static_cast<float*>(offset->data);

    // Register-resident variant: rows of whole 16-byte vectors and aligned
    // buffers.  A row goes to the smallest team of waves (1, 2 or 4) that
    // holds it within 4 vectors per lane; wider rows take 8 or 16 vectors
    // per lane on a team of 4; longer rows go to the generic variant.
    const bool vec_ok = n % 8 == 0 && aligned(p.x, 16) && (!p.smooth || aligned(p.smooth, 16)) &&
                        aligned(p.y, p.out_kind == dq::OUT_I8 ? 8 : 4);
    p.variant = dq::DQ_VAR_GENERIC;
    if (vec_ok) {
        const int64_t nvec = n / 8;
        for (int t = 1; t <= dq::kDqWaves; t *= 2) {
            if (nvec <= dq::kDqTeamVpl * 64 * t) {
                static const int kVpl[] = {1, 2, 4};
                p.vpl = pick_vpl((nvec + 64 * t - 1) / (64 * t), kVpl, 3);
                p.team = t;
                p.variant = dq::DQ_VAR_VECTOR;
                break;
            }
        }
        if (p.variant != dq::DQ_VAR_VECTOR && n <= dq::kDqVecMaxRow) {
            static const int kVplWide[] = {8, 16};
            p.vpl = pick_vpl((nvec + 64 * dq::kDqWaves - 1) / (64 * dq::kDqWaves), kVplWide, 2);
            p.team = dq::kDqWaves;
            p.variant = dq::DQ_VAR_VECTOR;
        }
        // Where that team would hold duplicate vectors and 2 (or 1) vectors
        // per lane over 5 to 16 waves cover the row exactly, one workgroup is
        // one such team: no lane loads, converts or stores a duplicate (bf16
        // [8192, 7168]: 31.62 against 31.58 us in interleaved runs, the
        // same time; the kernel's memory traffic is what bounds it).
        if (p.variant == dq::DQ_VAR_VECTOR && int64_t{p.team} * p.vpl * 64 > nvec && nvec % 64 == 0) {
            for (int v = 2; v >= 1; --v) {
                const int64_t w = nvec / 64 / v;
                if ((nvec / 64) % v == 0 && w >= 5 && w <= dq::kDqMaxTeam) {
                    p.variant = dq::DQ_VAR_TEAM;
                    p.vpl = v;
                    p.team = static_cast<int>(w);
                    p.long_rows = !p.group_index && rows >= dq::kDqTeamLongMinRows;
                    break;
                }
            }
        }
    }
    *executor = e;
    return ok();
}

dq_status dq_dynamic_quant(void* workspace, size_t workspace_size, dq_executor* executor,
                           hipStream_t stream)
{
    (void)workspace;
    (void)workspace_size;  // no workspace is needed
    if (!executor)
        return fail(DQ_ERR_NULLPTR, "executor is NULL");
    dq_executor* e = executor;
    if (e->op != OP_DYNAMIC_QUANT) {
        delete e;
        return fail(DQ_ERR_PARAM, "executor was not made by dq_dynamic_quant_get_workspace_size");
    }
    dq::DqPlan p = e->dq;
    delete e;
    if (p.rows == 0)
        return ok();
    hipError_t err = dq::launch_dynamic_quant(p, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "dynamic_quant launch failed: %s", hipGetErrorString(err));
    return ok();
}

// ---------------------------------------------------------------------------
// AdaLayerNorm-quant
// ---------------------------------------------------------------------------
dq_status dq_ada_layernorm_quant_get_workspace_size(const dq_tensor* x, const dq_tensor* scale,
                                                    const dq_tensor* shift,
                                                    const dq_tensor* weight,
                                                    const dq_tensor* bias,
                                                    const dq_tensor* smooth_scales,
                                                    double epsilon, const dq_tensor* out,
                                                    const dq_tensor* quant_scale,
                                                    size_t* workspace_size,
                                                    dq_executor** executor)
{
    if (!workspace_size || !executor)
        return fail(DQ_ERR_NULLPTR, "workspace_size and executor must not be NULL");
    *executor = nullptr;
    *workspace_size = 0;
    dq_status st;
    if ((st = check_tensor(x, "x", nullptr)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(scale, "scale", nullptr)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(shift, "shift", nullptr)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(out, "out", nullptr)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(quant_scale, "quant_scale", nullptr)) != DQ_SUCCESS) return st;
    if (weight && (st = check_tensor(weight, "weight", nullptr)) != DQ_SUCCESS) return st;
    if (bias && (st = check_tensor(bias, "bias", nullptr)) != DQ_SUCCESS) return st;
    if (smooth_scales && (st = check_tensor(smooth_scales, "smooth_scales", nullptr)) != DQ_SUCCESS)
        return st;

    if (x->dtype != DQ_F16 && x->dtype != DQ_BF16)
        return fail(DQ_ERR_DTYPE, "x must be F16 or BF16, got %s", dtype_name(x->dtype));
    const dq_tensor* same[] = {scale, shift, weight, bias};
    const char* names[] = {"scale", "shift", "weight", "bias"};
    for (int i = 0; i < 4; ++i)
        if (same[i] && same[i]->dtype != x->dtype)
            return fail(DQ_ERR_DTYPE, "%s must have x's dtype %s, got %s", names[i],
                        dtype_name(x->dtype), dtype_name(same[i]->dtype));
    if (smooth_scales && smooth_scales->dtype != DQ_F32)
        return fail(DQ_ERR_DTYPE, "smooth_scales must be F32, got %s", dtype_name(smooth_scales->dtype));
    if (out->dtype != DQ_I8)
        return fail(DQ_ERR_DTYPE, "out must be I8 (only symmetric INT8 is fused), got %s",
                    dtype_name(out->dtype));
    if (quant_scale->dtype != DQ_F32)
        return fail(DQ_ERR_DTYPE, "quant_scale must be F32, got %s", dtype_name(quant_scale->dtype));

    if (x->ndim != 3)
        return fail(DQ_ERR_SHAPE, "x must be [B, S, H]");
    const int64_t B = x->dims[0], S = x->dims[1], H = x->dims[2];
    if (S > 0 && B > dq::kMaxGridBlocks / S)
        return fail(DQ_ERR_SHAPE, "at most %lld rows (B * S) are supported", (long long)dq::kMaxGridBlocks);
    if (H < 1)
        return fail(DQ_ERR_SHAPE, "H must be >= 1");
    if (!(is_shape(scale, {B, 1, H}) || is_shape(scale, {B, H})))
        return fail(DQ_ERR_SHAPE, "scale must be [B, 1, H] or [B, H]");
    if (!(is_shape(shift, {B, 1, H}) || is_shape(shift, {B, H})))
        return fail(DQ_ERR_SHAPE, "shift must be [B, 1, H] or [B, H]");
    if (weight && !is_shape(weight, {H}))
        return fail(DQ_ERR_SHAPE, "weight must be [H]");
    if (bias && !is_shape(bias, {H}))
        return fail(DQ_ERR_SHAPE, "bias must be [H]");
    if (smooth_scales && !is_shape(smooth_scales, {H}))
        return fail(DQ_ERR_SHAPE, "smooth_scales must be [H]");
    if (!same_dims(out, x->dims, 3))
        return fail(DQ_ERR_SHAPE, "out must have the shape of x");
    if (!is_shape(quant_scale, {B, S}))
        return fail(DQ_ERR_SHAPE, "quant_scale must be [B, S]");
    if (!(epsilon > 0.0) || !std::isfinite(epsilon))
        return fail(DQ_ERR_PARAM, "epsilon must be positive and finite");
    if (H > 0 && B > 0 && (!scale->data || !shift->data))
        return fail(DQ_ERR_NULLPTR, "scale/shift data is NULL");

    dq_executor* e = new_executor(OP_ADA_LAYERNORM_QUANT);
    if (!e)
        return fail(DQ_ERR_RUNTIME, "out of host memory");
    dq::AdaPlan& p = e->ada;
    p.x = x->data;
    p.scale = scale->data;
    p.shift = shift->data;
    p.weight = weight ? weight->data : nullptr;
    p.bias = bias ? bias->data : nullptr;
    p.smooth = smooth_scales ? static_cast<const float*>(smooth_scales->data) : nullptr;
    p.B = B;
    p.S = S;
    p.H = H;
    p.x_type = x->dtype == DQ_F16 ? dq::X_F16 : dq::X_BF16;
    p.eps = static_cast<float>(epsilon);
    p.out = static_cast<int8_t*>(out->data);
    p.quant_scale = static_cast<float*>(quant_scale->data);

    static const int kVpl[] = {1, 2, 4, 6, 8, 12, 16};
    // The vector variant reads eight columns of every parameter with one
    // 16-byte load, so they need 16-byte alignment too.
    const bool vec_ok = H % 8 == 0 && aligned(p.x, 16) && aligned(p.out, 8) && aligned(p.scale, 16) &&
                        aligned(p.shift, 16) && (!p.weight || aligned(p.weight, 16)) &&
                        (!p.bias || aligned(p.bias, 16)) && (!p.smooth || aligned(p.smooth, 16));
    int v = vec_ok ? pick_vpl((H / 8 + 63) / 64, kVpl, 7) : -1;
    p.variant = v > 0 ? dq::ADA_VAR_VECTOR : dq::ADA_VAR_GENERIC;
    p.vpl = v;
    *executor = e;
    return ok();
}

dq_status dq_ada_layernorm_quant(void* workspace, size_t workspace_size, dq_executor* executor,
                                 hipStream_t stream)
{
    (void)workspace;
    (void)workspace_size;
    if (!executor)
        return fail(DQ_ERR_NULLPTR, "executor is NULL");
    dq_executor* e = executor;
    if (e->op != OP_ADA_LAYERNORM_QUANT) {
        delete e;
        return fail(DQ_ERR_PARAM,
                    "executor was not made by dq_ada_layernorm_quant_get_workspace_size");
    }
    dq::AdaPlan p = e->ada;
    delete e;
    if (p.B * p.S == 0)
        return ok();
    hipError_t err = dq::launch_ada_layernorm_quant(p, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "ada_layernorm_quant launch failed: %s", hipGetErrorString(err));
    return ok();
}

// ---------------------------------------------------------------------------
// AntiQuantize
// ---------------------------------------------------------------------------
dq_status dq_antiquantize_get_workspace_size(const dq_tensor* src, const dq_tensor* scale,
                                             const dq_tensor* offset, int32_t policy,
                                             int32_t k_dim, uint32_t group_size,
                                             const dq_tensor* dst, size_t* workspace_size,
                                             dq_executor** executor)
{
    if (!workspace_size || !executor)
        return fail(DQ_ERR_NULLPTR, "workspace_size and executor must not be NULL");
    *executor = nullptr;
    *workspace_size = 0;
    dq_status st;
    int64_t nsrc = 0, ndst = 0;
    if ((st = check_tensor(src, "src", &nsrc)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(scale, "scale", nullptr)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(dst, "dst", &ndst)) != DQ_SUCCESS) return st;
    if (offset && (st = check_tensor(offset, "offset", nullptr)) != DQ_SUCCESS) return st;

    const bool fp4 = src->dtype == DQ_F4E2M1;
    if (src->dtype != DQ_I8 && src->dtype != DQ_F8E4M3 && src->dtype != DQ_F8E5M2 && !fp4)
        return fail(DQ_ERR_DTYPE, "src must be I8, F8E4M3, F8E5M2 or F4E2M1, got %s", dtype_name(src->dtype));
    if (dst->dtype != DQ_BF16 && dst->dtype != DQ_F16 && (dst->dtype != DQ_F32 || fp4))
        return fail(DQ_ERR_DTYPE, "dst must be BF16 or F16%s, got %s", fp4 ? " for an F4E2M1 source" : " or F32",
                    dtype_name(dst->dtype));
    if (fp4 ? scale->dtype != DQ_E8M0
            : (scale->dtype != DQ_F32 && scale->dtype != DQ_F16 && scale->dtype != DQ_BF16))
        return fail(DQ_ERR_DTYPE, "scale must be %s, got %s", fp4 ? "E8M0 for an F4E2M1 source" : "F32, F16 or BF16",
                    dtype_name(scale->dtype));
    if (offset && (fp4 || offset->dtype != scale->dtype))
        return fail(DQ_ERR_DTYPE, fp4 ? "an F4E2M1 source takes no offset" : "offset must have the scale's dtype");
    if (src->ndim != 2)
        return fail(DQ_ERR_SHAPE, "src must be 2-D [m, n] (got %d dims)", src->ndim);
    const int64_t m = src->dims[0], n = src->dims[1];
    if (fp4 && n % 2 != 0)
        return fail(DQ_ERR_SHAPE, "an F4E2M1 source needs an even n, got %lld", (long long)n);
    if (m > dq::kMaxGridBlocks)
        return fail(DQ_ERR_SHAPE, "at most %lld rows are supported, got %lld", (long long)dq::kMaxGridBlocks,
                    (long long)m);
    if (!same_dims(dst, src->dims, 2))
        return fail(DQ_ERR_SHAPE, "dst must have the shape of src");
    if (policy < DQ_PER_TENSOR || policy > DQ_PER_GROUP)
        return fail(DQ_ERR_PARAM, "unknown policy %d", (int)policy);
    if (fp4 && policy != DQ_PER_GROUP)
        return fail(DQ_ERR_PARAM, "an F4E2M1 source supports PER_GROUP only");
    if (policy == DQ_PER_GROUP) {
        if (k_dim != 0 && k_dim != 1)
            return fail(DQ_ERR_PARAM, "k_dim must be 0 or 1 for PER_GROUP, got %d", k_dim);
        if (group_size == 0 || group_size % 32 != 0)
            return fail(DQ_ERR_PARAM, "group_size must be > 0 and a multiple of 32, got %u",
                        group_size);
    }
    bool shape_good = false;
    const int64_t gs = group_size;
    switch (policy) {
    case DQ_PER_TENSOR:
        shape_good = is_shape(scale, {1}) || scale->ndim == 0 || is_shape(scale, {1, 1});
        break;
    case DQ_PER_CHANNEL:
        shape_good = is_shape(scale, {1, n}) || is_shape(scale, {n});
        break;
    case DQ_PER_TOKEN:
        shape_good = is_shape(scale, {m, 1}) || is_shape(scale, {m});
        break;
    case DQ_PER_GROUP:
        shape_good = k_dim == 1 ? is_shape(scale, {m, (n + gs - 1) / gs})
                                : is_shape(scale, {(m + gs - 1) / gs, n});
        break;
    }
    if (!shape_good)
        return fail(DQ_ERR_SHAPE, "scale shape does not match the policy");
    if (offset) {
        if (offset->ndim != scale->ndim || !same_dims(offset, scale->dims, scale->ndim))
            return fail(DQ_ERR_SHAPE, "offset must have the shape of scale");
    }
    // 32-byte rule on the contiguous (n) direction for src and dst.
    if ((n * elem_bytes_x16(src->dtype) / 2) % 32 != 0 || (n * elem_bytes_x16(dst->dtype) / 2) % 32 != 0)
        return fail(DQ_ERR_ALIGN, "n * sizeof(src) and n * sizeof(dst) must be multiples of 32 bytes (n = %lld)",
                    (long long)n);
    if (nsrc > 0) {
        if (!aligned(src->data, 16) || !aligned(dst->data, 16))
            return fail(DQ_ERR_ALIGN, "src and dst must be 16-byte aligned");
        const bool vec_params = policy == DQ_PER_CHANNEL || (policy == DQ_PER_GROUP && k_dim == 0);
        const uintptr_t pa = fp4 ? 8 : 16;
        if (vec_params && (!aligned(scale->data, pa) || (offset && !aligned(offset->data, pa))))
            return fail(DQ_ERR_ALIGN, "scale/offset must be %d-byte aligned for this policy", (int)pa);
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(src->data);
        const uintptr_t s1 = s0 + static_cast<uintptr_t>(nsrc * elem_bytes_x16(src->dtype) / 2);
        const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst->data);
        const uintptr_t d1 = d0 + static_cast<uintptr_t>(ndst * elem_bytes_x16(dst->dtype) / 2);
        if (s0 < d1 && d0 < s1)
            return fail(DQ_ERR_OVERLAP, "src and dst overlap");
        if (!scale->data || (offset && !offset->data))
            return fail(DQ_ERR_NULLPTR, "scale/offset data is NULL");
    }

    dq_executor* e = new_executor(OP_ANTIQUANTIZE);
    if (!e)
        return fail(DQ_ERR_RUNTIME, "out of host memory");
    dq::AqPlan& p = e->aq;
    p.src = src->data;
    p.scale = scale->data;
    p.offset = offset ? offset->data : nullptr;
    p.param_kind = scale->dtype == DQ_F16 ? dq::PARAM_F16 : scale->dtype == DQ_BF16 ? dq::PARAM_BF16
                 : scale->dtype == DQ_E8M0 ? dq::PARAM_E8M0 : dq::PARAM_F32;
    p.m = m;
    p.n = n;
    p.policy = policy;
    p.k_dim = policy == DQ_PER_GROUP ? k_dim : 1;
    p.group_size = policy == DQ_PER_GROUP ? gs : 0;
    p.src_kind = src->dtype == DQ_I8 ? dq::SRC_I8 : src->dtype == DQ_F8E4M3 ? dq::SRC_F8E4M3
               : src->dtype == DQ_F8E5M2 ? dq::SRC_F8E5M2 : dq::SRC_F4E2M1;
    p.dst_kind = dst->dtype == DQ_BF16 ? dq::DST_BF16 : dst->dtype == DQ_F16 ? dq::DST_F16 : dq::DST_F32;
    p.dst = dst->data;
    *executor = e;
    return ok();
}

dq_status dq_antiquantize(void* workspace, size_t workspace_size, dq_executor* executor,
                          hipStream_t stream)
{
    (void)workspace;
    (void)workspace_size;
    if (!executor)
        return fail(DQ_ERR_NULLPTR, "executor is NULL");
    dq_executor* e = executor;
    if (e->op != OP_ANTIQUANTIZE) {
        delete e;
        return fail(DQ_ERR_PARAM, "executor was not made by dq_antiquantize_get_workspace_size");
    }
    dq::AqPlan p = e->aq;
    delete e;
    if (p.m == 0)
        return ok();
    hipError_t err = dq::launch_antiquantize(p, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "antiquantize launch failed: %s", hipGetErrorString(err));
    return ok();
}

// ---------------------------------------------------------------------------
// mx block quantization
// ---------------------------------------------------------------------------
dq_status dq_mx_quantize_get_workspace_size(const dq_tensor* x, int32_t axis, const dq_tensor* y,
                                            const dq_tensor* scale, size_t* workspace_size,
                                            dq_executor** executor)
{
    if (!workspace_size || !executor)
        return fail(DQ_ERR_NULLPTR, "workspace_size and executor must not be NULL");
    *executor = nullptr;
    *workspace_size = 0;
    dq_status st;
    int64_t nx = 0, ny = 0, ns = 0;
    if ((st = check_tensor(x, "x", &nx)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(y, "y", &ny)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(scale, "scale", &ns)) != DQ_SUCCESS) return st;
    if (x->dtype != DQ_F16 && x->dtype != DQ_BF16)
        return fail(DQ_ERR_DTYPE, "x must be F16 or BF16, got %s", dtype_name(x->dtype));
    if (y->dtype != DQ_F8E4M3 && y->dtype != DQ_F8E5M2 && y->dtype != DQ_F4E2M1)
        return fail(DQ_ERR_DTYPE, "y must be F8E4M3, F8E5M2 or F4E2M1, got %s", dtype_name(y->dtype));
    if (scale->dtype != DQ_E8M0)
        return fail(DQ_ERR_DTYPE, "scale must be E8M0, got %s", dtype_name(scale->dtype));
    if (axis != 0 && axis != 1)
        return fail(DQ_ERR_PARAM, "axis must be 0 or 1, got %d", axis);
    if (x->ndim != 2)
        return fail(DQ_ERR_SHAPE, "x must be 2-D [rows, n], got ndim %d", x->ndim);
    const int64_t rows = x->dims[0], n = x->dims[1];
    if (n < 1 || n > dq::kMaxGridBlocks)
        return fail(DQ_ERR_SHAPE, "the last dimension of x must be in [1, 2^31 - 1], got %lld", (long long)n);
    const bool fp4 = y->dtype == DQ_F4E2M1;
    if (fp4 && n % 2 != 0)
        return fail(DQ_ERR_SHAPE, "F4E2M1 codes need an even last dimension, got %lld", (long long)n);
    if (!same_dims(y, x->dims, 2))
        return fail(DQ_ERR_SHAPE, "y must have the shape of x");
    const int64_t blk = 32;
    const bool scale_ok = axis == 1 ? is_shape(scale, {rows, (n + blk - 1) / blk})
                                    : is_shape(scale, {(rows + blk - 1) / blk, n});
    if (!scale_ok)
        return fail(DQ_ERR_SHAPE, axis == 1 ? "scale must be [rows, ceil(n/32)]" : "scale must be [ceil(rows/32), n]");

    if (nx > 0) {
        const uintptr_t x0 = reinterpret_cast<uintptr_t>(x->data), x1 = x0 + static_cast<uintptr_t>(nx) * 2;
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(y->data);
        const uintptr_t y1 = y0 + static_cast<uintptr_t>(fp4 ? nx / 2 : nx);
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(scale->data), s1 = s0 + static_cast<uintptr_t>(ns);
        if ((x0 < y1 && y0 < x1) || (x0 < s1 && s0 < x1) || (y0 < s1 && s0 < y1))
            return fail(DQ_ERR_OVERLAP, "x, y and scale must not overlap");
    }

    dq_executor* e = new_executor(OP_MX_QUANTIZE);
    if (!e)
        return fail(DQ_ERR_RUNTIME, "out of host memory");
    dq::MxPlan& p = e->mx;
    p.x = x->data;
    p.x_type = x->dtype == DQ_BF16 ? dq::X_BF16 : dq::X_F16;
    p.rows = rows;
    p.n = n;
    p.elem = y->dtype == DQ_F8E4M3 ? dq::MX_E4M3 : y->dtype == DQ_F8E5M2 ? dq::MX_E5M2 : dq::MX_E2M1;
    p.axis = axis;
    p.y = y->data;
    p.scale = static_cast<uint8_t*>(scale->data);
    const bool vec = n % 8 == 0 && aligned(x->data, 16) && aligned(y->data, fp4 ? 4 : 8);
    if (vec && axis == 1)
        p.variant = dq::MX_VAR_ROW;
    else if (vec && aligned(scale->data, 8))
        p.variant = dq::MX_VAR_COL;
    else
        p.variant = dq::MX_VAR_GENERIC;
    *executor = e;
    return ok();
}

dq_status dq_mx_quantize(void* workspace, size_t workspace_size, dq_executor* executor, hipStream_t stream)
{
    (void)workspace;
    (void)workspace_size;
    if (!executor)
        return fail(DQ_ERR_NULLPTR, "executor is NULL");
    dq_executor* e = executor;
    if (e->op != OP_MX_QUANTIZE) {
        delete e;
        return fail(DQ_ERR_PARAM, "executor was not made by dq_mx_quantize_get_workspace_size");
    }
    dq::MxPlan p = e->mx;
    delete e;
    if (p.rows == 0)
        return ok();
    hipError_t err = dq::launch_mx_quantize(p, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "mx quantize launch failed: %s", hipGetErrorString(err));
    return ok();
}

// ---------------------------------------------------------------------------
// Weight-quantized matmul
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// Validation and launch plan of the weight-quantized matmul, shared by the
// two-phase pair and the allocation-free entry point.  Host only; writes
// the plan and the split-k workspace size (0 when k is not split).
dq_status plan_weight_quant_matmul(const dq_tensor* x1, const dq_tensor* x2, int32_t transpose_x2,
                                   const dq_tensor* antiquant_scale, const dq_tensor* antiquant_offset,
                                   int64_t group_size, const dq_tensor* bias, const dq_tensor* x3,
                                   const dq_tensor* out, dq::WqPlan& p, size_t* workspace_size)
{
    *workspace_size = 0;
    dq_status st;
    int64_t nx1 = 0, nx2 = 0, ns = 0, no = 0;
    if ((st = check_tensor(x1, "x1", &nx1)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(x2, "x2", &nx2)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(antiquant_scale, "antiquant_scale", &ns)) != DQ_SUCCESS) return st;
    if ((st = check_tensor(out, "out", &no)) != DQ_SUCCESS) return st;
    const int32_t T = x1->dtype;
    if (T != DQ_F16 && T != DQ_BF16)
        return fail(DQ_ERR_DTYPE, "x1 must be F16 or BF16, got %s", dtype_name(T));
    if (x2->dtype != DQ_I8 && x2->dtype != DQ_I4)
        return fail(DQ_ERR_DTYPE, "x2 must be I8 or I4, got %s", dtype_name(x2->dtype));
    if (antiquant_scale->dtype != T || out->dtype != T)
        return fail(DQ_ERR_DTYPE, "antiquant_scale and out must have x1's dtype %s", dtype_name(T));
    if (x1->ndim != 2 && x1->ndim != 3)
        return fail(DQ_ERR_SHAPE, "x1 must be [m, k] or [b, s, k], got ndim %d", x1->ndim);
    if (x2->ndim != 2)
        return fail(DQ_ERR_SHAPE, "x2 must be 2-D, got ndim %d", x2->ndim);
    const int64_t k = x1->dims[x1->ndim - 1];
    const int64_t m = k > 0 ? nx1 / k : [&] { int64_t r = 1; for (int i = 0; i + 1 < x1->ndim; ++i) r *= x1->dims[i]; return r; }();
    const int64_t xk = transpose_x2 ? x2->dims[1] : x2->dims[0];
    const int64_t n = transpose_x2 ? x2->dims[0] : x2->dims[1];
    if (xk != k)
        return fail(DQ_ERR_SHAPE, "x1 and x2 disagree on k (%lld vs %lld)", (long long)k, (long long)xk);
    if (k > 65535 || n < 1 || n > 65535)
        return fail(DQ_ERR_SHAPE, "k must be in [0, 65535] and n in [1, 65535] (k %lld, n %lld)", (long long)k,
                    (long long)n);
    if (m > dq::kMaxGridBlocks)
        return fail(DQ_ERR_SHAPE, "at most 2^31 - 1 rows of x1 are supported");
    if (x2->dtype == DQ_I4 && x2->dims[1] % 2 != 0)
        return fail(DQ_ERR_SHAPE, "I4 weights need an even stored last dimension");
    int64_t want[DQ_MAX_DIMS];
    std::memcpy(want, x1->dims, sizeof want);
    want[x1->ndim - 1] = n;
    if (!same_dims(out, want, x1->ndim))
        return fail(DQ_ERR_SHAPE, "out must be x1.shape[:-1] + [n]");
    if (group_size < 0 || group_size % 32 != 0)
        return fail(DQ_ERR_PARAM, "group_size must be 0 or a positive multiple of 32, got %lld", (long long)group_size);
    int policy;
    if (group_size > 0) {
        policy = DQ_PER_GROUP;
        const int64_t G = k > 0 ? (k - 1) / group_size + 1 : 0;  // ceil, without k + group_size overflowing
        if (!(transpose_x2 ? is_shape(antiquant_scale, {n, G}) : is_shape(antiquant_scale, {G, n})))
            return fail(DQ_ERR_SHAPE, transpose_x2 ? "per-group scale must be [n, ceil(k/gs)]"
                                                   : "per-group scale must be [ceil(k/gs), n]");
    } else if (ns == 1 && (antiquant_scale->ndim == 1 || (antiquant_scale->ndim == 2 && n == 1))) {
        policy = DQ_PER_TENSOR;
    } else if (is_shape(antiquant_scale, {n}) || is_shape(antiquant_scale, {1, n})) {
        policy = DQ_PER_CHANNEL;
    } else {
        return fail(DQ_ERR_SHAPE, "antiquant_scale must be [1], [n] or [1, n] without a group size");
    }
    if (antiquant_offset) {
        int64_t nof = 0;
        if ((st = check_tensor(antiquant_offset, "antiquant_offset", &nof)) != DQ_SUCCESS) return st;
        if (antiquant_offset->dtype != T)
            return fail(DQ_ERR_DTYPE, "antiquant_offset must have x1's dtype");
        if (!same_dims(antiquant_offset, antiquant_scale->dims, antiquant_scale->ndim))
            return fail(DQ_ERR_SHAPE, "antiquant_offset must have the scale's shape");
    }
    if (bias) {
        int64_t nb = 0;
        if ((st = check_tensor(bias, "bias", &nb)) != DQ_SUCCESS) return st;
        if (bias->dtype != T)
            return fail(DQ_ERR_DTYPE, "bias must have x1's dtype");
        if (!is_shape(bias, {n}))
            return fail(DQ_ERR_SHAPE, "bias must be [n]");
    }
    if (x3) {
        int64_t n3 = 0;
        if ((st = check_tensor(x3, "x3", &n3)) != DQ_SUCCESS) return st;
        if (x3->dtype != T)
            return fail(DQ_ERR_DTYPE, "x3 must have x1's dtype");
        if (!same_dims(x3, want, x1->ndim))
            return fail(DQ_ERR_SHAPE, "x3 must have out's shape");
    }
    if (no > 0) {
        const uintptr_t o0 = reinterpret_cast<uintptr_t>(out->data), o1 = o0 + static_cast<uintptr_t>(no) * 2;
        auto hits = [&](const dq_tensor* t, int64_t bytes) {
            if (!t || bytes <= 0)
                return false;
            const uintptr_t t0 = reinterpret_cast<uintptr_t>(t->data), t1 = t0 + static_cast<uintptr_t>(bytes);
            return t0 < o1 && o0 < t1;
        };
        const int64_t w_bytes = x2->dtype == DQ_I4 ? nx2 / 2 : nx2;
        if (hits(x1, nx1 * 2) || hits(x2, w_bytes) || hits(antiquant_scale, ns * 2) ||
            hits(antiquant_offset, antiquant_offset ? ns * 2 : 0) || hits(bias, bias ? n * 2 : 0) ||
            hits(x3, x3 ? no * 2 : 0))
            return fail(DQ_ERR_OVERLAP, "out overlaps an input");
    }

    p = dq::WqPlan{};
    p.x1 = x1->data;
    p.x2 = x2->data;
    p.scale = antiquant_scale->data;
    p.offset = antiquant_offset ? antiquant_offset->data : nullptr;
    p.bias = bias ? bias->data : nullptr;
    p.x3 = x3 ? x3->data : nullptr;
    p.out = out->data;
    p.m = m;
    p.k = k;
    p.n = n;
    p.group_size = group_size;
    p.x_type = T == DQ_BF16 ? dq::X_BF16 : dq::X_F16;
    p.w_type = x2->dtype == DQ_I8 ? dq::WQ_I8 : dq::WQ_I4;
    p.policy = policy;
    p.transpose_x2 = transpose_x2 != 0;
    const bool kfit = x2->dtype == DQ_I8 ? k % 32 == 0 : k % 64 == 0;
    p.variant = p.transpose_x2 && kfit && aligned(x1->data, 16) && aligned(x2->data, 16) ? dq::WQ_VAR_MFMA
                                                                                       : dq::WQ_VAR_GENERIC;
    p.tile = m <= 16 ? dq::WQ_TILE_DECODE : dq::WQ_TILE_GEMM;
    if (p.variant == dq::WQ_VAR_MFMA && m >= dq::kWqWideRows && k % (2 * dq::kWqWideK) == 0 &&
        (policy != DQ_PER_GROUP || group_size % dq::kWqWideK == 0)) {
        const int64_t wide_tiles = ((n + dq::kWqWideCols - 1) / dq::kWqWideCols) *
                                   ((m + dq::kWqWideRows - 1) / dq::kWqWideRows);
        const int64_t groups = policy == DQ_PER_GROUP ? k / group_size : 1;
        const int64_t kw = x2->dtype == DQ_I4 ? k / 2 : k;  // weight bytes per column
        if (wide_tiles >= dq::kWqWideMinTiles && n * groups < (int64_t{1} << 31) &&
            int64_t{dq::kWqWideRows} * k * 2 < (int64_t{1} << 31) && int64_t{dq::kWqWideCols} * kw < (int64_t{1} << 31))
            p.tile = dq::WQ_TILE_WIDE;
    }
    // Decode shapes whose n / 16 column blocks divide evenly over the 256
    // compute units (int4 in groups of 128, k in whole 8 x 256 runs): the
    // balanced kernel, one workgroup per compute unit, no k split.
    if (p.variant == dq::WQ_VAR_MFMA && p.tile == dq::WQ_TILE_DECODE && x2->dtype == DQ_I4 && k > 0 &&
        policy == DQ_PER_GROUP && group_size == dq::kWqSuperK && k % dq::kWqBalKMultiple == 0 &&
        n % (16 * dq::kWqBalWorkgroups) == 0 && n / (16 * dq::kWqBalWorkgroups) <= dq::kWqBalMaxBlocks &&
        n * (k / 2) < (int64_t{1} << 31) && n * (k / group_size) * 2 < (int64_t{1} << 31))
        p.tile = dq::WQ_TILE_BALANCED;
    // Few output tiles: split k so that about the target number of
    // workgroups run; the binary32 partial sums [splits, m, n] live in the
    // workspace.
    p.splits = 1;
    p.k_chunk = k;
    if (p.variant == dq::WQ_VAR_MFMA && m > 0 && p.tile != dq::WQ_TILE_WIDE &&
        p.tile != dq::WQ_TILE_BALANCED) {  // m == 0 launches nothing
        const int64_t tiles = ((n + dq::wq_tile_cols(p.tile) - 1) / dq::wq_tile_cols(p.tile)) *
                              ((m + dq::wq_tile_rows(p.tile) - 1) / dq::wq_tile_rows(p.tile));
        const int64_t batch_k = static_cast<int64_t>(dq::wq_batch(p.tile, p.w_type)) * dq::kWqSuperK;
        const int64_t batches = (k + batch_k - 1) / batch_k;
        const int64_t target = p.tile == dq::WQ_TILE_DECODE ? kWqTargetBlocks : kWqGemmTargetBlocks;
        int64_t want = tiles < target ? (target + tiles - 1) / tiles : 1;
        want = want < batches ? want : batches;
        if (want > 1) {
            p.k_chunk = ((batches + want - 1) / want) * batch_k;
            // Keep whole parameter windows per split where the kernel uses them.
            const int64_t window = static_cast<int64_t>(dq::kWqParamWindow) * dq::kWqGemmK;
            if (p.tile == dq::WQ_TILE_GEMM && policy == DQ_PER_GROUP && group_size == dq::kWqGemmK)
                p.k_chunk = (p.k_chunk + window - 1) / window * window;
            p.splits = static_cast<int>((k + p.k_chunk - 1) / p.k_chunk);
        }
        if (p.splits > 1)
            *workspace_size = static_cast<size_t>(p.splits) * static_cast<size_t>(m) * static_cast<size_t>(n) * 4;
    }
    return DQ_SUCCESS;
}

}  // namespace

extern "C" {

dq_status dq_weight_quant_matmul_get_workspace_size(const dq_tensor* x1, const dq_tensor* x2,
                                                    int32_t transpose_x2,
                                                    const dq_tensor* antiquant_scale,
                                                    const dq_tensor* antiquant_offset,
                                                    int64_t group_size, const dq_tensor* bias,
                                                    const dq_tensor* x3, const dq_tensor* out,
                                                    size_t* workspace_size, dq_executor** executor)
{
    if (!workspace_size || !executor)
        return fail(DQ_ERR_NULLPTR, "workspace_size and executor must not be NULL");
    *executor = nullptr;
    *workspace_size = 0;
    dq::WqPlan plan;
    size_t ws = 0;
    const dq_status st = plan_weight_quant_matmul(x1, x2, transpose_x2, antiquant_scale, antiquant_offset,
                                                  group_size, bias, x3, out, plan, &ws);
    if (st != DQ_SUCCESS)
        return st;
    dq_executor* e = new_executor(OP_WEIGHT_QUANT_MATMUL);
    if (!e)
        return fail(DQ_ERR_RUNTIME, "out of host memory");
    e->wq = plan;
    *workspace_size = ws;
    *executor = e;
    return ok();
}

dq_status dq_weight_quant_matmul(void* workspace, size_t workspace_size, dq_executor* executor,
                                 hipStream_t stream)
{
    if (!executor)
        return fail(DQ_ERR_NULLPTR, "executor is NULL");
    dq_executor* e = executor;
    if (e->op != OP_WEIGHT_QUANT_MATMUL) {
        delete e;
        return fail(DQ_ERR_PARAM, "executor was not made by dq_weight_quant_matmul_get_workspace_size");
    }
    dq::WqPlan p = e->wq;
    delete e;
    if (p.m == 0)
        return ok();
    if (p.splits > 1) {
        const size_t need = static_cast<size_t>(p.splits) * static_cast<size_t>(p.m) * static_cast<size_t>(p.n) * 4;
        if (!workspace || workspace_size < need)
            return fail(DQ_ERR_WORKSPACE, "the workspace must hold %zu bytes, got %zu", need, workspace_size);
        if (!aligned(workspace, 16))
            return fail(DQ_ERR_ALIGN, "the workspace must be 16-byte aligned");
    }
    hipError_t err = dq::launch_weight_quant_matmul(p, workspace, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "weight quant matmul launch failed: %s", hipGetErrorString(err));
    return ok();
}

dq_status dq_weight_quant_matmul_noalloc(const dq_tensor* x1, const dq_tensor* x2, int32_t transpose_x2,
                                         const dq_tensor* antiquant_scale, const dq_tensor* antiquant_offset,
                                         int64_t group_size, const dq_tensor* bias, const dq_tensor* x3,
                                         const dq_tensor* out, hipStream_t stream)
{
    dq::WqPlan p;
    size_t ws = 0;
    const dq_status st = plan_weight_quant_matmul(x1, x2, transpose_x2, antiquant_scale, antiquant_offset,
                                                  group_size, bias, x3, out, p, &ws);
    if (st != DQ_SUCCESS)
        return st;
    if (ws > dq::kWqScratchBytes)
        return fail(DQ_ERR_WORKSPACE,
                    "the split-k partial sums need %zu bytes, more than the library's %zu-byte scratch; "
                    "call dq_weight_quant_matmul with a workspace instead", ws, dq::kWqScratchBytes);
    if (p.m == 0)
        return ok();
    void* scr = nullptr;
    if (ws > 0) {
        int cur = -1, sdev = -1;
        hipError_t err = hipGetDevice(&cur);
        if (err == hipSuccess)
            err = hipStreamGetDevice(stream, &sdev);
        if (err != hipSuccess)
            return fail(DQ_ERR_RUNTIME, "cannot query the current device: %s", hipGetErrorString(err));
        if (cur != sdev)
            return fail(DQ_ERR_PARAM, "the stream's device (%d) must be the current device (%d)", sdev, cur);
        err = dq::wq_scratch_address(&scr);
        if (err != hipSuccess)
            return fail(DQ_ERR_RUNTIME, "cannot locate the scratch array on device %d: %s", cur,
                        hipGetErrorString(err));
    }
    hipError_t err = dq::launch_weight_quant_matmul(p, scr, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "weight quant matmul launch failed: %s", hipGetErrorString(err));
    return ok();
}

// ---------------------------------------------------------------------------
// Copy probe
// ---------------------------------------------------------------------------
dq_status dq_copy_probe(void* dst, const void* src, size_t bytes, hipStream_t stream)
{
    if (bytes == 0)
        return ok();
    if (!dst || !src)
        return fail(DQ_ERR_NULLPTR, "dst/src is NULL");
    if (bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16))
        return fail(DQ_ERR_ALIGN, "copy probe needs 16-byte aligned pointers and size");
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes)
        return fail(DQ_ERR_OVERLAP, "copy probe buffers overlap");
    hipError_t err = dq::launch_copy_probe(dst, src, bytes, stream);
    if (err != hipSuccess)
        return fail(DQ_ERR_RUNTIME, "copy probe launch failed: %s", hipGetErrorString(err));
    return ok();
}

}  // extern "C"
