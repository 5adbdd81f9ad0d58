// dynamic_quant.hip -- per-token dynamic quantization on gfx950
// (aclnnDynamicQuantV2, Description and Formula).
//
// Vector variant: each row is owned by TEAM waves (1 or 4).  Lane l of
// wave w loads the 16-byte vectors k = (i*TEAM + w)*64 + l, i < VPL, so
// every load instruction covers TEAM*1 KiB of contiguous row; the row stays
// in VGPRs as fp32 (after the smooth multiply), is reduced through DPP
// (and LDS across the team), then quantized and stored from the same
// registers: one HBM read per input element and one write per code.
//
// Generic variant (rows with N % 8 != 0, unaligned buffers, or rows longer
// than 4 waves x 16 vectors): one workgroup per row, element loads, the row
// read twice (reduce, then quantize).
//
// Arithmetic: every formula step is one correctly rounded binary32
// operation in the printed order (no contraction: built with
// -ffp-contract=off); division by the row scale uses the per-row
// correctly rounded reciprocal plus Markstein's fma correction, which
// returns the IEEE quotient for the divisors it is used with.

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

struct DqArgs {
    const void* x;
    const float* smooth;
    const int32_t* gi;
    int64_t n_experts;
    int64_t rows;
    int64_t n;
    void* y;
    float* scale;
    float* offset;
    int64_t nblocks;
};

// (D or scale_opt, offset_opt, code range) per output type, from the
// Formula section: INT8 -> (255, 127); INT4 / INT32 -> (15, 7); the
// symmetric divisor is offset_opt.
template <int OUT>
struct Consts;
template <>
struct Consts<OUT_I8> {
    static constexpr float scale_opt = 255.0f, offset_opt = 127.0f, lo = -128.0f, hi = 127.0f;
};
template <>
struct Consts<OUT_I4> {
    static constexpr float scale_opt = 15.0f, offset_opt = 7.0f, lo = -8.0f, hi = 7.0f;
};

// First expert e with row < gi[e]; the last expert when there is none.
// Lanes test 64 experts at a time and a ballot picks the first hit, so the
// result is wave-uniform.
__device__ __forceinline__ int64_t expert_of_row(int64_t row, const int32_t* gi, int64_t n_experts,
                                                 int lane)
{
    for (int64_t base = 0; base < n_experts; base += kWave) {
        const int64_t e = base + lane;
        const bool hit = e < n_experts && row < static_cast<int64_t>(gi[e]);
        const unsigned long long mask = __ballot(hit);
        if (mask)
            return base + __builtin_ctzll(mask);
    }
    return n_experts - 1;
}

// Row parameters from the reduced statistics (Formula):
//   symmetric:  scale = max|in| / offset_opt
//   asymmetric: scale = (max - min) / scale_opt, offset = offset_opt - max / scale
template <bool SYM, int OUT>
struct RowParams {
    float scale, offset, recip;
    bool fast;
    __device__ __forceinline__ RowParams(float a_hi, float a_lo)
    {
        using C = Consts<OUT>;
        if (SYM) {
            scale = a_hi / C::offset_opt;
            offset = 0.0f;
        } else {
            const float range = a_hi - a_lo;
            scale = range / C::scale_opt;
            const float q_hi = a_hi / scale;
            offset = C::offset_opt - q_hi;
        }
        fast = row_divisor_in_range(scale);
        recip = 1.0f / scale;
    }
};

// One code: sat(rne(RN(v / scale))) or sat(rne(RN(RN(v / scale) + offset))),
// returned as the encoding of t + 1.5*2^23 (its low bits are the code).
template <bool SYM, int OUT, bool FAST>
__device__ __forceinline__ uint32_t quant_code(float v, const RowParams<SYM, OUT>& rp)
{
    using C = Consts<OUT>;
    float t;
    if (FAST) {
        t = div_by_row(v, rp.scale, rp.recip);
        if (!SYM) {
            t = t + rp.offset;
            t = __builtin_amdgcn_fmed3f(t, C::lo, C::hi);
        }
        // Symmetric codes never leave [-offset_opt, offset_opt]: |v| <= max|v|
        // and scale = RN(max|v| / offset_opt) bound the quotient by
        // offset_opt * (1 + 2^-23) before rounding.
    } else {
        t = v / rp.scale;
        if (!SYM)
            t = t + rp.offset;
        if (t != t)
            t = 0.0f;  // NaN -> 0 (0/0 of an all-zero or constant row)
        t = __builtin_amdgcn_fmed3f(t, C::lo, C::hi);
    }
    return code_bits(t);
}

template <int OUT>
__device__ __forceinline__ void store_codes(void* y, int64_t row, int64_t n, int64_t k,
                                            const uint32_t (&c)[8])
{
    if (OUT == OUT_I8) {
        uint2* dst = reinterpret_cast<uint2*>(static_cast<int8_t*>(y) + row * n) + k;
        *dst = make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7]));
    } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(y) + row * (n >> 1)) + k;
        *dst = pack8_i4(c);
    }
}

template <int XT, bool SYM, int OUT, int VPL, int TEAM>
__global__ __launch_bounds__(kBlock) void dq_vec_kernel(DqArgs a)
{
    constexpr int RPB = 4 / TEAM;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wit = wave % TEAM;
    const int64_t row = xcd_block(blockIdx.x, a.nblocks) * RPB + wave / TEAM;
    if (row >= a.rows)
        return;  // wave-uniform; with TEAM = 4 the whole block leaves together

    const int64_t nvec = a.n >> 3;
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + row * a.n);
    uint4 raw[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int64_t k = static_cast<int64_t>(i * TEAM + wit) * kWave + lane;
        raw[i] = k < nvec ? xr[k] : make_uint4(0, 0, 0, 0);
    }

    const float4* sr = nullptr;
    if (a.smooth) {
        const int64_t e = a.gi ? expert_of_row(row, a.gi, a.n_experts, lane) : 0;
        sr = reinterpret_cast<const float4*>(a.smooth + e * a.n);
    }

    float v[VPL][8];
    float s_hi = SYM ? 0.0f : -__builtin_huge_valf();
    float s_lo = __builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int64_t k = static_cast<int64_t>(i * TEAM + wit) * kWave + lane;
        widen8<XT>(raw[i], v[i]);
        if (k < nvec) {
            if (sr) {
                const float4 s0 = sr[2 * k], s1 = sr[2 * k + 1];
                v[i][0] = v[i][0] * s0.x;
                v[i][1] = v[i][1] * s0.y;
                v[i][2] = v[i][2] * s0.z;
                v[i][3] = v[i][3] * s0.w;
                v[i][4] = v[i][4] * s1.x;
                v[i][5] = v[i][5] * s1.y;
                v[i][6] = v[i][6] * s1.z;
                v[i][7] = v[i][7] * s1.w;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (SYM) {
                    s_hi = __builtin_fmaxf(s_hi, __builtin_fabsf(v[i][j]));
                } else {
                    s_hi = __builtin_fmaxf(s_hi, v[i][j]);
                    s_lo = __builtin_fminf(s_lo, v[i][j]);
                }
            }
        }
    }

    s_hi = wave_max(s_hi);
    if (!SYM)
        s_lo = wave_min(s_lo);
    if (TEAM > 1) {
        __shared__ float red[2][4];
        if (lane == 0) {
            red[0][wave] = s_hi;
            red[1][wave] = s_lo;
        }
        __syncthreads();
        s_hi = red[0][0];
        s_lo = red[1][0];
#pragma unroll
        for (int w = 1; w < TEAM; ++w) {
            s_hi = __builtin_fmaxf(s_hi, red[0][w]);
            s_lo = __builtin_fminf(s_lo, red[1][w]);
        }
    }

    const RowParams<SYM, OUT> rp(s_hi, s_lo);
    if (wit == 0 && lane == 0) {
        a.scale[row] = rp.scale;
        if (!SYM)
            a.offset[row] = rp.offset;
    }

    if (rp.fast) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t k = static_cast<int64_t>(i * TEAM + wit) * kWave + lane;
            if (k < nvec) {
                uint32_t c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    c[j] = quant_code<SYM, OUT, true>(v[i][j], rp);
                store_codes<OUT>(a.y, row, a.n, k, c);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t k = static_cast<int64_t>(i * TEAM + wit) * kWave + lane;
            if (k < nvec) {
                uint32_t c[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    c[j] = quant_code<SYM, OUT, false>(v[i][j], rp);
                store_codes<OUT>(a.y, row, a.n, k, c);
            }
        }
    }
}

// Generic variant: one workgroup per row, any N, any alignment.
template <int XT, bool SYM, int OUT>
__device__ __forceinline__ float load_in(const uint16_t* xr, const float* srow, int64_t j)
{
    const float xv = widen1<XT>(xr[j]);
    return srow ? xv * srow[j] : xv;
}

template <int XT, bool SYM, int OUT, bool FAST>
__device__ __forceinline__ void generic_store(const DqArgs& a, const uint16_t* xr, const float* srow,
                                              int64_t row, const RowParams<SYM, OUT>& rp)
{
    if (OUT == OUT_I8) {
        int8_t* yr = static_cast<int8_t*>(a.y) + row * a.n;
        for (int64_t j = threadIdx.x; j < a.n; j += kBlock)
            yr[j] = static_cast<int8_t>(quant_code<SYM, OUT, FAST>(load_in<XT, SYM, OUT>(xr, srow, j), rp) & 0xFFu);
    } else {
        uint8_t* yr = static_cast<uint8_t*>(a.y) + row * (a.n >> 1);
        for (int64_t p = threadIdx.x; p < (a.n >> 1); p += kBlock) {
            const uint32_t c0 = quant_code<SYM, OUT, FAST>(load_in<XT, SYM, OUT>(xr, srow, 2 * p), rp);
            const uint32_t c1 = quant_code<SYM, OUT, FAST>(load_in<XT, SYM, OUT>(xr, srow, 2 * p + 1), rp);
            yr[p] = static_cast<uint8_t>((c0 & 0xFu) | ((c1 & 0xFu) << 4));
        }
    }
}

template <int XT, bool SYM, int OUT>
__global__ __launch_bounds__(kBlock) void dq_generic_kernel(DqArgs a)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t row = xcd_block(blockIdx.x, a.nblocks);
    if (row >= a.rows)
        return;
    const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * a.n;
    const float* srow = nullptr;
    if (a.smooth) {
        const int64_t e = a.gi ? expert_of_row(row, a.gi, a.n_experts, lane) : 0;
        srow = a.smooth + e * a.n;
    }
    float s_hi = SYM ? 0.0f : -__builtin_huge_valf();
    float s_lo = __builtin_huge_valf();
    for (int64_t j = threadIdx.x; j < a.n; j += kBlock) {
        const float v = load_in<XT, SYM, OUT>(xr, srow, j);
        if (SYM) {
            s_hi = __builtin_fmaxf(s_hi, __builtin_fabsf(v));
        } else {
            s_hi = __builtin_fmaxf(s_hi, v);
            s_lo = __builtin_fminf(s_lo, v);
        }
    }
    s_hi = wave_max(s_hi);
    if (!SYM)
        s_lo = wave_min(s_lo);
    __shared__ float red[2][4];
    if (lane == 0) {
        red[0][wave] = s_hi;
        red[1][wave] = s_lo;
    }
    __syncthreads();
    s_hi = __builtin_fmaxf(__builtin_fmaxf(red[0][0], red[0][1]), __builtin_fmaxf(red[0][2], red[0][3]));
    s_lo = __builtin_fminf(__builtin_fminf(red[1][0], red[1][1]), __builtin_fminf(red[1][2], red[1][3]));

    const RowParams<SYM, OUT> rp(s_hi, s_lo);
    if (threadIdx.x == 0) {
        a.scale[row] = rp.scale;
        if (!SYM)
            a.offset[row] = rp.offset;
    }
    if (rp.fast)
        generic_store<XT, SYM, OUT, true>(a, xr, srow, row, rp);
    else
        generic_store<XT, SYM, OUT, false>(a, xr, srow, row, rp);
}

using KernelFn = void (*)(DqArgs);

template <int XT, bool SYM, int OUT>
KernelFn pick_vec(int vpl, int team)
{
    if (team == 4) {
        switch (vpl) {
        case 8: return dq_vec_kernel<XT, SYM, OUT, 8, 4>;
        case 16: return dq_vec_kernel<XT, SYM, OUT, 16, 4>;
        }
        return nullptr;
    }
    switch (vpl) {
    case 1: return dq_vec_kernel<XT, SYM, OUT, 1, 1>;
    case 2: return dq_vec_kernel<XT, SYM, OUT, 2, 1>;
    case 4: return dq_vec_kernel<XT, SYM, OUT, 4, 1>;
    case 8: return dq_vec_kernel<XT, SYM, OUT, 8, 1>;
    case 12: return dq_vec_kernel<XT, SYM, OUT, 12, 1>;
    case 14: return dq_vec_kernel<XT, SYM, OUT, 14, 1>;
    case 16: return dq_vec_kernel<XT, SYM, OUT, 16, 1>;
    }
    return nullptr;
}

template <int XT, bool SYM, int OUT>
KernelFn pick(const DqPlan& p)
{
    if (p.variant == DQ_VAR_VECTOR)
        return pick_vec<XT, SYM, OUT>(p.vpl, p.team);
    return dq_generic_kernel<XT, SYM, OUT>;
}

template <int XT>
KernelFn pick_x(const DqPlan& p)
{
    if (p.symmetric)
        return p.out_kind == OUT_I8 ? pick<XT, true, OUT_I8>(p) : pick<XT, true, OUT_I4>(p);
    return p.out_kind == OUT_I8 ? pick<XT, false, OUT_I8>(p) : pick<XT, false, OUT_I4>(p);
}

}  // namespace

hipError_t launch_dynamic_quant(const DqPlan& p, hipStream_t stream)
{
    KernelFn fn = p.x_type == X_F16 ? pick_x<X_F16>(p) : pick_x<X_BF16>(p);
    if (!fn)
        return hipErrorInvalidValue;
    DqArgs a{p.x, p.smooth, p.group_index, p.n_experts, p.rows, p.n, p.y, p.scale, p.offset, 0};
    const int64_t rows_per_block = p.variant == DQ_VAR_VECTOR ? 4 / p.team : 1;
    a.nblocks = (p.rows + rows_per_block - 1) / rows_per_block;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(a.nblocks)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace dq
