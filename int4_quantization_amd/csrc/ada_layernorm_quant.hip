// ada_layernorm_quant.hip -- AdaLayerNorm fused with symmetric INT8
// dynamic quantization on gfx950 (aclnnAdaLayerNormQuant, Formula 1-5):
//   LN = (x - E(x)) / sqrt(Var(x) + eps) * weight + bias
//   y  = LN * (1 + scale[b]) + shift[b];   y = y * smooth
//   quantScale = row_max(|y|) / 127;      out = round(y / quantScale)
//
// Layout of the work: a workgroup owns a contiguous chunk of rows (workgroups
// in launch order, so the running ones cover one band of rows).  For each
// batch b its chunk touches, it first writes the per-column coefficients
//   A_j = w_j * (1 + scale_bj) * smooth_j
//   C_j = (bias_j * (1 + scale_bj) + shift_bj) * smooth_j
// into LDS, so that y_j = ((x_j - mean) * rstd) * A_j + C_j is one multiply
// and one fma per element.  Each row is then held in VGPRs by one wave
// (16-byte non-temporal loads, one HBM read per element); its statistics
// are Welford style: every lane forms (count, mean, M2) of its own elements
// from the registers, and the lanes merge with Chan's pairwise update in a
// fixed butterfly (a reciprocal-free form when every lane holds the same
// count).  Statistics, normalization and modulation are fp32 with hardware
// rsq / rcp; quantScale is the exact binary32 RN(max|y| / 127).
//
// Rows that are not whole 16-byte vectors or are longer than 16 vectors
// per lane use the generic kernel (one workgroup per row, three passes over
// the row from global memory, same arithmetic).

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

// Launch one workgroup per chunk of rows (false) or a persistent grid that
// sweeps the chunks and rebuilds its LDS table only when the batch changes.
constexpr bool kAdaPersistent = false;

struct AdaArgs {
    const void* x;
    const void* scale;
    const void* shift;
    const void* weight;
    const void* bias;
    const float* smooth;
    int64_t S, H, rows;
    float eps;
    int8_t* out;
    float* qs;
    int64_t rpb;
    int64_t nblocks;
    int equal_counts;  // every lane holds the same number of elements (H % 512 == 0)
    float inv_h;       // RN(1 / H)
};

// Modulation coefficients of column j for batch b (fp32, formula order).
template <int XT>
__device__ __forceinline__ void coeffs(const AdaArgs& a, int64_t b, int64_t j, float& A, float& C)
{
    const uint16_t* sc = static_cast<const uint16_t*>(a.scale);
    const uint16_t* sh = static_cast<const uint16_t*>(a.shift);
    const float w = a.weight ? widen1<XT>(static_cast<const uint16_t*>(a.weight)[j]) : 1.0f;
    const float bb = a.bias ? widen1<XT>(static_cast<const uint16_t*>(a.bias)[j]) : 0.0f;
    const float one_plus = 1.0f + widen1<XT>(sc[b * a.H + j]);
    A = w * one_plus;
    C = bb * one_plus;
    C = C + widen1<XT>(sh[b * a.H + j]);
    if (a.smooth) {
        const float s = a.smooth[j];
        A = A * s;
        C = C * s;
    }
}

// Chan et al.'s pairwise merge of (count, mean, M2), written so that the
// result does not depend on the order of the two operands: both lanes of a
// butterfly pair then hold identical bits.
struct Stats {
    float n, mean, m2;
};

__device__ __forceinline__ Stats merge(const Stats& p, const Stats& q)
{
    const float n = p.n + q.n;
    if (n == 0.0f)
        return {0.0f, 0.0f, 0.0f};
    const float rn = __builtin_amdgcn_rcpf(n);
    const float mean = (p.n * p.mean + q.n * q.mean) * rn;
    const float d = q.mean - p.mean;
    const float m2 = (p.m2 + q.m2) + d * d * ((p.n * q.n) * rn);
    return {n, mean, m2};
}

// The same merge when both sides hold the same count n: the weights are
// exact halves, no reciprocal is needed.
__device__ __forceinline__ Stats merge_equal(const Stats& p, const Stats& q)
{
    const float mean = (p.mean + q.mean) * 0.5f;
    const float d = q.mean - p.mean;
    const float m2 = (p.m2 + q.m2) + d * d * (p.n * 0.5f);
    return {p.n + q.n, mean, m2};
}

template <int CTRL>
__device__ __forceinline__ Stats dpp_stats(const Stats& s)
{
    return {dpp_f<CTRL>(s.n), dpp_f<CTRL>(s.mean), dpp_f<CTRL>(s.m2)};
}

__device__ __forceinline__ Stats wave_merge_equal(Stats s)
{
    s = merge_equal(s, dpp_stats<kDppQuadXor1>(s));
    s = merge_equal(s, dpp_stats<kDppQuadXor2>(s));
    s = merge_equal(s, dpp_stats<kDppHalfMirror>(s));
    s = merge_equal(s, dpp_stats<kDppMirror>(s));
    s = merge_equal(s, Stats{swz_xor16(s.n), swz_xor16(s.mean), swz_xor16(s.m2)});
    return merge_equal(Stats{lane_f(s.n, 0), lane_f(s.mean, 0), lane_f(s.m2, 0)},
                       Stats{lane_f(s.n, 32), lane_f(s.mean, 32), lane_f(s.m2, 32)});
}

__device__ __forceinline__ Stats wave_merge(Stats s)
{
    s = merge(s, dpp_stats<kDppQuadXor1>(s));
    s = merge(s, dpp_stats<kDppQuadXor2>(s));
    s = merge(s, dpp_stats<kDppHalfMirror>(s));
    s = merge(s, dpp_stats<kDppMirror>(s));
    s = merge(s, Stats{swz_xor16(s.n), swz_xor16(s.mean), swz_xor16(s.m2)});
    return merge(Stats{lane_f(s.n, 0), lane_f(s.mean, 0), lane_f(s.m2, 0)},
                 Stats{lane_f(s.n, 32), lane_f(s.mean, 32), lane_f(s.m2, 32)});
}

// Symmetric INT8 quantization of a row from max|y| (Formula steps 4-5).
// quantScale = RN(max|y| / 127) exactly (it is an output, checked to 1e-5);
// the codes take y * RN~(1 / quantScale), which differs from the IEEE
// quotient by at most an ulp and moves a code only when y / quantScale sits
// within about 2^-17 of a rounding tie -- far inside the stated bar of codes
// within +-1 on at most 0.01 % of the elements.  Rows whose quantScale is 0,
// tiny, huge or not finite take a true division and the saturating rule.
struct QParams {
    float qs, recip;
    bool fast;
    __device__ __forceinline__ explicit QParams(float amax)
    {
        qs = div_by_const(amax, 127.0f, 1.0f / 127.0f);
        recip = __builtin_amdgcn_rcpf(qs);
        fast = row_divisor_in_range(qs);
    }
};

template <bool FAST>
__device__ __forceinline__ uint32_t q8(float y, const QParams& qp)
{
    // |y| <= max|y| = 127 quantScale (1 + 2^-24) and recip is within an ulp
    // of 1 / quantScale, so |y * recip| < 127.00004: no clamp is needed.
    if (FAST)
        return code_bits(y * qp.recip);
    float t = y / qp.qs;
    if (t != t)
        t = 0.0f;
    return code_bits(__builtin_amdgcn_fmed3f(t, -128.0f, 127.0f));
}

// LDS table: four float4 planes of H/8 entries each: A[8k..8k+3],
// A[8k+4..8k+7], C[8k..8k+3], C[8k+4..8k+7], so that lane k's 16-byte
// reads of consecutive k are contiguous.
__device__ __forceinline__ int64_t tab_index(int64_t H, int plane, int64_t j)
{
    const int64_t k = j >> 3;
    const int r = static_cast<int>(j & 7);
    const int q = plane * 2 + (r >> 2);
    return (q * (H >> 3) + k) * 4 + (r & 3);
}

template <int XT, int VPL>
__global__ __launch_bounds__(kBlock) void ada_vec_kernel(AdaArgs a)
{
    extern __shared__ float4 tab4[];
    float* tab = reinterpret_cast<float*>(tab4);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t H = a.H;
    const int64_t nvec = H >> 3;
    const int64_t plane = nvec;  // float4 entries per plane
    const int64_t nchunks = (a.rows + a.rpb - 1) / a.rpb;
    int64_t tab_batch = -1;

    // Chunks of rpb rows, strided over the grid (one chunk per workgroup when
    // the grid covers them all; a sweep of persistent workgroups otherwise).
    for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {
    const int64_t r0 = chunk * a.rpb;
    const int64_t r1 = r0 + a.rpb < a.rows ? r0 + a.rpb : a.rows;
    int64_t r = r0;
    int64_t b = r0 / a.S;
    while (r < r1) {
        const int64_t r_end = (b + 1) * a.S < r1 ? (b + 1) * a.S : r1;
        if (b != tab_batch) {  // workgroup-uniform
            __syncthreads();  // earlier readers of the table are done
            for (int64_t j = threadIdx.x; j < H; j += kBlock) {
                float A, C;
                coeffs<XT>(a, b, j, A, C);
                tab[tab_index(H, 0, j)] = A;
                tab[tab_index(H, 1, j)] = C;
            }
            __syncthreads();
            tab_batch = b;
        }

        for (int64_t row = r + wave; row < r_end; row += 4) {
            // Every load is unconditional: lanes past the row end re-load the
            // row's last vector (their results are never stored).
            const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + row * H);
            uint4 raw[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t k = static_cast<int64_t>(i) * kWave + lane;
                raw[i] = ld_stream16(xr + (k < nvec ? k : nvec - 1));
            }
            // Welford-style statistics: each lane forms (count, mean, M2) of
            // its own elements from the registers (two passes over them), and
            // the lanes merge with Chan's pairwise update in a fixed butterfly.
            float v[VPL][8];
            float cnt = 0.0f, sum = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t k = static_cast<int64_t>(i) * kWave + lane;
                widen8<XT>(raw[i], v[i]);
                if (k < nvec) {
                    cnt += 8.0f;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        sum += v[i][j];
                }
            }
            Stats st{cnt, 0.0f, 0.0f};
            if (cnt > 0.0f) {
                st.mean = sum / cnt;
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    const int64_t k = static_cast<int64_t>(i) * kWave + lane;
                    if (k < nvec) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float d = v[i][j] - st.mean;
                            st.m2 = __builtin_fmaf(d, d, st.m2);
                        }
                    }
                }
            }
            st = a.equal_counts ? wave_merge_equal(st) : wave_merge(st);
            const float var = st.m2 * a.inv_h;
            const float rstd = __builtin_amdgcn_rsqf(var + a.eps);
            const float mean = st.mean;

            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t k = static_cast<int64_t>(i) * kWave + lane;
                if (k < nvec) {
                    const float4 A0 = tab4[0 * plane + k], A1 = tab4[1 * plane + k];
                    const float4 C0 = tab4[2 * plane + k], C1 = tab4[3 * plane + k];
                    const float Av[8] = {A0.x, A0.y, A0.z, A0.w, A1.x, A1.y, A1.z, A1.w};
                    const float Cv[8] = {C0.x, C0.y, C0.z, C0.w, C1.x, C1.y, C1.z, C1.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float nrm = (v[i][j] - mean) * rstd;
                        v[i][j] = __builtin_fmaf(nrm, Av[j], Cv[j]);
                        amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i][j]));
                    }
                }
            }
            amax = wave_max_f(amax);
            const QParams qp(amax);
            if (lane == 0)
                a.qs[row] = qp.qs;
            uint2* orow = reinterpret_cast<uint2*>(a.out + row * H);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t k = static_cast<int64_t>(i) * kWave + lane;
                if (k < nvec) {
                    uint32_t c[8];
                    if (qp.fast) {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            c[j] = q8<true>(v[i][j], qp);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            c[j] = q8<false>(v[i][j], qp);
                    }
                    st_stream8(orow + k, make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7])));
                }
            }
                }
        r = r_end;
        ++b;
    }
    }
}

// Generic variant: one workgroup per row.
__device__ __forceinline__ Stats block_merge(Stats s, Stats* red)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    s = wave_merge(s);
    if (lane == 0)
        red[wave] = s;
    __syncthreads();
    Stats t = merge(merge(red[0], red[1]), merge(red[2], red[3]));
    __syncthreads();
    return t;
}

__device__ __forceinline__ float block_max(float v, float* red)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    v = wave_max(v);
    if (lane == 0)
        red[wave] = v;
    __syncthreads();
    const float m = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    __syncthreads();
    return m;
}

template <int XT>
__global__ __launch_bounds__(kBlock) void ada_generic_kernel(AdaArgs a)
{
    __shared__ Stats red_s[4];
    __shared__ float red_f[4];
    const int64_t row = blockIdx.x;
    if (row >= a.rows)
        return;
    const int64_t b = row / a.S;
    const uint16_t* xr = static_cast<const uint16_t*>(a.x) + row * a.H;

    // Welford's running update per thread, then Chan merges.
    Stats st{0.0f, 0.0f, 0.0f};
    for (int64_t j = threadIdx.x; j < a.H; j += kBlock) {
        const float xv = widen1<XT>(xr[j]);
        st.n += 1.0f;
        const float d = xv - st.mean;
        st.mean = st.mean + d / st.n;
        st.m2 = __builtin_fmaf(d, xv - st.mean, st.m2);
    }
    st = block_merge(st, red_s);
    const float var = st.m2 / static_cast<float>(a.H);
    const float rstd = 1.0f / __builtin_sqrtf(var + a.eps);

    float amax = 0.0f;
    for (int64_t j = threadIdx.x; j < a.H; j += kBlock) {
        float A, C;
        coeffs<XT>(a, b, j, A, C);
        const float nrm = (widen1<XT>(xr[j]) - st.mean) * rstd;
        amax = __builtin_fmaxf(amax, __builtin_fabsf(__builtin_fmaf(nrm, A, C)));
    }
    amax = block_max(amax, red_f);
    const QParams qp(amax);
    if (threadIdx.x == 0)
        a.qs[row] = qp.qs;
    int8_t* orow = a.out + row * a.H;
    for (int64_t j = threadIdx.x; j < a.H; j += kBlock) {
        float A, C;
        coeffs<XT>(a, b, j, A, C);
        const float nrm = (widen1<XT>(xr[j]) - st.mean) * rstd;
        const float y = __builtin_fmaf(nrm, A, C);
        orow[j] = static_cast<int8_t>((qp.fast ? q8<true>(y, qp) : q8<false>(y, qp)) & 0xFFu);
    }
}

using KernelFn = void (*)(AdaArgs);

template <int XT>
KernelFn pick_vec(int vpl)
{
    switch (vpl) {
    case 1: return ada_vec_kernel<XT, 1>;
    case 2: return ada_vec_kernel<XT, 2>;
    case 4: return ada_vec_kernel<XT, 4>;
    case 6: return ada_vec_kernel<XT, 6>;
    case 8: return ada_vec_kernel<XT, 8>;
    case 12: return ada_vec_kernel<XT, 12>;
    case 16: return ada_vec_kernel<XT, 16>;
    }
    return nullptr;
}

}  // namespace

hipError_t launch_ada_layernorm_quant(const AdaPlan& p, hipStream_t stream)
{
    AdaArgs a{};
    a.x = p.x;
    a.scale = p.scale;
    a.shift = p.shift;
    a.weight = p.weight;
    a.bias = p.bias;
    a.smooth = p.smooth;
    a.S = p.S;
    a.H = p.H;
    a.rows = p.B * p.S;
    a.eps = p.eps;
    a.out = p.out;
    a.qs = p.quant_scale;
    a.equal_counts = (p.H % 512) == 0;
    a.inv_h = 1.0f / static_cast<float>(p.H);
    KernelFn fn;
    size_t lds = 0;
    if (p.variant == ADA_VAR_VECTOR) {
        fn = p.x_type == X_F16 ? pick_vec<X_F16>(p.vpl) : pick_vec<X_BF16>(p.vpl);
        a.rpb = p.rows_per_block;
        lds = static_cast<size_t>(p.H) * 2 * sizeof(float);
    } else {
        fn = p.x_type == X_F16 ? ada_generic_kernel<X_F16> : ada_generic_kernel<X_BF16>;
        a.rpb = 1;
    }
    if (!fn)
        return hipErrorInvalidValue;
    a.nblocks = (a.rows + a.rpb - 1) / a.rpb;
    if (p.variant == ADA_VAR_VECTOR && kAdaPersistent) {
        int per_cu = 0, cus = 0, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kBlock, lds) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidValue;
        const int64_t resident = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * cus;
        if (a.nblocks > resident)
            a.nblocks = resident;
    }
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(a.nblocks)),
                           dim3(kBlock), args, lds, stream);
}

}  // namespace dq
