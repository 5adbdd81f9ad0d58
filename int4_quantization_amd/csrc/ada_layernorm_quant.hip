// ada_layernorm_quant.hip -- AdaLayerNorm fused with symmetric INT8
// dynamic quantization on gfx950 (aclnnAdaLayerNormQuant, Formula 1-5):
//   LN = (x - E(x)) / sqrt(Var(x) + eps) * weight + bias
//   y  = LN * (1 + scale[b]) + shift[b];   y = y * smooth
//   quantScale = row_max(|y|) / 127;      out = round(y / quantScale)
//
// Layout of the work: a workgroup of four waves converts 4*T consecutive
// rows (T = 4 per wave, each next row's loads in flight while the current
// one is processed) and exits.  When its rows share a batch b, it first writes the
// per-column coefficients
//   A_j = w_j * (1 + scale_bj) * smooth_j
//   C_j = (bias_j * (1 + scale_bj) + shift_bj) * smooth_j
// into LDS from 16-byte parameter loads, so that
// y_j = ((x_j - mean) * rstd) * A_j + C_j is one multiply and one fma per
// element.  Each row is held in VGPRs by one wave (16-byte non-temporal
// loads, one HBM read per element); its statistics are Welford style: every
// lane forms (count, mean, M2) of its own elements from the registers, and
// the lanes merge with Chan's pairwise update in a fixed butterfly (a
// reciprocal-free form when every lane holds the same count).  Statistics,
// normalization and modulation are fp32 with hardware rsq; quantScale is
// the exact binary32 RN(max|y| / 127).  Loads and stores are unconditional
// (clamped) so that no wait for the next row's data also waits for this
// row's stores.
//
// Rows that are not whole 16-byte vectors or are longer than 16 vectors
// per lane use the generic kernel (one workgroup per row, three passes over
// the row from global memory, same arithmetic).

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

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

// Rows each wave converts in one workgroup: each next row's loads are in
// flight while the current one is reduced and stored, and the workgroup's
// coefficient table serves 4 * kAdaRowsPerWave rows.
constexpr int kAdaRowsPerWave = 4;

// Eight consecutive columns 8k..8k+7 of the modulation coefficients for
// batch b (same formula order as coeffs()), from 16-byte loads.  Every load
// is unconditional, so all of them are in flight together: an absent
// weight, bias or smooth vector reads a stand-in of the same size from the
// batch's scale row (always present) and its values are replaced after.
template <int XT>
__device__ __forceinline__ void coeffs8(const AdaArgs& a, int64_t b, int64_t k, float (&A)[8], float (&C)[8])
{
    const uint4* scrow = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.scale) + b * a.H);
    const uint4* shrow = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.shift) + b * a.H);
    const uint4 scv = scrow[k];
    const uint4 shv = shrow[k];
    const uint4 wv = (a.weight ? static_cast<const uint4*>(a.weight) : scrow)[k];
    const uint4 bv = (a.bias ? static_cast<const uint4*>(a.bias) : shrow)[k];
    const float4* sm4 = reinterpret_cast<const float4*>(a.smooth);
    const float4* stand_in = reinterpret_cast<const float4*>(scrow + k);
    const float4 s0 = *(a.smooth ? sm4 + 2 * k : stand_in);
    const float4 s1 = *(a.smooth ? sm4 + 2 * k + 1 : stand_in);
    float w[8], bb[8], sc[8], sh[8];
    widen8<XT>(scv, sc);
    widen8<XT>(shv, sh);
    widen8<XT>(wv, w);
    widen8<XT>(bv, bb);
    const float sm[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float wj = a.weight ? w[j] : 1.0f;
        const float bj = a.bias ? bb[j] : 0.0f;
        const float one_plus = 1.0f + sc[j];
        A[j] = wj * one_plus;
        C[j] = bj * one_plus;
        C[j] = C[j] + sh[j];
        if (a.smooth) {
            A[j] = A[j] * sm[j];
            C[j] = C[j] * sm[j];
        }
    }
}

// LDS table of one batch's coefficients: four float4 planes of H/8 entries,
// A[8k..8k+3], A[8k+4..8k+7], C[8k..8k+3], C[8k+4..8k+7], so that lane k's
// 16-byte reads of consecutive k are contiguous and conflict-free.
template <int XT>
__device__ __forceinline__ void build_table(const AdaArgs& a, int64_t b, float4* tab4, int64_t nvec)
{
    // Threads past the last entry rewrite it with the same values.
    for (int64_t k0 = 0; k0 < nvec; k0 += kBlock) {
        int64_t k = k0 + threadIdx.x;
        k = k < nvec ? k : nvec - 1;
        float A[8], C[8];
        coeffs8<XT>(a, b, k, A, C);
        tab4[0 * nvec + k] = make_float4(A[0], A[1], A[2], A[3]);
        tab4[1 * nvec + k] = make_float4(A[4], A[5], A[6], A[7]);
        tab4[2 * nvec + k] = make_float4(C[0], C[1], C[2], C[3]);
        tab4[3 * nvec + k] = make_float4(C[4], C[5], C[6], C[7]);
    }
}

// One row held in raw[] (wave-wide): statistics, modulation, quantization
// and stores.  FULL: every lane holds VPL whole vectors of the row (no
// tail).  Otherwise a lane whose vector lies past the row end holds a copy
// of the last vector (clamped load): it is left out of the statistics, and
// its y values and codes equal those of the vector it copies, so it changes
// neither max|y| nor the bytes stored (it writes that vector's codes again).
// Coefficients come from the LDS table.  Straight-line except the
// row-uniform fast/slow choice, whose paths join before the stores.
template <int XT, int VPL, bool FULL>
__device__ __forceinline__ void ada_row(const AdaArgs& a, const uint4 (&raw)[VPL], int64_t row, int64_t nvec,
                                        int lane, const float4* tab4)
{
    float v[VPL][8];
    float sum = 0.0f, cnt = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        widen8<XT>(raw[i], v[i]);
        const bool ok = FULL || static_cast<int64_t>(i) * kWave + lane < nvec;
        if (!FULL)
            cnt += ok ? 8.0f : 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sum += FULL ? v[i][j] : (ok ? v[i][j] : 0.0f);
    }
    if (FULL)
        cnt = 8.0f * VPL;
    // Welford-style statistics: (count, mean, M2) of the lane's own elements
    // from the registers, then Chan's pairwise merge across the lanes.
    Stats st{cnt, 0.0f, 0.0f};
    st.mean = cnt > 0.0f ? sum / cnt : 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const bool ok = FULL || static_cast<int64_t>(i) * kWave + lane < nvec;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float d = FULL ? v[i][j] - st.mean : (ok ? v[i][j] - st.mean : 0.0f);
            st.m2 = __builtin_fmaf(d, d, st.m2);
        }
    }
    st = (FULL || a.equal_counts) ? wave_merge_equal(st) : wave_merge(st);
    const float var = st.m2 * a.inv_h;
    const float rstd = __builtin_amdgcn_rsqf(var + a.eps);
    const float mean = st.mean;

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int64_t k = static_cast<int64_t>(i) * kWave + lane;
        if (!FULL)
            k = k < nvec ? k : nvec - 1;
        const float4 A0 = tab4[0 * nvec + k], A1 = tab4[1 * nvec + k];
        const float4 C0 = tab4[2 * nvec + k], C1 = tab4[3 * nvec + k];
        const float Av[8] = {A0.x, A0.y, A0.z, A0.w, A1.x, A1.y, A1.z, A1.w};
        const float Cv[8] = {C0.x, C0.y, C0.z, C0.w, C1.x, C1.y, C1.z, C1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float nrm = (v[i][j] - mean) * rstd;
            v[i][j] = __builtin_fmaf(nrm, Av[j], Cv[j]);
            amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i][j]));
        }
    }
    amax = wave_max_f(amax);
    const QParams qp(amax);
    a.qs[row] = qp.qs;  // every lane writes the same value
    uint2 pk[VPL];
    if (qp.fast) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            uint32_t c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = q8<true>(v[i][j], qp);
            pk[i] = make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7]));
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            uint32_t c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = q8<false>(v[i][j], qp);
            pk[i] = make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7]));
        }
    }
    uint2* orow = reinterpret_cast<uint2*>(a.out + row * a.H);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int64_t k = static_cast<int64_t>(i) * kWave + lane;
        if (!FULL)
            k = k < nvec ? k : nvec - 1;
        st_stream8(orow + k, pk[i]);
    }
}

template <int VPL, bool FULL>
__device__ __forceinline__ void ada_load(uint4 (&raw)[VPL], const AdaArgs& a, int64_t row, int64_t nvec, int lane)
{
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + row * a.H);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int64_t k = static_cast<int64_t>(i) * kWave + lane;
        if (!FULL)
            k = k < nvec ? k : nvec - 1;
        raw[i] = ld_stream16(xr + k);
    }
}

// A workgroup converts rows r0 .. r0 + 4T - 1 (T = kAdaRowsPerWave): step t
// of wave w takes row r0 + 4t + w (clamped to the last row, whose duplicate
// writes the bytes its owner writes).  When all of them belong to one
// batch, the workgroup writes that batch's coefficients into LDS once and
// streams its rows; otherwise (rows across a batch boundary, e.g. S < 4T)
// it goes through the batches its rows touch, one table each.
template <int XT, int VPL, bool FULL>
__global__ __launch_bounds__(kBlock) void ada_vec_kernel(AdaArgs a)
{
    extern __shared__ float4 tab4[];
    constexpr int T = kAdaRowsPerWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t nvec = a.H >> 3;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * (4 * T);
    auto row_of = [&](int t) -> int64_t {
        const int64_t r = r0 + 4 * t + wave;
        return r < a.rows ? r : a.rows - 1;
    };
    const int64_t r_last = r0 + 4 * T - 1 < a.rows ? r0 + 4 * T - 1 : a.rows - 1;
    const int64_t b0 = r0 / a.S, b_last = r_last / a.S;

    if (b0 == b_last) {  // workgroup-uniform
        uint4 buf[2][VPL];
        ada_load<VPL, FULL>(buf[0], a, row_of(0), nvec, lane);
        build_table<XT>(a, b0, tab4, nvec);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t + 1 < T)
                ada_load<VPL, FULL>(buf[(t + 1) & 1], a, row_of(t + 1), nvec, lane);
            __builtin_amdgcn_sched_barrier(0);
            ada_row<XT, VPL, FULL>(a, buf[t & 1], row_of(t), nvec, lane, tab4);
        }
    } else {
        for (int64_t b = b0; b <= b_last; ++b) {
            __syncthreads();  // the previous table's readers are done
            build_table<XT>(a, b, tab4, nvec);
            __syncthreads();
            for (int t = 0; t < T; ++t) {
                const int64_t r = r0 + 4 * t + wave;
                if (r < a.rows && r / a.S == b) {
                    uint4 raw[VPL];
                    ada_load<VPL, FULL>(raw, a, r, nvec, lane);
                    ada_row<XT, VPL, FULL>(a, raw, r, nvec, lane, tab4);
                }
            }
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

template <int XT, bool FULL>
KernelFn pick_vec(int vpl)
{
    switch (vpl) {
    case 1: return ada_vec_kernel<XT, 1, FULL>;
    case 2: return ada_vec_kernel<XT, 2, FULL>;
    case 4: return ada_vec_kernel<XT, 4, FULL>;
    case 6: return ada_vec_kernel<XT, 6, FULL>;
    case 8: return ada_vec_kernel<XT, 8, FULL>;
    case 12: return ada_vec_kernel<XT, 12, FULL>;
    case 16: return ada_vec_kernel<XT, 16, FULL>;
    }
    return nullptr;
}

template <int XT>
KernelFn pick_vec_x(int vpl, bool full)
{
    return full ? pick_vec<XT, true>(vpl) : pick_vec<XT, false>(vpl);
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
    int64_t rows_per_block = 1;
    if (p.variant == ADA_VAR_VECTOR) {
        const bool full = p.H == static_cast<int64_t>(p.vpl) * kWave * 8;
        fn = p.x_type == X_F16 ? pick_vec_x<X_F16>(p.vpl, full) : pick_vec_x<X_BF16>(p.vpl, full);
        rows_per_block = 4 * kAdaRowsPerWave;
        lds = static_cast<size_t>(p.H) * 2 * sizeof(float);
    } else {
        fn = p.x_type == X_F16 ? ada_generic_kernel<X_F16> : ada_generic_kernel<X_BF16>;
    }
    if (!fn)
        return hipErrorInvalidValue;
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > kMaxGridBlocks)
        return hipErrorInvalidValue;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock),
                           args, lds, stream);
}

}  // namespace dq
