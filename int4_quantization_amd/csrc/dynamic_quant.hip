// dynamic_quant.hip -- per-token dynamic quantization on gfx950
// (aclnnDynamicQuantV2, Description and Formula).
//
// Vector variant (rows of whole 16-byte vectors up to 4 waves x 16 vectors
// per lane): persistent workgroups of four waves; TEAM waves (1, 2 or 4)
// own one row at a time, so a workgroup converts 4/TEAM rows per step.
// Lane l of team wave w holds the 16-byte vectors k = (i*TEAM + w)*64 + l,
// i < VPL, so every load instruction covers contiguous row bytes; the row
// stays in VGPRs as fp32 (after the smooth multiply), is reduced through
// DPP (and LDS across the team), then quantized and stored from the same
// registers: one HBM read per input element and one write per code, both
// streamed with non-temporal accesses.  Workgroups sweep down the matrix in
// tiles of T row groups interleaved across the grid, so all of them work
// inside one band of rows at a time (a compact DRAM footprint) while each
// one's consecutive rows mostly share an expert.  Each lane always owns the
// same columns, so its smooth scales live in VGPRs and are reloaded only
// when the row's expert changes.  With PF, the next row's loads are issued
// before the current row is reduced.
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

#include <mutex>

#include "dq_device.h"
#include "dq_internal.h"

namespace dq {
namespace {

constexpr bool kDqPrefetch = false;  // issue the next row's loads before reducing this one
                                      // (measured no faster once loads are unconditional)
constexpr uint64_t kDqTile = 4;      // row groups a workgroup converts before jumping ahead (power of 2)

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
    int64_t tile;  // row groups per tile (vector variant)
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
            scale = div_by_const(a_hi, C::offset_opt, 1.0f / C::offset_opt);
        } else {
            const float range = a_hi - a_lo;
            scale = div_by_const(range, C::scale_opt, 1.0f / C::scale_opt);
        }
        recip = 1.0f / scale;
        fast = row_divisor_in_range(scale);
        if (SYM) {
            offset = 0.0f;
        } else {
            // max / scale; a quotient too small for the correction step to be
            // exact (|q| < 2^-40) leaves offset_opt - q at offset_opt either way.
            const float q_hi = fast ? div_by_row(a_hi, scale, recip) : a_hi / scale;
            offset = C::offset_opt - q_hi;
        }
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
        st_stream8(dst, make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7])));
    } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(y) + row * (n >> 1)) + k;
        st_stream4(dst, pack8_i4(c));
    }
}

// Loads of a row for one team wave.  Lanes whose vector lies past the row
// end re-load the row's last vector: a duplicate changes neither max nor
// min, and every load is unconditional, so each register's load is always
// consumed before it is loaded again (no divergent paths that would force a
// full wait on outstanding memory before the next prefetch).
template <int VPL, int TEAM>
__device__ __forceinline__ void load_x(uint4 (&raw)[VPL], const void* x, int64_t row, int64_t n, int64_t nvec,
                                       int wit, int lane)
{
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * n);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int64_t k = static_cast<int64_t>(i * TEAM + wit) * kWave + lane;
        raw[i] = ld_stream16(xr + (k < nvec ? k : nvec - 1));
    }
}

template <int XT, bool SYM, int OUT, int VPL, int TEAM, bool PF>
__global__ __launch_bounds__(kBlock) void dq_vec_kernel(DqArgs a)
{
    constexpr int RPS = 4 / TEAM;  // rows per workgroup step
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slot = wave / TEAM;
    const int wit = wave % TEAM;
    const int64_t nvec = a.n >> 3;
    const uint64_t G = static_cast<uint64_t>(a.nblocks);
    const uint64_t b = blockIdx.x;
    constexpr uint64_t T = kDqTile;
    // Step s of this workgroup converts row group ((b + (s / T) * G) * T + s % T).
    auto group_of = [&](int64_t step) -> int64_t {
        const uint64_t u = static_cast<uint64_t>(step);
        return static_cast<int64_t>((b + (u / T) * G) * T + u % T);
    };
    auto row_of = [&](int64_t step) -> int64_t { return group_of(step) * RPS + slot; };
    const int64_t groups = (a.rows + RPS - 1) / RPS;

    // Expert bounds cached per lane (first 64 experts).
    const bool moe = a.gi != nullptr;
    int32_t gi_lane = 0;
    if (moe && lane < a.n_experts)
        gi_lane = a.gi[lane];

    float sreg[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sreg[i][j] = 1.0f;
    int64_t cur_e = -1;
    __shared__ float red[2][2][4];

    uint4 buf0[VPL], buf1[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        buf0[i] = buf1[i] = make_uint4(0, 0, 0, 0);
    if (group_of(0) < groups && row_of(0) < a.rows)
        load_x<VPL, TEAM>(buf0, a.x, row_of(0), a.n, nvec, wit, lane);

    // One step: row_of(s) is in cur; with PF the next row is requested into
    // nxt before any arithmetic, otherwise after the stores.  Returns false
    // when the workgroup has no more rows (workgroup-uniform).
    auto step = [&](int64_t s, uint4 (&cur)[VPL], uint4 (&nxt)[VPL]) -> bool {
        if (group_of(s) >= groups)
            return false;
        const int64_t row = row_of(s);
        const bool active = row < a.rows;  // team-uniform
        const int64_t nrow = row_of(s + 1);
        const bool has_next = group_of(s + 1) < groups && nrow < a.rows;
        if (PF && has_next)
            load_x<VPL, TEAM>(nxt, a.x, nrow, a.n, nvec, wit, lane);

        if (a.smooth && active) {
            int64_t e = 0;
            if (moe) {
                if (a.n_experts <= kWave) {
                    const unsigned long long mask = __ballot(lane < a.n_experts && row < gi_lane);
                    e = mask ? __builtin_ctzll(mask) : a.n_experts - 1;
                } else {
                    e = expert_of_row(row, a.gi, a.n_experts, lane);
                }
            }
            if (e != cur_e) {
                const float4* sr = reinterpret_cast<const float4*>(a.smooth + e * a.n);
#pragma unroll
                for (int i = 0; i < VPL; ++i) {
                    int64_t k = static_cast<int64_t>(i * TEAM + wit) * kWave + lane;
                    k = k < nvec ? k : nvec - 1;
                    const float4 s0 = sr[2 * k], s1 = sr[2 * k + 1];
                    sreg[i][0] = s0.x;
                    sreg[i][1] = s0.y;
                    sreg[i][2] = s0.z;
                    sreg[i][3] = s0.w;
                    sreg[i][4] = s1.x;
                    sreg[i][5] = s1.y;
                    sreg[i][6] = s1.z;
                    sreg[i][7] = s1.w;
                }
                cur_e = e;
            }
        }

        // Widen, smooth and reduce every vector, including the duplicated
        // tail vectors and an inactive tail row (its results are dropped).
        float s_hi = SYM ? 0.0f : -__builtin_huge_valf();
        float s_lo = __builtin_huge_valf();
        float v[VPL][8];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            widen8<XT>(cur[i], v[i]);
            if (a.smooth) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[i][j] = v[i][j] * sreg[i][j];
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
        s_hi = wave_max_f(s_hi);
        if (!SYM)
            s_lo = wave_min_f(s_lo);
        if (TEAM > 1) {
            // One barrier per step: partials alternate between two LDS slots,
            // so a slot is rewritten only after every wave has passed the
            // barrier of the step that read it.
            const int par = static_cast<int>(s & 1);
            if (lane == 0) {
                red[par][0][wave] = s_hi;
                red[par][1][wave] = s_lo;
            }
            __syncthreads();
            const int w0 = slot * TEAM;
            s_hi = red[par][0][w0];
            s_lo = red[par][1][w0];
#pragma unroll
            for (int w = 1; w < TEAM; ++w) {
                s_hi = __builtin_fmaxf(s_hi, red[par][0][w0 + w]);
                s_lo = __builtin_fminf(s_lo, red[par][1][w0 + w]);
            }
        }

        if (active) {
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
        if (!PF && has_next)
            load_x<VPL, TEAM>(nxt, a.x, nrow, a.n, nvec, wit, lane);
        return true;
    };

    for (int64_t s = 0;; s += 2) {
        if (!step(s, buf0, buf1))
            break;
        if (!step(s + 1, buf1, buf0))
            break;
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
    const int64_t row = blockIdx.x;
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

template <int XT, bool SYM, int OUT, int TEAM>
KernelFn pick_vpl(int vpl)
{
    switch (vpl) {
    case 1: return dq_vec_kernel<XT, SYM, OUT, 1, TEAM, kDqPrefetch>;
    case 2: return dq_vec_kernel<XT, SYM, OUT, 2, TEAM, kDqPrefetch>;
    case 4: return dq_vec_kernel<XT, SYM, OUT, 4, TEAM, kDqPrefetch>;
    case 8: return dq_vec_kernel<XT, SYM, OUT, 8, TEAM, kDqPrefetch>;
    case 16: return dq_vec_kernel<XT, SYM, OUT, 16, TEAM, kDqPrefetch>;
    }
    return nullptr;
}

template <int XT, bool SYM, int OUT>
KernelFn pick(const DqPlan& p)
{
    if (p.variant != DQ_VAR_VECTOR)
        return dq_generic_kernel<XT, SYM, OUT>;
    switch (p.team) {
    case 1: return pick_vpl<XT, SYM, OUT, 1>(p.vpl);
    case 2: return pick_vpl<XT, SYM, OUT, 2>(p.vpl);
    case 4: return pick_vpl<XT, SYM, OUT, 4>(p.vpl);
    }
    return nullptr;
}

template <int XT>
KernelFn pick_x(const DqPlan& p)
{
    if (p.symmetric)
        return p.out_kind == OUT_I8 ? pick<XT, true, OUT_I8>(p) : pick<XT, true, OUT_I4>(p);
    return p.out_kind == OUT_I8 ? pick<XT, false, OUT_I8>(p) : pick<XT, false, OUT_I4>(p);
}

// Resident workgroups per CU for a kernel, and the CU count, looked up once
// per device and kernel.
int64_t resident_blocks(KernelFn fn)
{
    struct Entry { int device; KernelFn fn; int64_t blocks; };
    static Entry cache[64];
    static int used = 0;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].device == dev && cache[i].fn == fn)
            return cache[i].blocks;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), kBlock, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    const int64_t blocks = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * cus;
    if (used < 64)
        cache[used++] = Entry{dev, fn, blocks};
    return blocks;
}

}  // namespace

hipError_t launch_dynamic_quant(const DqPlan& p, hipStream_t stream)
{
    KernelFn fn = p.x_type == X_F16 ? pick_x<X_F16>(p) : pick_x<X_BF16>(p);
    if (!fn)
        return hipErrorInvalidValue;
    DqArgs a{p.x, p.smooth, p.group_index, p.n_experts, p.rows, p.n, p.y, p.scale, p.offset, 0, 1};
    if (p.variant == DQ_VAR_VECTOR) {
        const int64_t rps = 4 / p.team;
        const int64_t groups = (p.rows + rps - 1) / rps;
        a.tile = static_cast<int64_t>(kDqTile);
        const int64_t tiles = (groups + a.tile - 1) / a.tile;
        const int64_t resident = resident_blocks(fn);
        if (resident <= 0)
            return hipErrorInvalidValue;
        a.nblocks = tiles < resident ? tiles : resident;
    } else {
        a.nblocks = p.rows;
    }
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(a.nblocks)),
                           dim3(kBlock), args, 0, stream);
}

}  // namespace dq
