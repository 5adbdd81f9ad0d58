// dynamic_quant.hip -- per-token dynamic quantization on gfx950
// (aclnnDynamicQuantV2, Description and Formula).
//
// Vector variant (rows of whole 16-byte vectors up to 4 waves x 16 vectors
// per lane): TEAM waves (1, 2 or 4) share a row, so a workgroup of four
// waves holds 4/TEAM teams; each team converts T consecutive rows (2 for
// rows of up to 4 vectors per lane, else 1) and the workgroup exits.  Lane
// l of team wave w holds the 16-byte vectors k = (i*TEAM + w)*64 + l,
// i < VPL, so every load instruction covers contiguous row bytes; the row
// stays in VGPRs, is widened, smoothed and reduced through DPP (and LDS
// across the team), then quantized and stored from the same registers: one
// HBM read per input element and one write per code, both streamed with
// non-temporal accesses.  The next row's loads are issued before this row
// is reduced, and the smooth scales are loaded once per team.
//
// Why short-lived workgroups rather than a persistent loop over rows: the
// vector memory counter counts stores as well as loads, so a wave that
// loads its next row after storing the last one also waits for those stores
// before it can use the new data; and many short workgroups let the
// dispatcher keep every CU busy with loads while earlier ones' stores
// drain, with the rows in flight inside a compact band of the matrix.
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
    int64_t long_teams;  // > 0: team kernel's long schedule (the count of strided teams)
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

// Eight codes of one vector packed for storing: INT8 as two dwords (four
// bytes each), INT4 as one dword (eight nibbles, low nibble first).
template <int OUT>
__device__ __forceinline__ uint2 pack_codes(const uint32_t (&c)[8])
{
    if (OUT == OUT_I8)
        return make_uint2(pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7]));
    return make_uint2(pack8_i4(c), 0u);
}

template <int OUT>
__device__ __forceinline__ void store_packed(void* y, int64_t row, int64_t n, int64_t k, uint2 pk)
{
    if (OUT == OUT_I8) {
        uint2* dst = reinterpret_cast<uint2*>(static_cast<int8_t*>(y) + row * n) + k;
        st_stream8(dst, pk);
    } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(y) + row * (n >> 1)) + k;
        st_stream4(dst, pk.x);
    }
}

// Loads of a row for one team wave.  Lanes whose vector lies past the row
// end re-load the row's last vector: a duplicate changes neither max nor
// min, and every load is unconditional, so each register's load is always
// consumed before it is loaded again (no divergent paths that would force a
// full wait on outstanding memory before the next prefetch).
template <int VPL>
__device__ __forceinline__ void load_x(uint4 (&raw)[VPL], const void* x, int64_t row, int64_t n, int64_t nvec,
                                       int team, int wit, int lane)
{
    const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * n);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int64_t k = static_cast<int64_t>(i * team + wit) * kWave + lane;
        raw[i] = ld_stream16(xr + (k < nvec ? k : nvec - 1));
    }
}

// One vector widened to fp32 and multiplied by its smooth scales (the
// Formula's x * smoothScales, one rounding per element).  Without smooth
// scales the registers hold 1.0, and x * 1 is x exactly, so the code has no
// branch here and the compiler can interleave widening with the reduction.
template <int XT>
__device__ __forceinline__ void smoothed(const uint4 raw, const float (&sr)[8], float (&v)[8])
{
    widen8<XT>(raw, v);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = v[j] * sr[j];
}

// Expert of a row: the cached bounds of the first 64 experts (one per lane)
// through a ballot, else the general search.  Wave-uniform.
__device__ __forceinline__ int64_t row_expert(int64_t row, int32_t gi_lane, const DqArgs& a, int lane)
{
    if (a.n_experts <= kWave) {
        // Rows fit in int32 (the host limits them), so the bound is compared
        // without widening the loaded value, which would consume it (and
        // wait for it) where it is loaded.
        const unsigned long long mask = __ballot(lane < a.n_experts && static_cast<int32_t>(row) < gi_lane);
        return mask ? __builtin_ctzll(mask) : a.n_experts - 1;
    }
    return expert_of_row(row, a.gi, a.n_experts, lane);
}

template <int VPL>
__device__ __forceinline__ void load_smooth(float (&sreg)[VPL][8], const DqArgs& a, int64_t e, int64_t nvec,
                                            int team, int wit, int lane)
{
    if (a.smooth) {
        const float4* sr = reinterpret_cast<const float4*>(a.smooth + e * a.n);
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int64_t k = static_cast<int64_t>(i * team + wit) * kWave + lane;
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
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sreg[i][j] = 1.0f;
    }
}

// Reduce, quantize and store one row held in raw[] (step t of the team).
// Straight-line code: every store is unconditional.  A lane whose vector
// lies past the row end holds a copy of the last vector (clamped load) and
// stores its identical codes to that vector's place; a row past the matrix
// end is a clamped copy of the last row, written with the same bytes its
// owner writes.  With no branch between this row's stores and the next
// row's loads, the compiler neither moves those loads below the stores nor
// makes their wait also wait for the stores.
// TMAX: the largest team the caller has (1: a wave per row, no exchange).
template <int XT, bool SYM, int OUT, int VPL, int TMAX>
__device__ __forceinline__ void convert_row(const DqArgs& a, const uint4 (&raw)[VPL], const float (&sreg)[VPL][8],
                                            int64_t row, int t, int64_t nvec, int slot, int team, int wit, int lane,
                                            float2 (&red)[2][kDqMaxTeam])
{
    float s_hi = SYM ? 0.0f : -__builtin_huge_valf();
    float s_lo = __builtin_huge_valf();
    float v[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        smoothed<XT>(raw[i], sreg[i], v[i]);
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
    if (TMAX > 1) {
        // Partials alternate between two LDS slots by step, so a slot is
        // rewritten only after every wave has passed the barrier of the step
        // that read it.  All TMAX slots are read at once (slots past the
        // team repeat the first), so the reads do not wait on one another.
        const int par = t & 1;
        const int w0 = slot * team;
        if (lane == 0)
            red[par][w0 + wit] = make_float2(s_hi, s_lo);
        __syncthreads();
        const float2 p0 = red[par][w0];
        s_hi = p0.x;
        s_lo = p0.y;
#pragma unroll
        for (int w = 1; w < TMAX; ++w) {
            const float2 pw = red[par][w0 + (w < team ? w : 0)];
            s_hi = __builtin_fmaxf(s_hi, pw.x);
            s_lo = __builtin_fminf(s_lo, pw.y);
        }
        // The values are the same in every lane; saying so keeps the row
        // parameters in scalar registers and makes the branch below a
        // scalar one.  (A branch the compiler takes for divergent runs both
        // store blocks one after the other, and the wait for the next row
        // then also waits for these stores.)
        s_hi = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s_hi)));
        s_lo = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s_lo)));
    }

    const RowParams<SYM, OUT> rp(s_hi, s_lo);
    // The team's first wave writes the row parameters (all its lanes the same
    // value to the same place): one store instruction per row, under a
    // wave-uniform branch.
    if (__builtin_amdgcn_readfirstlane(wit) == 0) {
        a.scale[row] = rp.scale;
        if (!SYM)
            a.offset[row] = rp.offset;
    }
    // Codes are computed on one of two paths and stored after they join, so
    // the stores are one straight sequence whichever path ran.
    uint2 pk[VPL];
    if (rp.fast) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            uint32_t c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = quant_code<SYM, OUT, true>(v[i][j], rp);
            pk[i] = pack_codes<OUT>(c);
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            uint32_t c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = quant_code<SYM, OUT, false>(v[i][j], rp);
            pk[i] = pack_codes<OUT>(c);
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int64_t k = static_cast<int64_t>(i * team + wit) * kWave + lane;
        k = k < nvec ? k : nvec - 1;
        store_packed<OUT>(a.y, row, a.n, k, pk[i]);
    }
}

// Rows each team converts in one workgroup, one after another, with the
// next kDqPrefetch rows' loads in flight while a row is reduced and stored;
// the smooth scales are loaded once for all of them.
constexpr int dq_rows_per_team(int vpl, int team)
{
    return vpl > 4 ? 1 : team >= 4 ? 4 : 2;
}

template <int XT, bool SYM, int OUT, int VPL, int TEAM>
__global__ __launch_bounds__(kDqWaves * kWave) void dq_vec_kernel(DqArgs a)
{
    constexpr int RPS = kDqWaves / TEAM;  // teams per workgroup
    constexpr int T = dq_rows_per_team(VPL, TEAM);
    constexpr int PD = kDqPrefetch < T ? kDqPrefetch : (T > 1 ? T - 1 : 1);
    constexpr int NB = PD + 1;  // row buffers
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int slot = wave / TEAM;
    const int wit = wave % TEAM;
    const int64_t nvec = a.n >> 3;
    // MoE: the workgroup converts rows r0 .. r0 + T*RPS - 1 (rows are
    // sorted by expert, so they share smooth rows): step t of team `slot`
    // takes row r0 + t*RPS + slot.  Otherwise step t takes row group
    // blockIdx.x + t * gridDim.x, so the resident workgroups sweep one
    // compact band of rows at a time (measured 2.7% faster on bf16
    // [8192, 7168] than consecutive rows per workgroup).  Rows past the end
    // clamp to the last row, which is then written twice with equal values.
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * (T * RPS);
    auto row_of = [&](int t) -> int64_t {
        const int64_t r = a.gi ? r0 + static_cast<int64_t>(t) * RPS + slot
                               : (static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(t) * gridDim.x) * RPS + slot;
        return r < a.rows ? r : a.rows - 1;
    };
    __shared__ float2 red[2][kDqMaxTeam];

    // Every load is unconditional or under a workgroup-uniform branch (a
    // load under a divergent branch makes the compiler wait for everything
    // outstanding where the branch ends).  Expert bounds are requested
    // first, so the wait for them does not also wait for the row.
    const bool moe = a.gi != nullptr;
    int32_t gi_lane = 0;
    if (moe)
        gi_lane = a.gi[lane < a.n_experts ? lane : a.n_experts - 1];

    uint4 buf[NB][VPL];
    load_x<VPL>(buf[0], a.x, row_of(0), a.n, nvec, TEAM, wit, lane);

    float sreg[VPL][8];
    int64_t e0 = 0;
    bool one_expert = true;
    if (moe && a.smooth) {
        const int64_t r_last = r0 + T * RPS - 1 < a.rows ? r0 + T * RPS - 1 : a.rows - 1;
        e0 = row_expert(r0, gi_lane, a, lane);
        one_expert = e0 == row_expert(r_last, gi_lane, a, lane);  // workgroup-uniform
    }
    if (one_expert) {
        load_smooth<VPL>(sreg, a, e0, nvec, TEAM, wit, lane);
#pragma unroll
        for (int t = 1; t < PD && t < T; ++t)
            load_x<VPL>(buf[t % NB], a.x, row_of(t), a.n, nvec, TEAM, wit, lane);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t + PD < T)
                load_x<VPL>(buf[(t + PD) % NB], a.x, row_of(t + PD), a.n, nvec, TEAM, wit, lane);
            __builtin_amdgcn_sched_barrier(0);
            convert_row<XT, SYM, OUT, VPL, TEAM>(a, buf[t % NB], sreg, row_of(t), t, nvec, slot, TEAM, wit, lane, red);
        }
    } else {
        // The rows straddle an expert boundary (rare): one row at a time,
        // each with its own expert's smooth scales.
        for (int t = 0; t < T; ++t) {
            if (t > 0)
                load_x<VPL>(buf[0], a.x, row_of(t), a.n, nvec, TEAM, wit, lane);
            load_smooth<VPL>(sreg, a, row_expert(row_of(t), gi_lane, a, lane), nvec, TEAM, wit, lane);
            convert_row<XT, SYM, OUT, VPL, TEAM>(a, buf[0], sreg, row_of(t), t, nvec, slot, TEAM, wit, lane, red);
        }
    }
}

// Team variant: a workgroup is one team of W = blockDim.x / 64 waves whose
// W * VPL * 64 lanes' vectors cover the row exactly (the host picks it when
// the vector variant's fixed teams of 1, 2 or 4 waves would leave lanes
// holding duplicate vectors: bf16 [*, 7168] is 896 vectors, 7 waves of 2
// per lane instead of 4 waves of 4 with 128 duplicates).  Each team converts
// T rows with the next PD rows' loads in flight, then the workgroup exits;
// rows are assigned as in the vector variant.  T = 4, PD = 1 in general.
// Long inputs without a group index (a.long_teams > 0) take the long
// schedule: L = a.long_teams teams of T = 13 rows strided by L, PD = 2,
// about two workgroups per compute unit with up to three rows of loads
// outstanding each; the rows from 13 L on go to short workgroups of two
// consecutive rows (blockIdx.x >= L), which fill the third workgroup slot
// of the compute units as they free.  bf16 [8192, 7168], interleaved runs:
// 16 strided rows per team 30.8-30.9 against 31.3-31.4 us for 4 (deeper
// prefetch measured slower: 31.5 us with PD = 3, 32.2 with 4); 14 strided
// rows plus the short workgroups a further 1-1.7% in three sessions, and
// 13 another 0.7% (12 and three-row short workgroups measured slower).
template <int XT, bool SYM, int OUT, int VPL, int T, int PD>
__global__ __launch_bounds__(kDqMaxTeam * kWave) void dq_team_kernel(DqArgs a)
{
    constexpr int NB = PD + 1;  // row buffers
    const int lane = threadIdx.x & (kWave - 1);
    const int wit = threadIdx.x / kWave;
    const int team = blockDim.x / kWave;
    const int64_t nvec = a.n >> 3;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * T;
    __shared__ float2 red[2][kDqMaxTeam];
    if (a.long_teams > 0 && static_cast<int64_t>(blockIdx.x) >= a.long_teams) {
        // Short workgroup: kDqTeamShortRows consecutive rows after the
        // strided teams' rows, all loaded at once with the smooth scales.
        constexpr int TS = kDqTeamShortRows;
        const int64_t base = a.long_teams * T + (static_cast<int64_t>(blockIdx.x) - a.long_teams) * TS;
        auto row_s = [&](int t) -> int64_t {
            const int64_t r = base + t;
            return r < a.rows ? r : a.rows - 1;
        };
        uint4 sb[TS][VPL];
        float ss[VPL][8];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            load_x<VPL>(sb[t], a.x, row_s(t), a.n, nvec, team, wit, lane);
            if (t == 0)
                load_smooth<VPL>(ss, a, 0, nvec, team, wit, lane);
        }
#pragma unroll
        for (int t = 0; t < TS; ++t)
            convert_row<XT, SYM, OUT, VPL, kDqMaxTeam>(a, sb[t], ss, row_s(t), t, nvec, 0, team, wit, lane, red);
        return;
    }
    const int64_t stride = a.long_teams > 0 ? a.long_teams : static_cast<int64_t>(gridDim.x);
    auto row_of = [&](int t) -> int64_t {
        const int64_t r = a.gi ? r0 + t : static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(t) * stride;
        return r < a.rows ? r : a.rows - 1;
    };

    const bool moe = a.gi != nullptr;
    int32_t gi_lane = 0;
    if (moe)
        gi_lane = a.gi[lane < a.n_experts ? lane : a.n_experts - 1];

    uint4 buf[NB][VPL];
    load_x<VPL>(buf[0], a.x, row_of(0), a.n, nvec, team, wit, lane);

    float sreg[VPL][8];
    int64_t e0 = 0;
    bool one_expert = true;
    if (moe && a.smooth) {
        const int64_t r_last = r0 + T - 1 < a.rows ? r0 + T - 1 : a.rows - 1;
        e0 = row_expert(r0, gi_lane, a, lane);
        one_expert = e0 == row_expert(r_last, gi_lane, a, lane);  // workgroup-uniform
    }
    if (one_expert) {
        load_smooth<VPL>(sreg, a, e0, nvec, team, wit, lane);
#pragma unroll
        for (int t = 1; t < PD && t < T; ++t)
            load_x<VPL>(buf[t % NB], a.x, row_of(t), a.n, nvec, team, wit, lane);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            if (t + PD < T)
                load_x<VPL>(buf[(t + PD) % NB], a.x, row_of(t + PD), a.n, nvec, team, wit, lane);
            __builtin_amdgcn_sched_barrier(0);
            convert_row<XT, SYM, OUT, VPL, kDqMaxTeam>(a, buf[t % NB], sreg, row_of(t), t, nvec, 0, team, wit, lane,
                                                       red);
        }
    } else {
        for (int t = 0; t < T; ++t) {
            if (t > 0)
                load_x<VPL>(buf[0], a.x, row_of(t), a.n, nvec, team, wit, lane);
            load_smooth<VPL>(sreg, a, row_expert(row_of(t), gi_lane, a, lane), nvec, team, wit, lane);
            convert_row<XT, SYM, OUT, VPL, kDqMaxTeam>(a, buf[0], sreg, row_of(t), t, nvec, 0, team, wit, lane, red);
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
    case 1: return dq_vec_kernel<XT, SYM, OUT, 1, TEAM>;
    case 2: return dq_vec_kernel<XT, SYM, OUT, 2, TEAM>;
    case 4: return dq_vec_kernel<XT, SYM, OUT, 4, TEAM>;
    }
    if constexpr (TEAM == kDqWaves) {  // only the widest rows take more vectors per lane
        if (vpl == 8)
            return dq_vec_kernel<XT, SYM, OUT, 8, TEAM>;
        if (vpl == 16)
            return dq_vec_kernel<XT, SYM, OUT, 16, TEAM>;
    }
    return nullptr;
}

template <int XT, bool SYM, int OUT>
KernelFn pick(const DqPlan& p)
{
    if (p.variant == DQ_VAR_TEAM) {
        constexpr int TL = kDqTeamStridedRows, PL = kDqTeamPrefetchLong;
        switch (p.vpl) {
        case 1: return p.long_rows ? dq_team_kernel<XT, SYM, OUT, 1, TL, PL> : dq_team_kernel<XT, SYM, OUT, 1, kDqTeamRows, 1>;
        case 2: return p.long_rows ? dq_team_kernel<XT, SYM, OUT, 2, TL, PL> : dq_team_kernel<XT, SYM, OUT, 2, kDqTeamRows, 1>;
        }
        return nullptr;
    }
    if (p.variant != DQ_VAR_VECTOR)
        return dq_generic_kernel<XT, SYM, OUT>;
    switch (p.team) {
    case 1: return pick_vpl<XT, SYM, OUT, 1>(p.vpl);
    case 2: return pick_vpl<XT, SYM, OUT, 2>(p.vpl);
    case 4: return pick_vpl<XT, SYM, OUT, 4>(p.vpl);
    }
    if constexpr (kDqWaves >= 8) {
        if (p.team == 8)
            return pick_vpl<XT, SYM, OUT, 8>(p.vpl);
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

}  // namespace

hipError_t launch_dynamic_quant(const DqPlan& p, hipStream_t stream)
{
    KernelFn fn = p.x_type == X_F16 ? pick_x<X_F16>(p) : pick_x<X_BF16>(p);
    if (!fn)
        return hipErrorInvalidValue;
    DqArgs a{p.x, p.smooth, p.group_index, p.n_experts, p.rows, p.n, p.y, p.scale, p.offset, 0};
    // Vector variant: one workgroup per T * 4/TEAM rows; team variant: one
    // per kDqTeamRows rows (long schedule: below); generic: one per row.
    int64_t rpb = 1;
    int threads = kBlock;
    if (p.variant == DQ_VAR_VECTOR) {
        rpb = dq_rows_per_team(p.vpl, p.team) * (kDqWaves / p.team);
        threads = kDqWaves * kWave;
    } else if (p.variant == DQ_VAR_TEAM) {
        if (p.team < 2 || p.team > kDqMaxTeam)
            return hipErrorInvalidValue;
        if (p.long_rows && p.group_index)
            return hipErrorInvalidValue;
        rpb = p.long_rows ? kDqTeamRowsLong : kDqTeamRows;
        threads = p.team * kWave;
    }
    int64_t blocks = (p.rows + rpb - 1) / rpb;
    if (p.variant == DQ_VAR_TEAM && p.long_rows) {
        // Long schedule: `blocks` strided teams of kDqTeamStridedRows rows,
        // then short workgroups for the rest (the teams cover fewer than all
        // rows: 13 ceil(rows / 16) < rows for rows >= 8192).
        a.long_teams = blocks;
        const int64_t rest = p.rows - blocks * kDqTeamStridedRows;
        if (rest <= 0)
            return hipErrorInvalidValue;
        blocks += (rest + kDqTeamShortRows - 1) / kDqTeamShortRows;
    }
    if (blocks > kMaxGridBlocks)
        return hipErrorInvalidValue;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<uint32_t>(blocks)), dim3(threads),
                           args, 0, stream);
}

}  // namespace dq
