// dq_internal.h -- plans shared between the host validation layer
// (dquant_api.cpp) and the kernel launchers (*.hip).  Not installed.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "dquant.h"

namespace dq {

// Element codes used inside the kernels.
enum XType : int { X_F16 = 0, X_BF16 = 1 };
enum OutKind : int { OUT_I8 = 0, OUT_I4 = 1 };  // INT32 output shares the INT4 bytes

// ---- DynamicQuant --------------------------------------------------------
enum DqVariant : int {
    DQ_VAR_VECTOR = 0,   // row held in VGPRs, 16-byte loads, TEAM waves per row
    DQ_VAR_GENERIC = 1,  // one workgroup per row, element loads, two passes
    DQ_VAR_TEAM = 2,     // a workgroup is one team whose waves cover the row exactly
};

struct DqPlan {
    const void* x;
    const float* smooth;       // nullptr: no smooth step
    const int32_t* group_index;  // nullptr: one smooth row for all rows
    int64_t n_experts;
    int64_t rows;
    int64_t n;
    int x_type;    // XType
    int out_kind;  // OutKind
    bool symmetric;
    void* y;
    float* scale;
    float* offset;
    // launch choice
    int variant;
    int vpl;   // 16-byte vectors per lane (vector and team variants)
    int team;  // waves per row: 1, 2 or 4 (vector variant), 2 .. kDqMaxTeam (team variant)
    bool long_rows;  // team variant: the long schedule (strided teams, then short workgroups)
};

// Largest grid (workgroups along x) a launch may use, and the largest row
// count any operation accepts (row indices stay below 2^31 in the kernels).
constexpr int64_t kMaxGridBlocks = 0x7FFFFFFF;

// ---- AdaLayerNorm-quant ----------------------------------------------------
enum AdaVariant : int { ADA_VAR_VECTOR = 0, ADA_VAR_GENERIC = 1 };

struct AdaPlan {
    const void* x;
    const void* scale;   // [B, H]
    const void* shift;   // [B, H]
    const void* weight;  // [H] or nullptr
    const void* bias;    // [H] or nullptr
    const float* smooth; // [H] or nullptr
    int64_t B, S, H;
    int x_type;  // XType; parameters share it
    float eps;
    int8_t* out;
    float* quant_scale;
    int variant;
    int vpl;
};

// ---- AntiQuantize ---------------------------------------------------------
enum SrcKind : int { SRC_I8 = 0, SRC_F8E4M3 = 1, SRC_F8E5M2 = 2, SRC_F4E2M1 = 3 };
enum ParamKind : int { PARAM_F32 = 0, PARAM_F16 = 1, PARAM_BF16 = 2, PARAM_E8M0 = 3 };
enum DstKind : int { DST_BF16 = 0, DST_F16 = 1, DST_F32 = 2 };

struct AqPlan {
    const void* src;
    const void* scale;
    const void* offset;  // nullptr: hasOffset = false
    int param_kind;      // ParamKind of scale and offset
    int64_t m, n;
    int policy;  // dq_antiquant_policy
    int k_dim;
    int64_t group_size;
    int src_kind;
    int dst_kind;
    void* dst;
};

// Kernel launchers (defined in the .hip files).  They enqueue on `stream`
// and return the launch status; they never synchronize.
hipError_t launch_dynamic_quant(const DqPlan& p, hipStream_t stream);
hipError_t launch_ada_layernorm_quant(const AdaPlan& p, hipStream_t stream);
hipError_t launch_antiquantize(const AqPlan& p, hipStream_t stream);
hipError_t launch_copy_probe(void* dst, const void* src, size_t bytes, hipStream_t stream);

// DynamicQuant vector variant: waves per workgroup (the largest team), the
// most 16-byte vectors per lane a team takes before the next team size is
// used, rows a team has in flight ahead of the one it converts, and the
// largest row (in elements) it holds: 16 vectors of 8 elements per lane,
// 64 lanes, kDqWaves waves.
constexpr int kDqWaves = 4;
// Team variant: the most waves a team (one workgroup) has, and the rows each
// team converts before the workgroup exits.  Inputs without a group index
// and with at least kDqTeamLongMinRows rows take the long schedule:
// ceil(rows / kDqTeamRowsLong) teams (about two workgroups per compute unit
// at that size) with kDqTeamPrefetchLong rows in flight ahead of the one
// converted.
constexpr int kDqMaxTeam = 16;
constexpr int kDqTeamRows = 4;
constexpr int kDqTeamRowsLong = 16;
constexpr int kDqTeamPrefetchLong = 2;
constexpr int64_t kDqTeamLongMinRows = 8192;
// The long schedule's split: ceil(rows / kDqTeamRowsLong) teams convert
// kDqTeamStridedRows strided rows each, and the rows after theirs go to
// short workgroups of kDqTeamShortRows consecutive rows.
constexpr int kDqTeamStridedRows = 13;
constexpr int kDqTeamShortRows = 2;
constexpr int kDqTeamVpl = 4;
constexpr int kDqPrefetch = 1;
constexpr int64_t kDqVecMaxPerWave = 16 * 8 * 64;
constexpr int64_t kDqVecMaxRow = kDqWaves * kDqVecMaxPerWave;

}  // namespace dq
