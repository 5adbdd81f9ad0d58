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
    int vpl;   // 16-byte vectors per lane (vector variant)
    int team;  // waves per row (vector variant): 1, 2 or 4
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

// ---- mx block quantization ---------------------------------------------------
enum MxElem : int { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M1 = 2 };
enum MxVariant : int {
    MX_VAR_ROW = 0,      // axis 1, 16-byte loads, four lanes per 32-element block
    MX_VAR_COL = 1,      // axis 0, one lane per 8 columns of a 32-row block
    MX_VAR_GENERIC = 2,  // any shape and alignment, one thread per block
};

struct MxPlan {
    const void* x;
    int x_type;  // XType
    int64_t rows, n;
    int elem;    // MxElem
    int axis;    // 1: blocks along n; 0: blocks along rows
    void* y;
    uint8_t* scale;
    int variant;
};

// ---- weight-quantized matmul -------------------------------------------------
enum WqWeight : int { WQ_I8 = 0, WQ_I4 = 1 };
enum WqVariant : int {
    WQ_VAR_MFMA = 0,     // weights stored [n, k], matrix cores, no LDS
    WQ_VAR_GENERIC = 1,  // any layout: one thread per output element
};
enum WqTile : int {
    WQ_TILE_2x2 = 1,     // 17..128 rows: 2 x 2 blocks of 16 x 16 per wave, operands from global
    WQ_TILE_DECODE = 3,  // at most 16 rows: kWqDecodeCols blocks per wave, x1 staged in LDS
    WQ_TILE_GEMM = 4,    // more rows: 128 x 128 workgroup tiles, x1 and dequantized weights in LDS
};

struct WqPlan {
    const void* x1;
    const void* x2;
    const void* scale;
    const void* offset;  // nullptr: none
    const void* bias;    // nullptr: none
    const void* x3;      // nullptr: none
    void* out;
    int64_t m, k, n;
    int64_t group_size;  // > 0: per group
    int x_type;          // XType of x1, the parameters, bias, x3 and out
    int w_type;          // WqWeight
    int policy;          // dq_antiquant_policy: PER_TENSOR, PER_CHANNEL or PER_GROUP
    bool transpose_x2;   // weights stored [n, k]
    int variant;
    int tile;
    int splits;       // > 1: k split across workgroups, partial sums in the workspace
    int64_t k_chunk;  // k per split
};

// Matrix-core kernel geometry: k per superstep (four lane groups of 32) and
// supersteps whose loads are issued together, per register tile.
constexpr int kWqSuperK = 128;
constexpr int kWqDecodeCols = 1;  // 16-column blocks per wave in the decode kernel
constexpr int wq_batch(int tile)
{
    return tile == WQ_TILE_DECODE ? 2 : tile == WQ_TILE_2x2 ? 2 : 1;  // GEMM: one k-step of 128
}
constexpr int wq_tile_rows(int tile)
{
    return tile == WQ_TILE_DECODE ? 16 : tile == WQ_TILE_2x2 ? 32 : tile == WQ_TILE_GEMM ? 128 : 64;
}
constexpr int wq_tile_cols(int tile)  // four waves side by side
{
    return tile == WQ_TILE_DECODE ? 4 * 16 * kWqDecodeCols : tile == WQ_TILE_GEMM ? 128 : 4 * wq_tile_rows(tile);
}

// Kernel launchers (defined in the .hip files).  They enqueue on `stream`
// and return the launch status; they never synchronize.
hipError_t launch_dynamic_quant(const DqPlan& p, hipStream_t stream);
hipError_t launch_ada_layernorm_quant(const AdaPlan& p, hipStream_t stream);
hipError_t launch_antiquantize(const AqPlan& p, hipStream_t stream);
hipError_t launch_mx_quantize(const MxPlan& p, hipStream_t stream);
hipError_t launch_weight_quant_matmul(const WqPlan& p, void* workspace, hipStream_t stream);
hipError_t launch_copy_probe(void* dst, const void* src, size_t bytes, hipStream_t stream);

// DynamicQuant vector variant: waves per workgroup (the largest team), the
// most 16-byte vectors per lane a team takes before the next team size is
// used, rows a team has in flight ahead of the one it converts, and the
// largest row (in elements) it holds: 16 vectors of 8 elements per lane,
// 64 lanes, kDqWaves waves.
constexpr int kDqWaves = 4;
constexpr int kDqTeamVpl = 4;
constexpr int kDqPrefetch = 1;
constexpr int64_t kDqVecMaxPerWave = 16 * 8 * 64;
constexpr int64_t kDqVecMaxRow = kDqWaves * kDqVecMaxPerWave;

}  // namespace dq
