// dq_ext_internal.h -- plans shared between the host validation layer
// (dquant_api.cpp) and the kernel launchers of mx block quantization and the
// weight-quantized matmul.  Not installed.  (Kept apart from dq_internal.h,
// which the row-quantization kernels include.)
#pragma once

#include "dq_internal.h"

namespace dq {

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
    WQ_VAR_MFMA = 0,     // weights stored [n, k], matrix cores (decode or LDS-tiled kernel)
    WQ_VAR_GENERIC = 1,  // any layout: one thread per output element
};
enum WqTile : int {
    WQ_TILE_DECODE = 3,  // at most 16 rows: kWqDecodeCols blocks per wave, x1 staged in LDS
    WQ_TILE_GEMM = 4,    // more rows: 128 x 128 workgroup tiles, x1 and dequantized weights in LDS
    WQ_TILE_WIDE = 5,    // many rows: 256 x 256 workgroup tiles, x1 in LDS, weights straight to the operands
    WQ_TILE_BALANCED = 6,  // at most 16 rows, int4 in groups of 128: one 8-wave workgroup per CU, k split over its waves
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
constexpr int kWqDecodeCols = 1;   // 16-column blocks per wave in the decode kernel
constexpr int kWqDecodeWaves = 4;  // waves per decode workgroup (they share one x1 staging)
// LDS-tiled kernel: output tile and k-step (a divisor of kWqSuperK).
constexpr int kWqGemmRows = 128, kWqGemmCols = 128, kWqGemmK = 128;
// Wide kernel: output tile and k-step.  It is planned for at least 256 rows
// when the 256 x 256 tiles alone give kWqWideMinTiles workgroups or more
// (no k split), k is a multiple of two k-steps and the group size of one.
constexpr int kWqWideRows = 256, kWqWideCols = 256, kWqWideK = 64;
constexpr int64_t kWqWideMinTiles = 128;
// Balanced decode kernel: workgroups (one per compute unit of MI355X), the
// most 16-column blocks each takes, and the k multiple it needs (8 waves x
// parameter chunks of 1024).
constexpr int64_t kWqBalWorkgroups = 256;
constexpr int kWqBalMaxBlocks = 7;
constexpr int64_t kWqBalKMultiple = 8192;
// Wide kernel: x1 reaches LDS by direct-to-LDS buffer loads (three buffers)
// rather than through registers and LDS stores (two buffers).
constexpr bool kWqWideDma = true;
// Per-group parameters of the LDS-tiled kernel come in windows of this many
// groups when groups are one k-step long; k splits are then planned in
// multiples of the window.
constexpr int kWqParamWindow = 8;
// Supersteps per batch.  Decode: 256 bytes of each column's weights per
// batch (four supersteps of int4, two of int8); shorter runs per column
// (two int4 supersteps) and longer ones (eight), or more batches in flight,
// all measured slower.  GEMM: k splits in steps of 128.
constexpr int wq_batch(int tile, int weight)
{
    return tile == WQ_TILE_DECODE ? (weight == WQ_I4 ? 4 : 2) : 1;
}
constexpr int wq_tile_rows(int tile)
{
    return tile == WQ_TILE_DECODE ? 16 : kWqGemmRows;
}
constexpr int wq_tile_cols(int tile)
{
    return tile == WQ_TILE_DECODE ? kWqDecodeWaves * 16 * kWqDecodeCols : kWqGemmCols;  // decode: waves side by side
}

hipError_t launch_mx_quantize(const MxPlan& p, hipStream_t stream);
hipError_t launch_weight_quant_matmul(const WqPlan& p, void* workspace, hipStream_t stream);

// Library-owned split-k scratch of the allocation-free matmul entry point:
// its size, the most devices it is tracked on, and its address on the
// current device (looked up once per device, then cached).
constexpr size_t kWqScratchBytes = size_t{32} << 20;
constexpr int kWqScratchDevices = 64;
hipError_t wq_scratch_address(void** ptr);

}  // namespace dq
