// launch.h -- internal launchers between the C-ABI layer (fp4q_api.cpp) and
// the kernels.  Every launcher assumes its arguments were validated on the
// host (shapes, alignment, modes) and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

constexpr int kMaxGroupsPerLaunch = 64;
// Persistent tile workgroups resident per XCD (32 CUs x 8 workgroups of 4 waves).
constexpr int kTileWgsPerXcd = 256;

inline void set_tile_grid(int32_t total_tiles, int32_t& per_xcd, int32_t& wgs_per_xcd)
{
    per_xcd = (total_tiles + 7) / 8;
    wgs_per_xcd = per_xcd < kTileWgsPerXcd ? per_xcd : kTileWgsPerXcd;
    if (wgs_per_xcd < 1) wgs_per_xcd = 1;
}

// Rowwise NVFP4 / AMDFP4 parameters (modes none, tensorwise, 1D outer).
struct RowArgs {
    const void* x;           // bf16 or FP32 (the launcher's x_f32), [rows, ld]
    int64_t rows, cols, ld;
    uint8_t* codes;          // may be null (qdq without codes)
    uint8_t* scales;         // may be null
    float* outer;            // 1D: [rows, cols/obs]; tensorwise: [1]
    float* residual;         // may be null
    void* y;                 // bf16 or FP32 (y_f32) [rows, cols], may be null
    const float* tensor_scale;  // tensorwise: device scalar holding s_g
    uint64_t seed, step, index_base;
    int32_t obs16;           // 1D outer: obs / 16 (1, 2, 4, 8)
    int32_t outer_given;     // 1: read outer instead of computing it
    int32_t x_vec;           // 1: x and every row start 16-byte aligned (vector loads)
    int32_t y_f32;           // 1: y is FP32
};

// Tile parameters (64 x 64 tiles walked as 2 x 2 super-tiles): cast-transpose,
// grouped cast-transpose, and the rowwise-only 2D outer and 16 x 16 inner
// modes.
struct TileArgs {
    const uint16_t* x;
    int64_t ld, cols;
    uint8_t* row_codes;
    uint8_t* row_scales;
    float* row_outer;
    uint8_t* col_codes;      // null: rowwise only
    uint8_t* col_scales;
    float* col_outer;        // 1D only
    float* residual;
    uint16_t* y;             // rowwise dequantised output (qdq), may be null
    const float* tensor_scale;
    uint64_t seed, step, index_base;
    int32_t obs16;           // 1D: obs / 16 (1, 2, 4); 2D: 4
    int32_t outer_given;
    int32_t inner_2d;        // 1: one inner scale per 16 x 16 tile (none, tensorwise, 2D outer)
    int32_t ngroups;
    int32_t tiles_c;         // super-tile (128 x 128) columns: ceil(cols / 128)
    int32_t total_tiles;     // super-tiles in the launch
    int32_t per_xcd;         // super-tiles in each XCD's contiguous slice
    int32_t wgs_per_xcd;     // persistent workgroups per XCD (grid = 8 * wgs_per_xcd)
    int32_t row0[kMaxGroupsPerLaunch + 1];   // prefix rows of the groups
    int32_t tile0[kMaxGroupsPerLaunch + 1];  // prefix unit counts of the groups (super-tiles, or tiles when staged)
    // Staged output (cast-transpose calls with an error-feedback residual, see
    // stage_applies): when `stage` is set, the walk unit is one 64 x 64 tile
    // (tiles_c = ceil(cols / 64), tile0 in tiles) and every code, scale byte and
    // 1D outer scale goes to the staging area (stage_block bytes per tile,
    // layout below) as whole 128-byte lines; the host then launches the
    // gather (launch_gather) that moves them into the row-major outputs.
    uint8_t* stage;          // 128-byte aligned, or null for direct stores
    int32_t stage_block;     // bytes per tile block
};

enum OuterKind { kOuterNone = 0, kOuterTensor = 1, kOuter1D = 2, kOuter2D = 3 };

// Staging area of a launch of T tiles, T * stage_block bytes in three regions,
// every part a multiple of 128 bytes:
//   [0, 2048 T)          rowwise codes, tile t's [64 rows][32 bytes] at 2048 t
//                        (t in the launch's row-major tile order);
//   [2048 T, 4096 T)     columnwise codes, tile (g, ti, tj)'s [64 columns][32
//                        bytes] at 2048 (T + tile0[g] + tj * tiles_r(g) + ti),
//                        i.e. each group's tiles column by column;
//   [4096 T, ...)        per tile t, at (stage_block - 4096) t, its tail:
//     [0, 256)           rowwise scale bytes [64 rows][4]
//     [256, 512)         columnwise scale bytes [64 columns][4]
//     1D outer groups of obs (16, 32, 64) elements:
//     [512, +ob)         rowwise outer scales [64 rows][64 / obs] FP32
//     [512 + ob, +ob)    columnwise outer scales [64 columns][64 / obs] FP32
//   with ob = 64 * (64 / obs) * 4.
// So the gather reads each row band's and each column band's codes as one
// contiguous run (grouped 32 x 2880^2 step: 678 -> 672 us against per-tile
// blocks holding all four parts).  kStageTail and kStageRowOuter are the tail
// parts' offsets plus 4096, as if the tail followed the two code blocks.
constexpr int32_t kStageCodes = 2048;     // one tile's codes of one direction
constexpr int32_t kStageTail = 4096;      // scales and outer scales, staged in LDS
constexpr int32_t kStageRowOuter = 4608;

inline int32_t stage_outer_bytes(int outer_kind, int obs)
{
    return outer_kind == kOuter1D ? 64 * (64 / obs) * 4 : 0;
}

// The cast-transpose calls that stage their outputs when given the scratch:
// those with an error-feedback residual (without 16 x 16 inner tiles).  There
// the residual's read and rewrite (8 of ~11 bytes per element) dominate, and
// the extra pass over the 1.125 bytes per element of codes and scales costs
// less than the partial-line stores it replaces (grouped 32 x 2880^2 step:
// 0.90 -> 0.82 ms); without a residual the extra pass costs more than it
// saves (16384 x 2880 1D SR: 0.100 -> 0.124 ms), so those store directly.
// Both paths give identical bytes.
inline bool stage_applies(bool sr, bool ef, int outer_kind, bool inner2d)
{
    (void)sr;
    (void)outer_kind;
    return ef && !inner2d;
}

inline int32_t stage_block_bytes(int outer_kind, int obs)
{
    return kStageRowOuter + 2 * stage_outer_bytes(outer_kind, obs);
}

// MXFP4 projection and FP8 re-encodings (every output may be null).
struct Mx8Args {
    const uint16_t* x;
    int64_t rows, cols, ld;
    uint16_t* y;               // bf16 [rows, cols]
    uint8_t* mx8_row;          // E4M3 [rows, cols]
    uint8_t* mx8_row_sc;       // UE8M0 [rows, cols / 32]
    uint8_t* mx8_col;          // E4M3 [cols, rows]
    uint8_t* mx8_col_sc;       // UE8M0 [cols, rows / 32]
    uint8_t* blk;              // E4M3 [rows, cols]
    uint8_t* blk_t;            // E4M3 [cols, rows]
    float* blk_sc;             // FP32 [rows / 128, cols / 128]
};

hipError_t launch_mx_fp8(const Mx8Args& a, hipStream_t s);

// C = A . B^T with MXFP4 operands (rowwise codes [rows, K/2], UE8M0 scales
// [rows, K/32]); K % 64 == 0.
struct GemmArgs {
    const uint8_t* a;          // codes of A [M, K/2]
    const uint8_t* as;         // scales of A [M, K/32]
    const uint8_t* b;          // codes of B [N, K/2]
    const uint8_t* bs;         // scales of B [N, K/32]
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;  // 256 x 256 tiles of C
    int32_t c_f32;             // 1: C is FP32, 0: bf16
    int32_t scale_layout;      // 0: rowwise, byte loads; 1: rowwise, 8-byte loads
                               // (K % 256 == 0, 8-byte aligned); 2: GEMM-ready tiled
    void* c;                   // [M, ldc]
    int64_t ldc;
};

hipError_t launch_mx_gemm(const GemmArgs& g, hipStream_t s);

// GEMM-ready scale layout [ceil(rows/256)][ceil(K/256)][256][8] from rowwise
// UE8M0 scales [rows, K/32] (zero padding).
hipError_t launch_mx_scales_tiled(const uint8_t* in, int64_t rows, int64_t K, uint8_t* out, hipStream_t s);

// x: bf16 (x_f32 = false) or FP32 [rows, ld]; x_vec: x and every row start
// 16-byte aligned.  y: bf16 or FP32 (y_f32) [rows, cols].
hipError_t launch_mx_qdq(const void* x, bool x_f32, bool x_vec, int64_t rows, int64_t cols, int64_t ld, void* y,
                         bool y_f32, uint8_t* codes, uint8_t* scales, hipStream_t s);

hipError_t launch_amax(int scale_bias, const void* x, bool x_f32, bool x_vec, int64_t rows, int64_t cols, int64_t ld,
                       const float* residual, float* partials, int npartials, float* scale_out,
                       float* user_outer, hipStream_t s);

hipError_t launch_rows(int scale_bias, int outer_kind, bool stochastic, bool x_f32, const RowArgs& a,
                       hipStream_t s);

hipError_t launch_tiles(int scale_bias, int outer_kind, bool stochastic, const TileArgs& a, hipStream_t s);

// FP32 scales of 1D outer groups of 128 elements (both directions) for the
// groups of a tile launch, written to its row_outer / col_outer before the
// tile kernel reads them as precomputed scales (kernels_outer.hip).
hipError_t launch_outer128(int scale_bias, const TileArgs& a, hipStream_t s);

// Gather pass of the staged cast-transpose (kernels_stage.hip): the blocks of
// one tile-kernel launch into the rowwise and columnwise buffers.
struct GatherArgs {
    const uint8_t* stage;
    int32_t stage_block;
    int32_t ngroups;
    int64_t cols;
    int32_t tiles_c;         // ceil(cols / 64)
    int32_t obs;             // 1D outer group size, 0 without 1D outer scales
    int32_t scales4;         // 1: every scale row is a whole number of 4-byte words, buffers 4-byte aligned
    int32_t row0[kMaxGroupsPerLaunch + 1];
    int32_t tile0[kMaxGroupsPerLaunch + 1];   // prefix tile counts (ceil(rows / 64) * tiles_c)
    uint8_t* row_codes;
    uint8_t* row_scales;
    float* row_outer;        // 1D only
    uint8_t* col_codes;
    uint8_t* col_scales;
    float* col_outer;        // 1D only
    // filled by launch_gather: work units per output kind (prefix) and lines per unit
    int32_t kind_units[7];
    int32_t lines[6];
};

hipError_t launch_gather(GatherArgs a, hipStream_t s);

hipError_t launch_dequant_nv(int scale_bias, int outer_kind, int outer_transposed, int obs,
                             const uint8_t* codes, const uint8_t* scales, const float* outer,
                             int64_t rows, int64_t cols, void* y, bool y_f32, hipStream_t s);

hipError_t launch_dequant_mx(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                             void* y, bool y_f32, hipStream_t s);

// partial maxima used by the tensorwise amax pass
constexpr int kAmaxPartials = 512;

// Rowwise tensorwise calls on at most this many elements and without an
// error-feedback residual run in one launch: every workgroup reads the whole
// (cache-resident) tensor for its amax instead of a grid-wide amax pass and a
// scale pass before the quantiser.
constexpr int64_t kSmallTensorElems = (int64_t)1 << 18;

}  // namespace fp4q
