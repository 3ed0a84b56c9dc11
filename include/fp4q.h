/*
 * fp4q.h -- C ABI of the MI355X (gfx950) block-scaled FP4 quantisation library
 * (libfp4q.so).
 *
 * The library quantises bf16 tensors to 4-bit E2M1 codes packed two per byte,
 * with one of three inner block scales and an optional FP32 level above them:
 *
 *   NVFP4   per-16 E4M3 scale of block_absmax/6 ("fp4-train" README, Method);
 *           may run on the UE5M3 grid ("NVFP4 / AMD-FP4 outer-block (two-level)
 *           scaling for FP4 training", Implementation: scale_format="ue5m3").
 *   AMDFP4  per-16 UE5M3 scale, grid max 114688 (same page, Background).
 *   MXFP4   per-32 (1x32) UE8M0 power-of-two scale, floor 2^-126, cap 2^125,
 *           E2M1 RTNE ("MXFP4 weight QAT recipes on MXFP8 and FP8 block-scaling
 *           hosts", Overview and Design).
 *
 *   inner geometry (NVFP4 / AMDFP4): 1 x 16 blocks along the quantisation axis,
 *           or 16 x 16 tiles sharing one scale ("Block-Scaled FP8 and FP4 Weight
 *           Quantization", section 6: the transpose-consistent weight recipe).
 *
 *   two-level scaling (NVFP4 / AMDFP4 only; ALTO page, Technical design):
 *     NONE        inner scales only;
 *     TENSORWISE  one FP32 scale amax/(scale_max*6) for the whole tensor;
 *     OUTER_BLOCK one FP32 scale amax/(scale_max*6) per 1 x obs row segment
 *                 (and obs x 1 column segment for the columnwise buffer), or
 *                 per obs x obs tile shared by both directions (outer_2d).
 *   rounding: RNE, or stochastic rounding keyed on (seed, step, global index)
 *   with an optional in-place FP32 error-feedback residual ("fp4-train"
 *   README, API and Method).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *     except where an argument says "host".  `stream` is a hipStream_t (NULL =
 *     the null stream).  Calls are asynchronous: FP4Q_OK means "enqueued".
 *   - x and y are bf16 tensors passed as their 16-bit patterns, row-major.
 *     x has leading dimension ld_x >= cols (elements); every other tensor is
 *     contiguous.
 *   - Packed codes: uint8 [rows, cols/2], element (i, j) in byte j/2, the low
 *     nibble holding the even column; a code is sign<<3 | m with m indexing
 *     the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}.
 *   - Inner scale bytes: uint8 [rows, cols/16] (E4M3 / UE5M3 code) or
 *     [rows, cols/32] (UE8M0 code), row-major, unswizzled.
 *   - Outer FP32 scales: TENSORWISE [1]; OUTER_BLOCK 2D [rows/obs, cols/obs];
 *     OUTER_BLOCK 1D rowwise [rows, cols/obs], columnwise [cols, rows/obs].
 *   - Columnwise buffers are the rowwise layout of X^T: codes [cols, rows/2],
 *     scales [cols, rows/16] ("Block-Scaled FP8 and FP4 Weight Quantization",
 *     sections 1-3).
 *   - The caller owns and allocates every buffer; the library never allocates
 *     device memory.  Inputs must not alias outputs, except `residual`, which
 *     is read and rewritten in place.
 *   - All validation happens on the host before anything is enqueued; on an
 *     error status nothing is launched and no output byte is written.
 *   - x, y, codes, residual and workspace must be 16-byte aligned, outer
 *     arrays 4-byte aligned (scale bytes have no requirement); ld_x must be a
 *     multiple of 8.
 *   - An empty tensor (rows == 0 or cols == 0) is valid: the configuration is
 *     validated, nothing is launched, and pointers may be NULL.
 *   - No global mutable state: calls are thread-safe.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 2

/* Status codes. */
enum {
    FP4Q_OK = 0,
    FP4Q_ERR_NULL = 1,        /* a required pointer is NULL                               */
    FP4Q_ERR_DTYPE = 2,       /* input or output dtype other than bf16 / fp32 (fp16 is
                                 rejected: its range is smaller than the FP4 grid times
                                 the scales, "MXFP4 weight QAT recipes", Guards)          */
    FP4Q_ERR_SHAPE = 3,       /* cols % 16 (32 for MXFP4), rows % 16 for columnwise,
                                 outer_block_size not a multiple of 16 or not dividing a
                                 reduction dimension (ALTO page, Technical design),
                                 ld_x < cols, negative sizes                              */
    FP4Q_ERR_MODE = 4,        /* illegal combination: tensorwise with outer knobs, outer
                                 knobs outside outer-block mode, MXFP4 with a two-level
                                 mode, scale format not allowed for the format, a
                                 precomputed outer scale without a two-level mode,
                                 16 x 16 inner tiles with MXFP4 or 1D outer blocks        */
    FP4Q_ERR_UNSUPPORTED = 5, /* valid on the pages but not built here (see the function) */
    FP4Q_ERR_ALIGN = 6,       /* a pointer not 16-byte aligned, ld_x % 8 != 0 (the
                                 rowwise entry points accept any x aligned to its element
                                 size and any ld_x >= cols)                               */
    FP4Q_ERR_WORKSPACE = 7,   /* workspace smaller than fp4q_workspace_bytes()            */
    FP4Q_ERR_HIP = 8,         /* the HIP runtime reported a launch error                  */
    FP4Q_ERR_ABI = 9          /* cfg->abi_version != FP4Q_ABI_VERSION                     */
};

typedef enum { FP4Q_NVFP4 = 0, FP4Q_AMDFP4 = 1, FP4Q_MXFP4 = 2 } fp4q_format;
/* DEFAULT resolves to E4M3 (NVFP4), UE5M3 (AMDFP4), UE8M0 (MXFP4). */
typedef enum { FP4Q_SCALE_DEFAULT = 0, FP4Q_SCALE_E4M3 = 1, FP4Q_SCALE_UE5M3 = 2, FP4Q_SCALE_UE8M0 = 3 } fp4q_scale_format;
typedef enum { FP4Q_TWO_LEVEL_NONE = 0, FP4Q_TENSORWISE = 1, FP4Q_OUTER_BLOCK = 2 } fp4q_two_level;
typedef enum { FP4Q_RNE = 0, FP4Q_STOCHASTIC = 1 } fp4q_rounding;
typedef enum { FP4Q_DTYPE_BF16 = 0, FP4Q_DTYPE_FP16 = 1, FP4Q_DTYPE_FP32 = 2 } fp4q_dtype;

/* Per-call configuration (plain data, passed by host pointer). */
typedef struct {
    uint32_t abi_version;      /* must equal FP4Q_ABI_VERSION                                  */
    int32_t format;            /* fp4q_format                                                 */
    int32_t scale_format;      /* fp4q_scale_format                                           */
    int32_t two_level;         /* fp4q_two_level                                              */
    int32_t outer_block_size;  /* obs, OUTER_BLOCK only (0 otherwise); multiple of 16          */
    int32_t outer_2d;          /* OUTER_BLOCK only: 1 = obs x obs tiles, 0 = 1 x obs segments */
    int32_t rounding;          /* fp4q_rounding                                               */
    int32_t outer_mode;        /* 0: compute and write the outer scales; 1: read them from the
                                  outer buffers (a precomputed scale, ALTO page,
                                  Implementation: precomputed_outer_scale)                     */
    int32_t input_dtype;       /* fp4q_dtype of x: BF16, or FP32 for fp4_quantize / fp4_qdq in
                                  modes NONE, TENSORWISE and 1D OUTER_BLOCK and for MXFP4
                                  ("fp4-train" README, Requirements and limits: float32 or
                                  bfloat16 input; "MXFP4 weight QAT recipes", Correctness:
                                  fake-quant on bf16 and fp32).  A bf16 value widens to FP32
                                  exactly, so both give the same result on bf16 values.
                                  FP16: FP4Q_ERR_DTYPE.                                        */
    int32_t inner_2d;          /* NVFP4 / AMDFP4 inner scale geometry: 0 = one scale per 1 x 16
                                  block along the quantisation axis; 1 = one scale per 16 x 16
                                  tile of the source, from the largest normalised magnitude of
                                  all its 256 values ("Block-Scaled FP8 and FP4 Weight
                                  Quantization", section 6).  The scale byte is replicated for
                                  each of the tile's 16 rows in row_scales (the 1 x 16 microblock
                                  layout, same section), and the columnwise codes and scales are
                                  the transposes of the rowwise ones: one quantisation decision
                                  per element serves both directions.  Needs rows % 16 == 0;
                                  not with MXFP4 or 1D outer blocks (their scales differ per
                                  direction): FP4Q_ERR_MODE.                                   */
    int32_t output_dtype;      /* fp4q_dtype of y in fp4_qdq and fp4_dequantize: BF16 (RNE of
                                  the FP32 dequantised value) or FP32 (that value itself;
                                  "MXFP4 weight QAT recipes", Correctness: bf16 and fp32
                                  dequantise targets); FP32 with the 64 x 64 tile modes (2D
                                  outer, inner_2d): FP4Q_ERR_UNSUPPORTED; FP16: FP4Q_ERR_DTYPE.
                                  Ignored by entry points without a y of this kind.            */
    uint64_t seed;             /* SR key                                                       */
    uint64_t step;             /* SR step (counter high word)                                  */
    uint64_t index_base;       /* SR global index of element (0, 0): element (i, j) draws with
                                  index index_base + i*cols + j (shards, experts)              */
} fp4q_cfg;

/* Byte sizes of every buffer an entry point may touch, for (cfg, rows, cols).
 * A size of 0 means the buffer is not used by that configuration. */
typedef struct {
    size_t row_codes, row_scales, row_outer;
    size_t col_codes, col_scales, col_outer;   /* col_outer == 0 when it is shared */
    size_t y;                                  /* dequantised output (output_dtype)  */
    size_t residual;                           /* FP32 error-feedback residual       */
    size_t workspace;                          /* scratch the caller must provide    */
} fp4q_sizes;

/* ABI version compiled into the library. */
uint32_t fp4q_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* fp4q_status_str(int status);

/* Fills *out for an [rows, cols] source quantised by cfg.  Columnwise sizes are
 * those of fp4_cast_transpose.  Returns a status (validation as for the
 * entry points, without pointer checks). */
int fp4q_buffer_sizes(const fp4q_cfg* cfg, int64_t rows, int64_t cols, fp4q_sizes* out);

/* Workspace bytes the entry points need for cfg and shape (0 unless
 * TENSORWISE computes its scale: then a small array of partial maxima). */
size_t fp4q_workspace_bytes(const fp4q_cfg* cfg, int64_t rows, int64_t cols);

/* Workspace bytes for fp4_cast_transpose (groups = 1, rows_per_group =
 * &rows) and fp4_cast_transpose_grouped (host array of the G row counts), for
 * a call with (with_residual = 1) or without (0) an error-feedback residual:
 * the tensorwise partial maxima when the scale is computed, plus, for a call
 * with a residual (outer blocks of up to 64 elements, 16 x 16 inner tiles
 * excluded), one tile-major block per 64 x 64 tile of the largest launch
 * (4608 bytes, more with 1D outer scales) and 128 bytes of alignment slack.
 * Given at least this much, such a call stages its outputs: the tile kernel
 * writes every code, scale byte and 1D outer scale as whole 128-byte lines of
 * that scratch and a second kernel writes whole lines of the final buffers.
 * The results are identical; HBM time is lower where rows of the output
 * buffers are not whole 128-byte lines.  With less, the outputs are stored
 * directly (the tensorwise part must still be there).  0 for an invalid
 * configuration. */
size_t fp4q_cast_transpose_workspace_bytes(const fp4q_cfg* cfg, int32_t groups, const int64_t* rows_per_group,
                                           int64_t cols, int32_t with_residual);

/*
 * fp4_quantize -- rowwise quantisation ("fp4-train" README, API: quantize(x,
 * stochastic, residual, seed, step)).
 *   x         bf16 or FP32 (cfg->input_dtype) [rows, ld_x] device, read.  In
 *             modes NONE, TENSORWISE, 1D OUTER_BLOCK and MXFP4, x may be a view
 *             aligned only to its element size with any ld_x >= cols (a
 *             misaligned view: "MXFP4 weight QAT recipes", Correctness); the
 *             64 x 64 tile modes (2D outer, inner_2d) need bf16, a 16-byte
 *             aligned x and ld_x % 8 == 0.
 *   codes     uint8 [rows, cols/2] device, written.
 *   scales    uint8 [rows, cols/16] (cols/32 for MXFP4) device, written.
 *   outer     FP32 outer scales (layout above) device; written when
 *             cfg->outer_mode == 0, read when 1; NULL only for mode NONE/MXFP4.
 *   residual  FP32 [rows, cols] device or NULL.  When given, the value quantised
 *             is RN(x + residual) and residual is rewritten in place with
 *             RN(value - dequantised value) (error feedback, "fp4-train"
 *             README, Method).  NVFP4/AMDFP4 only.  Its values must be
 *             finite.  NaN / inf sanitisation (NaN -> +0, +-inf -> +-largest
 *             bf16; ALTO page, Op-level test coverage) applies to the value
 *             quantised, the sum: a NaN x gives +0, an infinite x or an
 *             overflowing sum the signed largest bf16.
 *   workspace device scratch of >= fp4q_workspace_bytes() bytes (NULL if 0).
 * OUTER_BLOCK 2D needs rows % obs == 0 and supports obs == 64; 1D supports
 * obs in {16, 32, 64, 128} (others: FP4Q_ERR_UNSUPPORTED).  MXFP4 supports RNE
 * only and no residual.  With cfg->inner_2d, rows % 16 == 0 (FP4Q_ERR_SHAPE
 * otherwise) and scales hold each 16 x 16 tile's byte in every one of its rows.
 */
int fp4_quantize(const fp4q_cfg* cfg, const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                 uint8_t* codes, uint8_t* scales, float* outer, float* residual,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp4_dequantize -- bf16 or FP32 from stored codes and scales ("fp4-train"
 * README, API: dequantize(packed, scale, M, K); ALTO page, Implementation:
 * convert_from).  w = RN(+-G[m] * dec(s_i) [* s_o]), y = bf16(w) or, with
 * cfg->output_dtype FP32, w itself; an MXFP4 scale byte 0xFF (NaN) gives the
 * quiet NaN (0x7FC0, 0x7FC00000).
 *   codes, scales, outer  as written by the entry points for a logical
 *                         [rows, cols] buffer (device, read).
 *   outer_transposed      1 when a 2D outer array belongs to the transpose of
 *                         this buffer, i.e. is [cols/obs, rows/obs] -- the case
 *                         of a columnwise buffer sharing its source's 2D outer
 *                         scale; 0 otherwise.
 *   y                     bf16 or FP32 [rows, cols] device, 16-byte aligned,
 *                         written.
 * rounding, seed, step, index_base and input_dtype are ignored; so is inner_2d,
 * whose replicated scale layout dequantises exactly like 1 x 16 blocks.
 */
int fp4_dequantize(const fp4q_cfg* cfg, const uint8_t* codes, const uint8_t* scales, const float* outer,
                   int64_t rows, int64_t cols, int32_t outer_transposed, void* y, void* stream);

/*
 * fp4_qdq -- quantise then dequantise, rowwise ("fp4-train" README, API: qdq;
 * "MXFP4 weight QAT recipes", Design: the fused bf16 -> mxfp4 -> bf16
 * projection is fp4_qdq with format MXFP4).
 *   x         as in fp4_quantize (bf16 or FP32, misaligned views).
 *   y         bf16 or FP32 (cfg->output_dtype) [rows, cols] device, 16-byte
 *             aligned, written.
 *   codes, scales, outer  optional outputs as in fp4_quantize (NULL to skip;
 *             outer is required when outer_mode == 1).
 *   residual, workspace   as in fp4_quantize.
 */
int fp4_qdq(const fp4q_cfg* cfg, const void* x, int64_t rows, int64_t cols, int64_t ld_x,
            void* y, uint8_t* codes, uint8_t* scales, float* outer, float* residual,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp4_qdq_noalloc -- fp4_qdq for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, results and errors as fp4_qdq, without the
 * workspace: the scratch fp4_qdq would take from it (the tensorwise mode's
 * partial maxima and global scale, fp4q_workspace_bytes() bytes) is a 4 KiB
 * device array inside the library, one per GPU, held until the process ends.
 * A configuration needing more scratch than that returns FP4Q_ERR_WORKSPACE
 * (none does today).  The library looks up the array's device address once
 * per device, on the first call made with that device current; it calls no
 * allocator.  All calls on one GPU share that GPU's array: calls that overlap
 * in time on one GPU (concurrent streams) race and give undefined results.
 */
int fp4_qdq_noalloc(const fp4q_cfg* cfg, const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                    void* y, uint8_t* codes, uint8_t* scales, float* outer, float* residual, void* stream);

/*
 * fp4_cast_transpose -- one read of x writes the rowwise buffers and the
 * columnwise buffers (the rowwise layout of X^T) ("Block-Scaled FP8 and FP4
 * Weight Quantization", sections 2-3: fused cast-transpose; ALTO page,
 * Implementation: an axis-invariant 2D outer scale computed once and used by
 * both directions).  NVFP4 / AMDFP4 only; x bf16 [rows, ld_x] (input_dtype
 * FP32: FP4Q_ERR_UNSUPPORTED), 16-byte aligned, ld_x % 8 == 0.
 *   row_codes [rows, cols/2], row_scales [rows, cols/16], row_outer (layout
 *   above) -- device, written (row_outer read when outer_mode == 1).
 *   col_codes [cols, rows/2], col_scales [cols, rows/16] -- device, written.
 *   col_outer  1D: [cols, rows/obs] (written, or read when outer_mode == 1).
 *              2D and TENSORWISE: the scale is shared, col_outer must be NULL or
 *              equal row_outer.
 *   residual   FP32 [rows, cols] or NULL; updated from the ROWWISE dequantised
 *              value; the columnwise direction reads the same value but does not
 *              update it.
 * Needs rows % 16 == 0.  OUTER_BLOCK supports obs == 64 (1D and 2D); 1D also
 * obs in {16, 32, 128} (groups of 128 span two 64 x 64 tiles: a first kernel
 * computes their scales, then the tile kernel reads them; one more read of x
 * and the residual).  Element (i, j) draws its SR variate once and uses it in
 * both directions.  With cfg->inner_2d the columnwise codes and scales are
 * exactly the transposes of the rowwise ones.
 */
int fp4_cast_transpose(const fp4q_cfg* cfg, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                       uint8_t* row_codes, uint8_t* row_scales, float* row_outer,
                       uint8_t* col_codes, uint8_t* col_scales, float* col_outer,
                       float* residual, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp4_cast_transpose_grouped -- fp4_cast_transpose of G independent groups
 * (experts) stacked along rows, in one launch (ALTO page, Implementation:
 * grouped MoE GEMM with a per-expert outer scale).
 *   groups          G >= 0.
 *   rows_per_group  HOST array of G row counts (each a multiple of 16, and of
 *                   obs in OUTER_BLOCK mode).
 *   x               bf16 [sum(rows), ld_x] device (16-byte aligned, ld_x % 8 == 0;
 *                   input_dtype FP32: FP4Q_ERR_UNSUPPORTED).
 *   row_codes/row_scales/residual  stacked along rows exactly as for one tensor
 *                   of sum(rows) rows.
 *   col_codes, col_scales  group g's [cols, rows_g/2] and [cols, rows_g/16]
 *                   buffers, stored one after another in group order.
 *   row_outer, col_outer   group g's outer arrays one after another (2D
 *                   [rows_g/obs, cols/obs]; 1D rowwise [rows_g, cols/obs] -- which
 *                   is again plain row stacking -- and columnwise
 *                   [cols, rows_g/obs]; TENSORWISE one value per group).
 * Group g draws SR variates with index_base + (rows before g) * cols + i*cols + j,
 * the global row-major index in the stacked tensor, so the result equals G
 * single calls (also with cfg->inner_2d).  TENSORWISE is not supported here
 * (FP4Q_ERR_UNSUPPORTED).
 */
int fp4_cast_transpose_grouped(const fp4q_cfg* cfg, int32_t groups, const int64_t* rows_per_group,
                               int64_t cols, const uint16_t* x, int64_t ld_x,
                               uint8_t* row_codes, uint8_t* row_scales, float* row_outer,
                               uint8_t* col_codes, uint8_t* col_scales, float* col_outer,
                               float* residual, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp4_mx_project_fp8 -- the MXFP4 projection of a bf16 weight and its FP8
 * re-encodings from one read of the weight ("MXFP4 weight QAT recipes on MXFP8
 * and FP8 block-scaling hosts", Overview, Design, Correctness: the projected
 * weight feeds MXFP8 and Float8 128x128 block-scaling hosts; the rowwise MXFP8
 * encoding is bitwise lossless, the 128x128 encoding lossless within a tile's
 * E4M3 headroom, the columnwise MXFP8 encoding a bounded re-quantisation).
 * cfg: format MXFP4 (RNE, no two-level mode), input and output dtype BF16
 * (FP32: FP4Q_ERR_UNSUPPORTED).  With y the bf16 projection
 * (as fp4_qdq writes it) every output is optional (NULL skips it):
 *   y              bf16 [rows, cols]
 *   mx8_row        E4M3 [rows, cols] and mx8_row_scales UE8M0 [rows, cols/32]:
 *                  1 x 32 blocks along rows, scale 2^E with
 *                  E = floor(log2(amax)) - 8 (the OCP microscaling rule for
 *                  E4M3) clamped to [-127, 127], amax over the block's finite
 *                  values (code 0 when there is none);
 *   mx8_col        E4M3 [cols, rows] and mx8_col_scales UE8M0 [cols, rows/32]:
 *                  the same on 32 x 1 blocks, stored as the rowwise layout of
 *                  y^T (needs rows % 32 == 0);
 *   blk            E4M3 [rows, cols], blk_t E4M3 [cols, rows] (its transpose)
 *                  and blk_scales FP32 [rows/128, cols/128]: 128 x 128 blocks
 *                  with the smallest power-of-two scale s for which
 *                  amax / s <= 448 (1 for a block without a finite nonzero
 *                  value); needs rows % 128 == 0 and cols % 128 == 0.
 * Payload = E4M3 of y / scale, round to nearest even with subnormals, sign kept
 * (also for zero); a NaN element of y (a poisoned MXFP4 block) encodes as 0xFF.
 * mx8_row and mx8_row_scales are given together or not at all, likewise
 * mx8_col and mx8_col_scales.  Needs cols % 32 == 0; rows and ld_x up to 2^22
 * (FP4Q_ERR_UNSUPPORTED beyond).  x, y, mx8_row, mx8_col, blk and blk_t
 * 16-byte aligned, ld_x % 8 == 0, blk_scales 4-byte aligned.
 */
int fp4_mx_project_fp8(const fp4q_cfg* cfg, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                       uint16_t* y, uint8_t* mx8_row, uint8_t* mx8_row_scales, uint8_t* mx8_col,
                       uint8_t* mx8_col_scales, uint8_t* blk, uint8_t* blk_t, float* blk_scales, void* stream);

/*
 * fp4_mm -- C = A . B^T with MXFP4 operands on gfx950's FP4 matrix cores
 * ("fp4-train" README, API: fp4_mm(a, b) is a @ b^T on the FP4 tensor cores;
 * Correctness: the FP4 GEMM equals the dequantise-then-multiply path).
 *   cfg        format MXFP4; output_dtype BF16 or FP32 is the type of C; the
 *              other fields are ignored.
 *   a_codes    uint8 [M, K/2] and a_scales uint8 [M, K/32]: A's rowwise MXFP4
 *              buffers as fp4_quantize writes them (device, read).
 *   b_codes    uint8 [N, K/2] and b_scales uint8 [N, K/32]: B's, B being
 *              [N, K] (both operands K-major).
 *   scale_layout  0: a_scales / b_scales are the rowwise [rows, K/32] buffers
 *              above; 1: both are in the GEMM-ready layout fp4_mx_scales_tiled
 *              writes (the faster path for every K).
 *   c          [M, ldc] device (ldc >= N), written, not accumulated into; bf16
 *              is the RNE of the FP32 sum.
 * Every product of two E2M1 values and two power-of-two scales is exact; the
 * sums accumulate in binary32 in an order of the kernel's choosing, so
 * |C - exact| <= (K - 1) 2^-24 sum_k |a_ik b_jk| (plus the bf16 rounding).
 * Needs K % 64 == 0 (FP4Q_ERR_SHAPE), K <= 2^22 and M, N <= 2^24
 * (FP4Q_ERR_UNSUPPORTED), code buffers 16-byte aligned and c aligned to its
 * element (FP4Q_ERR_ALIGN).  M == 0 or N == 0 writes nothing; K == 0 writes
 * zeros.  The kernel depends on the scale layout and C's dtype and, for
 * scale_layout 1, on the shape: K >= 8192 with at least 1024 tiles of
 * 256 x 256 (8192 x 8192 and up) takes a direct-to-LDS kernel, the rest a
 * register-staged one; both give bit-identical C.  The first call that selects
 * a kernel raises its LDS limit (a host-side attribute); later calls only
 * enqueue, so they may be captured in a HIP graph.
 */
int fp4_mm(const fp4q_cfg* cfg, const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
           const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, int32_t scale_layout, void* c, int64_t ldc,
           void* stream);

/*
 * fp4_mx_scales_tiled -- the GEMM-ready ("MFMA-ready") layout of MXFP4 scales
 * ("Block-Scaled FP8 and FP4 Weight Quantization", section 2: the scale tensor
 * indexed in the block order the matrix-core kernel consumes, materialised
 * once and cached while the weight is unchanged).
 *   scales     uint8 [rows, K/32] rowwise UE8M0 scales (device, read).
 *   out        uint8 [ceil(rows/256)][ceil(K/256)][256][8] (device, written,
 *              8-byte aligned): byte j of entry (t, kt, r) is scale
 *              [256 t + r][8 kt + j], and 0 where that lies outside the input.
 *              Each 2 KiB block holds the scales of one 256-row tile for one
 *              256-value K-tile of fp4_mm, so a workgroup reads it with one
 *              coalesced 8-byte load per lane.
 * fp4q_mx_scales_tiled_bytes gives the size of out.  Needs K % 32 == 0
 * (FP4Q_ERR_SHAPE), K <= 2^22, rows <= 2^24 (FP4Q_ERR_UNSUPPORTED).
 */
size_t fp4q_mx_scales_tiled_bytes(int64_t rows, int64_t K);
int fp4_mx_scales_tiled(const uint8_t* scales, int64_t rows, int64_t K, uint8_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
