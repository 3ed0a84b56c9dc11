// kernels_tile.hip -- 64 x 64 tile kernel for gfx950: fused cast-transpose
// (rowwise and columnwise NVFP4 / AMD-FP4 buffers from one read of the
// source), the 2D outer-block mode, and its grouped (per-expert) form.
//
// "Block-Scaled FP8 and FP4 Weight Quantization", sections 2-4: a fused
// cast-transpose scans the high-precision source once and writes both the
// rowwise buffer and the columnwise buffer (the rowwise layout of W^T); with
// 1D scaling the columnwise direction is its own quantisation of the source
// (blocks run down the columns), not a transpose of the rowwise result.
// "NVFP4 / AMD-FP4 outer-block (two-level) scaling", Technical design and
// Implementation: a 2D outer scale is axis-invariant, computed once per tile
// and used by both directions; 1D outer groups follow the direction
// (1 x obs along rows, obs x 1 along columns); grouped MoE quantisation keeps
// one outer grid per expert.
//
// Per workgroup (256 lanes, 4 waves) one 2 x 2 super-tile of 64 x 64 source
// tiles at a time, the four tiles one after another:
//   row phase  lane (r = t/4, s = t%4) owns the 16-element row block
//              [r, 16s .. 16s+15]: two 16-byte loads, (residual add),
//              outer scale (2D: tile-wide max through a DPP wave max and LDS;
//              1D: max over the obs/16 lanes of the row group), normalise,
//              quantise, store 8 bytes of codes and one scale byte; (qdq
//              output, residual update).
//   LDS        the tile's values (normalised for 2D / tensorwise / none, raw
//              for 1D) and SR draws, so each element keeps one draw in both
//              directions.  16-byte chunks are XOR-swizzled by row so that the
//              row phase's 128-bit writes and the column phase's 32-bit reads
//              are both free of bank conflicts.
//   col phase  lane (c = t/4, q = t%4) owns the column block [16q .. 16q+15, c]:
//              (1D: column outer scale over obs/16 lanes), quantise, store
//              8 bytes of columnwise codes; the 4 lanes of a column write its
//              32 contiguous bytes.
// Two workgroup barriers per tile: one before the tile's LDS writes (the
// previous tile's column reads are done; for 2D it also publishes the wave
// maxima) and one after them.  Codes, scale bytes and 1D outer scales of the
// two tiles of a super-tile row (column) are stored together, as runs of 64
// code bytes and 8 scale bytes per row (column).
//
// With 16 x 16 inner tiles ("Block-Scaled FP8 and FP4 Weight Quantization",
// section 6) the row phase takes each inner scale from the largest normalised
// magnitude of the 16 lanes holding one 16 x 16 tile (the lanes of equal
// column segment in one wave), publishes the 16 scale codes of the 64 x 64
// tile in LDS, and the column phase encodes its column block with the scale
// of the tile it lies in: the same quotient and the same SR variate as the
// row phase, so the columnwise codes and scales are the transposes of the
// rowwise ones.
//
// Super-tiles are taken in row-major order, split into 8 contiguous slices,
// one per XCD (workgroup ids are dealt round-robin to the XCDs), so the
// partial cache lines that neighbouring super-tiles write meet in the same
// L2.  Workgroups are persistent within their slice and load each tile's
// inputs before computing the tile before it.
#include <mutex>
#include <vector>

#include "launch.h"
#include "nv_block.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

// Physical 16-byte chunk (4 floats) of logical chunk ch = col / 4 in tile row
// `row`.  A bijection on ch for every row.  It spreads a ds_write_b128 group
// of 8 lanes {rows r, r+1} x {segments 0..3} over 8 distinct 4-bank groups,
// and the 32 lanes of each half-wave of the column phase (8 columns x 4 row
// quarters, one row each) over 32 distinct banks.
__device__ __forceinline__ int swz_chunk(int row, int ch)
{
    return ch ^ (((row >> 4) & 3) << 1) ^ (row & 1) ^ (((ch >> 3) & 1) << 1);
}

// Physical 16-byte chunk (8 u16 variates) of chunk ch = col / 8 in row `row`
// of the SR-variate tile: XOR by twice the 16-row band.  The column phase's
// u16 reads (one column per lane pair, the four bands of a wave at once) then
// spread over 8 chunks = all 32 banks.
__device__ __forceinline__ int swz_u_chunk(int row, int ch)
{
    return ch ^ (2 * ((row >> 4) & 3));
}

// Largest value of m over the 16 lanes of a wave whose lane index is congruent
// to this lane's modulo 4 (m >= 0): the lanes of one 16 x 16 inner tile in the
// row phase.  Two rotations within each 16-lane row, then two exchanges across
// rows.
__device__ __forceinline__ float tile16_max(float m)
{
    uint32_t v = __float_as_uint(m);
    v = max_dpp<kDppRowRor4>(v);
    v = max_dpp<kDppRowRor8>(v);
    uint32_t o = (uint32_t)__shfl_xor((int)v, 16, 64);
    v = v > o ? v : o;
    o = (uint32_t)__shfl_xor((int)v, 32, 64);
    v = v > o ? v : o;
    return __uint_as_float(v);
}

// Codes of 16 normalised values with a given inner scale (CLAMP: no outer
// scale bounds the quotients, see codes16_sr).
template <int BIAS, bool SR, bool CLAMP, int NU>
__device__ __forceinline__ uint2 encode16(const float (&vn)[16], const uint32_t (&u)[NU], const float2* ktab,
                                          const BlockScale<BIAS>& sc)
{
    if (SR) return codes16_sr<CLAMP>(vn, u, ktab[sc.code]);
    return codes16_rne(vn, ktab[sc.code]);
}

// One block's scale and codes; with I2D the scale comes from the 16 x 16 tile
// (tile16_max) instead of the lane's own 16 values.  u: SR variates, two per
// word (NU = 8) or one per word (NU = 16).
template <int BIAS, bool SR, bool I2D, bool CLAMP, int NU>
__device__ __forceinline__ uint2 quant16(const float (&vn)[16], const uint32_t (&u)[NU], const double* tab,
                                         const float2* ktab, BlockScale<BIAS>& sc)
{
    const float b = max_abs16(vn);
    sc = block_scale<BIAS>(I2D ? tile16_max(b) : b, tab);
    return encode16<BIAS, SR, CLAMP>(vn, u, ktab, sc);
}

// Super-tiles: the unit a workgroup walks is a 2 x 2 block of 64 x 64 tiles
// (128 x 128 elements), so that the outputs of horizontally (vertically)
// neighbouring tiles can be stored together: 64-byte code runs and 8-byte
// scale runs per row (column) instead of 32 and 4.
constexpr int kSuper = 2 * kTile;

// Walks a workgroup's super-tiles t = first, first + W, ... in the row-major
// order of (group, super-tile row, super-tile column) without dividing per
// step: the column advances by W % st_c and the row by W / st_c.  The current
// group's row range is kept in registers; crossing into another group (rare)
// re-derives the position from the prefix tables.  GROUPED is false for a
// launch of one group that starts at row 0 (every call on a single tensor):
// the walk never crosses a group, the group's rows are 0 .. row0[1] - 1 and
// its tiles start at 0, and the scalar registers that the group bookkeeping
// would hold stay free (the tile loop otherwise spills scalars into vector
// lanes: the 16384 x 2880 1D SR cast-transpose took 82.7 us with the
// bookkeeping and 80.1 us without, the 4096^2 2D one 18.8 and 18.2).
struct TileWalk {
    int t, g, si, sj, di, dj;
    int r0, Rg, tile_end;   // group's first row, row count, end of its super-tiles
};

template <bool GROUPED>
__device__ __forceinline__ void walk_locate(const TileArgs& a, TileWalk& w)
{
    if (GROUPED)
        while (w.g + 1 < a.ngroups && a.tile0[w.g + 1] <= w.t) ++w.g;
    const int lt = GROUPED ? w.t - a.tile0[w.g] : w.t;
    w.si = lt / a.tiles_c;
    w.sj = lt - w.si * a.tiles_c;
    w.r0 = GROUPED ? a.row0[w.g] : 0;
    w.Rg = GROUPED ? a.row0[w.g + 1] - w.r0 : a.row0[1];
    w.tile_end = GROUPED ? a.tile0[w.g + 1] : a.total_tiles;
}

template <bool GROUPED>
__device__ __forceinline__ void walk_next(const TileArgs& a, TileWalk& w, int step)
{
    w.t += step;
    if (GROUPED && w.t >= w.tile_end) {
        walk_locate<GROUPED>(a, w);
        return;
    }
    w.si += w.di;
    w.sj += w.dj;
    if (w.sj >= a.tiles_c) {
        w.sj -= a.tiles_c;
        ++w.si;
    }
}

// One 64 x 64 tile's place, uniform across the workgroup: group g (first row
// r0, Rg rows), tile row ti within the group, tile column tj, the valid extent
// (0 for a tile of a super-tile that lies outside the tensor), and the element
// indices of its (0, 0) element in the row-major source and in the columnwise
// buffers.
struct Tile {
    int g, r0, ti, tj, rows_valid, cols_valid, Rg, grow0, c0, lrow0;
    int64_t e_base;    // (grow0) * cols + c0
    int64_t ce_base;   // r0 * cols + c0 * Rg + lrow0
};

__device__ __forceinline__ Tile make_tile(const TileArgs& a, const TileWalk& w, int sub)
{
    Tile t;
    t.g = w.g;
    t.r0 = w.r0;
    t.ti = 2 * w.si + (sub >> 1);
    t.tj = 2 * w.sj + (sub & 1);
    t.Rg = w.Rg;
    t.lrow0 = t.ti * kTile;
    t.grow0 = w.r0 + t.lrow0;
    t.c0 = t.tj * kTile;
    t.rows_valid = max(0, min(kTile, t.Rg - t.lrow0));
    t.cols_valid = max(0, min(kTile, (int)a.cols - t.c0));
    t.e_base = (int64_t)t.grow0 * a.cols + t.c0;
    t.ce_base = (int64_t)w.r0 * a.cols + (int64_t)t.c0 * t.Rg + t.lrow0;
    return t;
}

// The tile of a walk whose unit is one tile (staged output).
__device__ __forceinline__ Tile make_tile_unit(const TileArgs& a, const TileWalk& w)
{
    Tile t;
    t.g = w.g;
    t.r0 = w.r0;
    t.ti = w.si;
    t.tj = w.sj;
    t.Rg = w.Rg;
    t.lrow0 = t.ti * kTile;
    t.grow0 = w.r0 + t.lrow0;
    t.c0 = t.tj * kTile;
    t.rows_valid = max(0, min(kTile, t.Rg - t.lrow0));
    t.cols_valid = max(0, min(kTile, (int)a.cols - t.c0));
    t.e_base = (int64_t)t.grow0 * a.cols + t.c0;
    t.ce_base = (int64_t)w.r0 * a.cols + (int64_t)t.c0 * t.Rg + t.lrow0;
    return t;
}

// The lane's raw inputs for one tile: 16 bf16 (two 16-byte loads) and, with
// error feedback, the 16 FP32 residuals.  Lanes outside the tensor (and every
// lane when `valid` is false) read zeros.
template <bool EF>
struct TileInput {
    uint4 w0, w1;
    uint4 z[EF ? 4 : 1];
};

template <bool EF>
__device__ __forceinline__ void load_tile_input(const TileArgs& a, const Tile& t, bool valid, int r, int sg,
                                                TileInput<EF>& in)
{
    const bool act = valid && r < t.rows_valid && 16 * sg < t.cols_valid;
    const rsrc_t rx = make_rsrc(a.x + (int64_t)t.grow0 * a.ld + t.c0);
    const uint32_t ox = act ? (uint32_t)(r * (int)a.ld + 16 * sg) * 2u : kOff;
    in.w0 = buf_load16(rx, ox);
    in.w1 = buf_load16(rx, ox + 16u);
    if (EF) {
        const rsrc_t rz = make_rsrc(a.residual + t.e_base);
        const uint32_t oz = act ? (uint32_t)(r * (int)a.cols + 16 * sg) * 4u : kOff;
#pragma unroll
        for (int q = 0; q < 4; ++q) in.z[q] = buf_load16<0>(rz, oz + 16u * q);
    }
}

// One direction's per-lane result for one tile: 16 packed codes, the scale
// byte and (1D) the lane's outer scale.
struct DirOut {
    uint2 codes;
    uint32_t scale;
    float outer;
};

// Per-wave staging used to pair two tiles' outputs: each lane deposits its 8
// code bytes and its scale byte, then reads back 16 contiguous code bytes
// (and lanes 0-1 four scale bytes) of the 64-byte / 8-byte run of its row
// (column).  Four lanes of a row share a wave, so no barrier is needed.
struct alignas(16) PairStage {
    uint2 codes[kThreads / 4][8];
    uint8_t scales[kThreads / 4][8];
};

// Orders this wave's LDS accesses before and after it (the lanes of a line
// exchange data through LDS within one wave).
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
}

// Stores one row (or column) run made of tile A's and tile B's results for
// the four lanes (k = lane & 3) of line `line`.  nvalid = valid 16-element
// blocks in the run (A's first, then B's; B is present only when A is full).
// Every lane issues the same five store instructions; the hardware drops the
// masked ones.
__device__ __forceinline__ void store_pair(PairStage& st, int line, int k, const DirOut& A, const DirOut& B,
                                           bool line_ok, int nvalid, rsrc_t rc, uint32_t oc, rsrc_t rsc,
                                           uint32_t osc)
{
    wave_lds_fence();   // earlier reads of this line's staging are done
    st.codes[line][k] = A.codes;
    st.codes[line][4 + k] = B.codes;
    st.scales[line][k] = (uint8_t)A.scale;
    st.scales[line][4 + k] = (uint8_t)B.scale;
    wave_lds_fence();   // the other lanes' deposits are visible
    const uint4 c16 = *reinterpret_cast<const uint4*>(&st.codes[line][2 * k]);
    const uint32_t s4 = *reinterpret_cast<const uint32_t*>(&st.scales[line][4 * (k & 1)]);
    // 16-byte code chunk k holds blocks 2k and 2k+1
    const bool full = line_ok && 2 * k + 1 < nvalid;
    const bool half = line_ok && 2 * k + 1 == nvalid;
    buf_store16(rc, full ? oc + 16u * k : kOff, c16);
    buf_store8(rc, half ? oc + 16u * k : kOff, make_uint2(c16.x, c16.y));
    // scale dword k (k < 2) holds blocks 4k .. 4k+3
    buf_store_u32(rsc, (line_ok && k < 2 && 4 * k + 3 < nvalid) ? osc + 4u * k : kOff, s4);
    // the remaining blocks of a partial run, one byte each
    const int full_words = nvalid >> 2;
    buf_store_u8(rsc, (line_ok && full_words == 0 && k < nvalid) ? osc + k : kOff, A.scale);
    buf_store_u8(rsc, (line_ok && full_words == 1 && 4 + k < nvalid) ? osc + 4u + k : kOff, B.scale);
}

// The straight-line (RTNE, no residual, not 1D) form of a super-tile.
template <int OUTER, bool SR, bool EF>
constexpr bool tile_unrolled()
{
    return !SR && !EF && OUTER != kOuter1D;
}

// Register budget per lane: 128 VGPRs (4 waves per SIMD) wherever the kernel
// fits in them without scratch spills, 168 (3 waves) for the stochastic-
// rounding variants that do not (2D / tensorwise / no outer scale without a
// residual, tensorwise with one, and 16 x 16 inner tiles with a residual and a
// 2D outer scale): a spill reload inside the tile loop waits for every load in
// flight, the next tile's prefetch included.
template <int BIAS, int OUTER, bool SR, bool COLS, bool EF, bool I2D>
constexpr int tile_waves_per_simd()
{
    const bool tight = SR && ((!EF && OUTER != kOuter1D) || (EF && OUTER == kOuterTensor) ||
                              (EF && I2D && COLS && OUTER == kOuter2D));
    return tight ? 3 : 4;
}

// Largest staged tail: scale bytes (2 x 256) and 1D outer scales of 16-element
// groups (2 x 1024).
constexpr int kTailMax = kStageRowOuter - kStageTail + 2 * 64 * 4 * 4;

// Every global access is a buffer instruction whose masked lanes carry an
// out-of-range offset, and every tile iteration issues the same sequence of
// memory instructions with no branch around any of them, so the compiler's
// wait for the next tile's loads never waits for earlier stores.
template <int BIAS, int OUTER, bool SR, bool COLS, bool EF, bool GIVEN, bool Y, bool I2D, bool STAGED, bool GROUPED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(tile_waves_per_simd<BIAS, OUTER, SR, COLS, EF, I2D>())))
void k_tile(TileArgs a)
{
    __shared__ float4 lds_v[COLS ? kTile * kTile / 4 : 1];
    __shared__ uint4 lds_u[(COLS && SR) ? kTile * kTile / 8 : 1];   // SR variates, [row][col] u16, swizzled
    __shared__ uint32_t lds_tsc[(COLS && I2D) ? 16 : 1];   // 16 x 16 inner scale codes, [tile row][tile col]
    __shared__ uint32_t red[2][kThreads / 64];
    __shared__ double rtab[kRecipTableSize];
    __shared__ float2 ktab[kRneTableSize];
    // paired-tile stores (direct path only)
    __shared__ uint4 pair_raw[STAGED ? 1 : (sizeof(PairStage) + 15) / 16];
    PairStage* const stage = reinterpret_cast<PairStage*>(pair_raw);
    // staged output: the tail of each tile's block (scale bytes and 1D outer
    // scales) gathered here, one buffer per tile parity, and written by the
    // workgroup as whole lines once every wave has finished the tile
    constexpr int kTailCap = OUTER == kOuter1D ? kTailMax : kStageRowOuter - kStageTail;
    __shared__ uint4 tail[STAGED ? 2 * kTailCap / 16 : 1];
    // error feedback with both directions: the new residual of the tile, so
    // that it is stored row-coalesced (16 lanes write one row's 256 bytes)
    // instead of as each lane's 64-byte run (measured on the grouped
    // 32 x 2880^2 step's traffic: 0.68 -> 0.58 ms)
    __shared__ float4 lds_res[(COLS && EF) ? kTile * kTile / 4 : 1];

    const int tid = (int)threadIdx.x;
    const int r = tid >> 2, sg = tid & 3;       // row phase: row, 16-column segment
    const int cc = tid >> 2, rs = tid & 3;      // column phase: column, 16-row segment
    // Direct stores: each XCD walks its own contiguous slice of the tiles,
    // so the partial lines that neighbouring tiles write meet in that XCD's
    // L2.  Staged output writes whole lines and reuses nothing across
    // workgroups: there the whole grid walks the tiles in turn, which keeps
    // every workgroup's residual and source rows in one narrow band of memory
    // (grouped 32 x 2880^2 step: 691 -> 681 us; with direct stores the same
    // order took the 16384 x 2880 1D SR cast-transpose from 80 to 87 us).
    const int xcd = (int)(blockIdx.x & 7u), slot = (int)(blockIdx.x >> 3);
    const int slice0 = STAGED ? 0 : xcd * a.per_xcd;
    const int slice_end = STAGED ? a.total_tiles : min(slice0 + a.per_xcd, a.total_tiles);
    const int W = STAGED ? (int)gridDim.x : a.wgs_per_xcd;
    TileWalk walk;
    walk.t = STAGED ? (int)blockIdx.x : slice0 + slot;
    if (walk.t >= slice_end) return;   // uniform per workgroup
    walk.g = 0;
    walk.di = W / a.tiles_c;
    walk.dj = W - walk.di * a.tiles_c;
    walk_locate<GROUPED>(a, walk);
    TileInput<EF> in;
    load_tile_input<EF>(a, STAGED ? make_tile_unit(a, walk) : make_tile(a, walk, 0), true, r, sg, in);
    fill_recip_table(rtab, tid);
    fill_rne_table<BIAS>(ktab, tid);
    lds_barrier();
    const float den = ScaleFmt<BIAS>::outer_den();
    const int cols = (int)a.cols;
    const int obs = 16 * a.obs16;
    // lane offsets that do not depend on the tile
    const uint32_t erow = (uint32_t)(r * cols + 16 * sg);   // row phase: first element, tile-relative
    const int lds_row = r * 16;
    const int lds_col = 4 * swz_chunk(16 * rs, cc >> 2) + (cc & 3);   // + row * kTile, swizzle parity below

    // tensorwise: one scale for the whole launch
    float s_tensor = 1.0f;
    double inv_tensor = 1.0;
    if (OUTER == kOuterTensor) {
        s_tensor = *a.tensor_scale;
        inv_tensor = outer_inv(s_tensor);
    }

    // Let the first tile's loads land here, so that at the loop head the
    // current tile's registers are complete on every path.
    wait_vmem_all();

    int iter = 0;   // tiles processed (parity of the reduction slots)

    // staged output: the block of the previous tile, whose tail is written
    // once every wave is past the current tile's first barrier
    const uint8_t* prev_blk = nullptr;
    bool prev_ok = false;
    uint8_t* const tail8 = reinterpret_cast<uint8_t*>(tail);
    float* const tailf = reinterpret_cast<float*>(tail);
    const int opr = 4 / a.obs16;                                   // 1D outer groups per tile row
    const int tail_bytes = (kStageRowOuter - kStageTail) + (OUTER == kOuter1D ? 2 * 64 * opr * 4 : 0);
    auto emit_tail = [&](int par) {
        const int n16 = tail_bytes / 16;
        const uint4 v = tail[par * (kTailCap / 16) + min(tid, n16 - 1)];
        buf_store16(make_rsrc(prev_blk), (prev_ok && tid < n16) ? (uint32_t)(16 * tid) : kOff, v);
    };

    // One tile: row phase, LDS transpose, column phase.  Writes the dequantised
    // output, the residual and 2D outer scales itself; returns the codes, scale
    // bytes and 1D outer scales of both directions for the paired stores.
    auto tile_body = [&](const Tile& cur, const TileInput<EF>& tin, DirOut& ro, DirOut& co) {
        const bool act = r < cur.rows_valid && 16 * sg < cur.cols_valid;
        // ---------------- row phase
        float v[16];
        uint32_t am_bits = 0;    // bit pattern of max |v| over the lane's 16 values
        {
            const uint32_t w[8] = {tin.w0.x, tin.w0.y, tin.w0.z, tin.w0.w, tin.w1.x, tin.w1.y, tin.w1.z, tin.w1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) { v[2 * k] = bf16_lo(w[k]); v[2 * k + 1] = bf16_hi(w[k]); }
            if (EF) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[4 * q] = v[4 * q] + __uint_as_float(tin.z[q].x);
                    v[4 * q + 1] = v[4 * q + 1] + __uint_as_float(tin.z[q].y);
                    v[4 * q + 2] = v[4 * q + 2] + __uint_as_float(tin.z[q].z);
                    v[4 * q + 3] = v[4 * q + 3] + __uint_as_float(tin.z[q].w);
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t b = __float_as_uint(v[k]) & 0x7FFFFFFFu;
                    am_bits = am_bits > b ? am_bits : b;
                }
            } else {
                am_bits = bf16_absmax_bits(w) << 16;
            }
            // NaN / inf anywhere in the lane's 16 values (rare): sanitise them
            if (__builtin_expect(am_bits >= 0x7F800000u, 0)) {
                am_bits = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    v[k] = sanitize(v[k]);
                    const uint32_t b = __float_as_uint(v[k]) & 0x7FFFFFFFu;
                    am_bits = am_bits > b ? am_bits : b;
                }
            }
        }
        uint32_t u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) u[k] = 0;
        if (SR && act) sr_draws16(a.seed, a.step, a.index_base + (uint64_t)cur.e_base, erow, u);   // erow % 16 == 0

        bool barrier_done = false;   // the pre-LDS-write barrier has been passed
        float s_row = 1.0f;
        double inv_row = 1.0;
        ro.outer = 0.0f;
        co.outer = 0.0f;
        if (OUTER == kOuterTensor) {
            s_row = s_tensor;
            inv_row = inv_tensor;
        } else if (OUTER == kOuter2D) {
            const int64_t oidx = (int64_t)(cur.grow0 / kTile) * (cols / kTile) + cur.tj;
            const rsrc_t ro2 = make_rsrc(a.row_outer ? a.row_outer + oidx : nullptr);
            const bool tile_ok = cur.rows_valid > 0 && cur.cols_valid > 0;
            if (GIVEN) {
                s_row = buf_load_f32(ro2, tile_ok ? 0u : kOff);
            } else {
                const uint32_t m = wave_max_u32(am_bits);
                uint32_t* rb = red[iter & 1];
                if ((tid & 63) == 0) rb[__builtin_amdgcn_readfirstlane(tid >> 6)] = m;   // wave index, uniform
                lds_barrier();
                barrier_done = true;
                const uint32_t mm = max(max(rb[0], rb[1]), max(rb[2], rb[3]));
                s_row = outer_scale(__uint_as_float(mm), den);
                buf_store_u32(ro2, (tid == 0 && tile_ok) ? 0u : kOff, __float_as_uint(s_row));
            }
            inv_row = outer_inv(s_row);
        } else if (OUTER == kOuter1D) {
            // rowwise 1D groups: [rows, cols / obs]
            const int gpr = cols / obs;
            const rsrc_t ro1 =
                make_rsrc(a.row_outer ? a.row_outer + (int64_t)cur.grow0 * gpr + cur.c0 / obs : nullptr);
            const uint32_t oo = (uint32_t)(r * gpr + (16 * sg) / obs) * 4u;
            if (GIVEN) {
                s_row = buf_load_f32(ro1, act ? oo : kOff);
                if (!act) s_row = 1.0f;
            } else {
                s_row = outer_scale(__uint_as_float(quad_max_u32(am_bits, a.obs16)), den);
                ro.outer = s_row;
            }
            inv_row = outer_inv(s_row);
        }

        float vn[16];
        float res[EF ? 16 : 1];   // the new residual (error feedback)
        if (OUTER == kOuterNone) {
#pragma unroll
            for (int k = 0; k < 16; ++k) vn[k] = v[k];
        } else {
            normalize16<SR, !EF>(v, s_row, inv_row, vn);
        }
        {
            BlockScale<BIAS> sc;
            const uint2 packed = quant16<BIAS, SR, I2D, OUTER == kOuterNone>(vn, u, rtab, ktab, sc);
            ro.codes = packed;
            ro.scale = sc.code;
            if (STAGED) {
                const int par = iter & 1;
                tail8[par * kTailCap + r * 4 + sg] = (uint8_t)sc.code;
                if (OUTER == kOuter1D && !GIVEN && (sg % a.obs16) == 0)
                    tailf[par * (kTailCap / 4) + 128 + r * opr + sg / a.obs16] = ro.outer;
            }
            if (EF || Y) {
                float w[16];
                decode16(packed, sc.d, w);
                if (OUTER != kOuterNone) {
#pragma unroll
                    for (int k = 0; k < 16; ++k) w[k] = w[k] * s_row;
                }
                if (Y) {
                    uint32_t o[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) o[k] = f32_to_bf16(w[2 * k]) | (f32_to_bf16(w[2 * k + 1]) << 16);
                    const rsrc_t ry = make_rsrc(a.y + cur.e_base);
                    const uint32_t oy = act ? erow * 2u : kOff;
                    buf_store16<kNT>(ry, oy, make_uint4(o[0], o[1], o[2], o[3]));
                    buf_store16<kNT>(ry, oy + 16u, make_uint4(o[4], o[5], o[6], o[7]));
                }
                if (EF) {
#pragma unroll
                    for (int k = 0; k < 16; ++k) res[k] = v[k] - w[k];
                    if (!COLS) {
                        const rsrc_t rz = make_rsrc(a.residual + cur.e_base);
                        const uint32_t oz = act ? erow * 4u : kOff;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            buf_store16(rz, oz + 16u * q,
                                        make_uint4(__float_as_uint(res[4 * q]), __float_as_uint(res[4 * q + 1]),
                                                   __float_as_uint(res[4 * q + 2]), __float_as_uint(res[4 * q + 3])));
                    }
                }
            }
        }
        if (COLS) {
            // ---------------- stage through LDS
            if (!barrier_done) lds_barrier();   // previous tile's column reads are done
            if (STAGED) emit_tail((iter & 1) ^ 1);
            const float* src = (OUTER == kOuter1D) ? v : vn;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_v[lds_row + swz_chunk(r, 4 * sg + j)] =
                    make_float4(src[4 * j], src[4 * j + 1], src[4 * j + 2], src[4 * j + 3]);
            if (SR) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    lds_u[r * 8 + swz_u_chunk(r, 2 * sg + j)] =
                        make_uint4(u[4 * j], u[4 * j + 1], u[4 * j + 2], u[4 * j + 3]);
            }
            if (I2D && (r & 15) == 0) lds_tsc[(r >> 4) * 4 + sg] = ro.scale;
            if (EF) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    lds_res[lds_row + swz_chunk(r, 4 * sg + j)] =
                        make_float4(res[4 * j], res[4 * j + 1], res[4 * j + 2], res[4 * j + 3]);
            }
            lds_barrier();
            if (EF) {
                // row-coalesced residual store: pass q, lane t takes row 16 q + t / 16, columns 4 (t % 16) .. + 3
                const rsrc_t rz = make_rsrc(a.residual + cur.e_base);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 16 * q + (tid >> 4), ch = tid & 15;
                    const float4 f = lds_res[row * 16 + swz_chunk(row, ch)];
                    const bool ok = row < cur.rows_valid && 4 * ch < cur.cols_valid;
                    buf_store16(rz, ok ? (uint32_t)(row * cols + 4 * ch) * 4u : kOff,
                                make_uint4(__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z),
                                           __float_as_uint(f.w)));
                }
            }

            // ---------------- column phase
            const float* lf = reinterpret_cast<const float*>(lds_v);
            float cv[16];
            uint32_t cu[16];   // one variate per word
            const uint16_t* lu = reinterpret_cast<const uint16_t*>(lds_u);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int row = 16 * rs + k;
                // rows of one parity share the swizzled column
                cv[k] = lf[row * kTile + (lds_col ^ (4 * (k & 1)))];
            }
            // column cc of rows 16 rs .. 16 rs + 15, all in 16-row band rs
            const int lu_col = 8 * swz_u_chunk(16 * rs, cc >> 3) + (cc & 7);
#pragma unroll
            for (int k = 0; k < 16; ++k) cu[k] = SR ? (uint32_t)lu[(16 * rs + k) * kTile + lu_col] : 0u;
            if (OUTER == kOuter1D) {
                const bool actc = (cc < cur.cols_valid) && (16 * rs < cur.rows_valid);
                float s_col;
                if (GIVEN) {
                    // columnwise 1D groups: [cols, Rg / obs] per group
                    const int gpc = cur.Rg / obs;
                    const rsrc_t rco =
                        make_rsrc(a.col_outer ? a.col_outer + (int64_t)cur.r0 * cols / obs +
                                                    (int64_t)cur.c0 * gpc + cur.lrow0 / obs
                                              : nullptr);
                    const uint32_t oo = (uint32_t)(cc * gpc + (16 * rs) / obs) * 4u;
                    s_col = buf_load_f32(rco, actc ? oo : kOff);
                    if (!actc) s_col = 1.0f;
                } else {
                    s_col = outer_scale(quad_max(max_abs16(cv), a.obs16), den);
                    co.outer = s_col;
                }
                float cn[16];
                normalize16<SR, !EF>(cv, s_col, outer_inv(s_col), cn);
#pragma unroll
                for (int k = 0; k < 16; ++k) cv[k] = cn[k];
            }
            if (I2D) {
                // the scale of the 16 x 16 tile holding this column block
                BlockScale<BIAS> sc;
                sc.code = lds_tsc[rs * 4 + (cc >> 4)];
                sc.d = 0.0f;   // not needed for encoding
                sc.rd = inner_recip<BIAS>(sc.code, rtab);
                co.codes = encode16<BIAS, SR, OUTER == kOuterNone>(cv, cu, ktab, sc);
                co.scale = sc.code;
            } else {
                BlockScale<BIAS> sc;
                co.codes = quant16<BIAS, SR, false, OUTER == kOuterNone>(cv, cu, rtab, ktab, sc);
                co.scale = sc.code;
            }
            if (STAGED) {
                const int par = iter & 1;
                tail8[par * kTailCap + 256 + cc * 4 + rs] = (uint8_t)co.scale;
                if (OUTER == kOuter1D && !GIVEN && (rs % a.obs16) == 0)
                    tailf[par * (kTailCap / 4) + 128 + 64 * opr + cc * opr + rs / a.obs16] = co.outer;
            }
        }
        ++iter;
    };

    // 1D outer scales of a tile pair: with 64-element groups one lane per line
    // holds both tiles' values (stored as one 8-byte run); smaller groups are
    // stored lane by lane.
    auto store_outer_pair = [&](rsrc_t rb, uint32_t off_a, uint32_t off_b, bool lead, bool ok_a, bool ok_b,
                                const DirOut& A, const DirOut& B) {
        const bool wide = a.obs16 == 4;
        buf_store8(rb, (wide && lead && ok_a && ok_b) ? off_a : kOff,
                   make_uint2(__float_as_uint(A.outer), __float_as_uint(B.outer)));
        buf_store_u32(rb, ((wide && ok_a && !ok_b) || (!wide && ok_a)) && lead ? off_a : kOff,
                      __float_as_uint(A.outer));
        buf_store_u32(rb, (!wide && lead && ok_b) ? off_b : kOff, __float_as_uint(B.outer));
    };

    // Row runs of tiles (sub, sub + 1) of the current super-tile.
    auto emit_rows = [&](const Tile& ta, const Tile& tb, const DirOut& A, const DirOut& B, bool enable) {
        const int nvalid = ta.cols_valid / 16 + tb.cols_valid / 16;
        const bool line_ok = enable && r < ta.rows_valid;
        const rsrc_t rc = make_rsrc(a.row_codes ? a.row_codes + ta.e_base / 2 : nullptr);
        const rsrc_t rsc = make_rsrc(a.row_scales ? a.row_scales + ta.e_base / 16 : nullptr);
        store_pair(*stage, r, sg, A, B, line_ok, nvalid, rc, (uint32_t)(r * cols) / 2u, rsc,
                   (uint32_t)(r * cols) / 16u);
        if (OUTER == kOuter1D && !GIVEN) {
            const int gpr = cols / obs;
            const rsrc_t rb =
                make_rsrc(a.row_outer ? a.row_outer + (int64_t)ta.grow0 * gpr + ta.c0 / obs : nullptr);
            const uint32_t off_a = (uint32_t)(r * gpr + (16 * sg) / obs) * 4u;
            store_outer_pair(rb, off_a, off_a + (uint32_t)(kTile / obs) * 4u, (sg % a.obs16) == 0,
                             line_ok && 16 * sg < ta.cols_valid, line_ok && 16 * sg < tb.cols_valid, A, B);
        }
    };

    // Column runs of tiles (sub, sub + 2) of the current super-tile.
    auto emit_cols = [&](const Tile& ta, const Tile& tb, const DirOut& A, const DirOut& B, bool enable) {
        const int nvalid = ta.rows_valid / 16 + tb.rows_valid / 16;
        const bool line_ok = enable && cc < ta.cols_valid;
        const uint32_t ecol = (uint32_t)(cc * ta.Rg);   // lane's column, relative to the run start
        store_pair(*stage, cc, rs, A, B, line_ok, nvalid, make_rsrc(a.col_codes + ta.ce_base / 2), ecol / 2u,
                   make_rsrc(a.col_scales + ta.ce_base / 16), ecol / 16u);
        if (OUTER == kOuter1D && !GIVEN) {
            const int gpc = ta.Rg / obs;
            const rsrc_t rb = make_rsrc(a.col_outer ? a.col_outer + (int64_t)ta.r0 * cols / obs +
                                                          (int64_t)ta.c0 * gpc + ta.lrow0 / obs
                                                    : nullptr);
            const uint32_t off_a = (uint32_t)(cc * gpc + (16 * rs) / obs) * 4u;
            store_outer_pair(rb, off_a, off_a + (uint32_t)(kTile / obs) * 4u, (rs % a.obs16) == 0,
                             line_ok && 16 * rs < ta.rows_valid, line_ok && 16 * rs < tb.rows_valid, A, B);
        }
    };

    // A tile stored on its own: 8 code bytes and a scale byte per lane in
    // each direction, and the lane's 1D outer scale.
    auto emit_single = [&](const Tile& t, const DirOut& ro, const DirOut& co) {
        const bool act = r < t.rows_valid && 16 * sg < t.cols_valid;
        const uint32_t erow_t = (uint32_t)(r * cols + 16 * sg);
        buf_store8(make_rsrc(a.row_codes ? a.row_codes + t.e_base / 2 : nullptr), act ? erow_t / 2u : kOff, ro.codes);
        buf_store_u8(make_rsrc(a.row_scales ? a.row_scales + t.e_base / 16 : nullptr), act ? erow_t / 16u : kOff,
                     ro.scale);
        if (OUTER == kOuter1D && !GIVEN) {
            const int gpr = cols / obs;
            const rsrc_t rb =
                make_rsrc(a.row_outer ? a.row_outer + (int64_t)t.grow0 * gpr + t.c0 / obs : nullptr);
            const uint32_t oo = (uint32_t)(r * gpr + (16 * sg) / obs) * 4u;
            buf_store_u32(rb, (act && (sg % a.obs16) == 0) ? oo : kOff, __float_as_uint(ro.outer));
        }
        if (COLS) {
            const bool actc = (cc < t.cols_valid) && (16 * rs < t.rows_valid);
            const uint32_t ecol = (uint32_t)(cc * t.Rg + 16 * rs);
            buf_store8(make_rsrc(a.col_codes + t.ce_base / 2), actc ? ecol / 2u : kOff, co.codes);
            buf_store_u8(make_rsrc(a.col_scales + t.ce_base / 16), actc ? ecol / 16u : kOff, co.scale);
            if (OUTER == kOuter1D && !GIVEN) {
                const int gpc = t.Rg / obs;
                const rsrc_t rb = make_rsrc(a.col_outer ? a.col_outer + (int64_t)t.r0 * cols / obs +
                                                              (int64_t)t.c0 * gpc + t.lrow0 / obs
                                                        : nullptr);
                const uint32_t oo = (uint32_t)(cc * gpc + (16 * rs) / obs) * 4u;
                buf_store_u32(rb, (actc && (rs % a.obs16) == 0) ? oo : kOff, __float_as_uint(co.outer));
            }
        }
    };

    TileWalk st = walk;
    if constexpr (STAGED) {
        // One tile per iteration in row-major tile order; codes go to the
        // tile's block as whole lines (a wave's 64 lanes write 512 contiguous
        // bytes), the tail through LDS (emit_tail).
        for (;;) {
            const Tile cur = make_tile_unit(a, st);
            const bool has_next = st.t + W < slice_end;
            TileWalk nst = st;
            if (has_next) walk_next<GROUPED>(a, nst, W);
            TileInput<EF> nin;
            load_tile_input<EF>(a, make_tile_unit(a, nst), has_next, r, sg, nin);
            DirOut ro, co;
            tile_body(cur, in, ro, co);
            const bool ok = cur.rows_valid > 0 && cur.cols_valid > 0;
            // staging regions (launch.h): row codes by tile index, column
            // codes by the tile's column-major index in its group, tails
            const int64_t ntiles = a.total_tiles;
            const int tr = (cur.Rg + 63) >> 6;                   // tile rows of the group
            const int64_t cidx = (int64_t)a.tile0[GROUPED ? cur.g : 0] + (int64_t)cur.tj * tr + cur.ti;
            buf_store8(make_rsrc(a.stage + (int64_t)st.t * kStageCodes), ok ? (uint32_t)(r * 32 + sg * 8) : kOff,
                       ro.codes);
            buf_store8(make_rsrc(a.stage + (ntiles + cidx) * kStageCodes), ok ? (uint32_t)(cc * 32 + rs * 8) : kOff,
                       co.codes);
            prev_blk = a.stage + 2 * ntiles * kStageCodes + (int64_t)st.t * (a.stage_block - kStageTail);
            prev_ok = ok;
            if (!has_next) break;
            st = nst;
            in = nin;
        }
        lds_barrier();
        emit_tail((iter & 1) ^ 1);
    } else if constexpr (tile_unrolled<OUTER, SR, EF>()) {
        // RTNE: the four tiles of a super-tile as straight-line code; the row
        // runs of tiles (0, 1) and (2, 3) are stored after tiles 1 and 3, the
        // column runs of tiles (0, 2) and (1, 3) after tiles 2 and 3.
        for (;;) {
            const bool has_next = st.t + W < slice_end;
            TileWalk nst = st;
            if (has_next) walk_next<GROUPED>(a, nst, W);
            DirOut r0o, c0o, r1o, c1o, r2o, c2o, r3o, c3o;
            TileInput<EF> nin;

            load_tile_input<EF>(a, make_tile(a, st, 1), true, r, sg, nin);
            tile_body(make_tile(a, st, 0), in, r0o, c0o);
            in = nin;
            __builtin_amdgcn_sched_barrier(0);
            load_tile_input<EF>(a, make_tile(a, st, 2), true, r, sg, nin);
            tile_body(make_tile(a, st, 1), in, r1o, c1o);
            emit_rows(make_tile(a, st, 0), make_tile(a, st, 1), r0o, r1o, true);
            in = nin;
            __builtin_amdgcn_sched_barrier(0);
            load_tile_input<EF>(a, make_tile(a, st, 3), true, r, sg, nin);
            tile_body(make_tile(a, st, 2), in, r2o, c2o);
            if (COLS) emit_cols(make_tile(a, st, 0), make_tile(a, st, 2), c0o, c2o, true);
            in = nin;
            __builtin_amdgcn_sched_barrier(0);
            load_tile_input<EF>(a, make_tile(a, nst, 0), has_next, r, sg, nin);
            tile_body(make_tile(a, st, 3), in, r3o, c3o);
            emit_rows(make_tile(a, st, 2), make_tile(a, st, 3), r2o, r3o, true);
            if (COLS) emit_cols(make_tile(a, st, 1), make_tile(a, st, 3), c1o, c3o, true);
            if (!has_next) break;
            st = nst;
            in = nin;
        }
    } else {
        // Stochastic rounding, a residual or 1D outer groups need about twice
        // the registers, so the tiles run as a loop, one per iteration; every
        // iteration issues the same memory instructions (on iterations without
        // a finished pair the pair stores are issued fully masked).  With 1D
        // outer groups each tile is stored on its own (no results are held
        // across iterations).
        constexpr bool kPair = OUTER != kOuter1D;
        int sub = 0;
        DirOut row_a = {}, col_a0 = {}, col_a1 = {};   // results waiting for their partner tile
        for (;;) {
            const Tile cur = make_tile(a, st, sub);
            const bool last_sub = sub == 3;
            const bool has_next = !last_sub || st.t + W < slice_end;
            TileWalk nst = st;
            if (last_sub && has_next) walk_next<GROUPED>(a, nst, W);
            const int nsub = (sub + 1) & 3;
            TileInput<EF> nin;
            load_tile_input<EF>(a, make_tile(a, nst, nsub), has_next, r, sg, nin);

            DirOut ro, co;
            tile_body(cur, in, ro, co);
            const bool odd = (sub & 1) != 0;
            if (kPair) {
                emit_rows(make_tile(a, st, sub & 2), make_tile(a, st, sub | 1), row_a, ro, odd);
                if (COLS) {
                    emit_cols(make_tile(a, st, sub & 1), make_tile(a, st, (sub & 1) | 2), odd ? col_a1 : col_a0, co,
                              sub >= 2);
                    if (sub == 0) col_a0 = co;
                    if (sub == 1) col_a1 = co;
                }
                if (!odd) row_a = ro;
            } else {
                emit_single(cur, ro, co);
            }
            if (!has_next) break;
            st = nst;
            sub = nsub;
            in = nin;
        }
    }
}

// Workgroups of `fn` resident per CU, and the CU count, of the current
// device (queried once per device and kernel).
struct Residency {
    int wgs_per_cu;
    int cus;
};

Residency residency(const void* fn)
{
    struct Entry {
        int dev;
        const void* fn;
        Residency r;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return {1, 8};
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& e : cache)
        if (e.dev == dev && e.fn == fn) return e.r;
    Residency r{1, 8};
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) == hipSuccess && n > 0) r.wgs_per_cu = n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8) r.cus = n;
    cache.push_back({dev, fn, r});
    return r;
}

// Staged (error-feedback) launches: workgroups per CU.  Their traffic is the
// residual's read-modify-write plus bf16 reads and whole-line block stores;
// measured on the grouped 32 x 2880^2 step with 1 / 2 / 3 (the LDS limit)
// workgroups per CU: 0.49 / 0.535 / 0.53 of the HBM peak.
constexpr int kStagedWgsPerCu = 2;

// Launch one persistent grid: as many workgroups per XCD as fit at once
// (staged launches: at most kStagedWgsPerCu per CU), spread so that every
// workgroup of a slice takes the same number of tiles (to within one).
hipError_t launch_persistent(void (*fn)(TileArgs), TileArgs a, hipStream_t s)
{
    const Residency r = residency(reinterpret_cast<const void*>(fn));
    const int per_cu = a.stage ? min(r.wgs_per_cu, kStagedWgsPerCu) : r.wgs_per_cu;
    const int cap = per_cu * (r.cus / 8);
    int w = a.wgs_per_xcd < cap ? a.wgs_per_xcd : cap;
    if (w < 1) w = 1;
    const int rounds = (a.per_xcd + w - 1) / w;
    if (rounds > 1) w = (a.per_xcd + rounds - 1) / rounds;
    a.wgs_per_xcd = w;
    hipLaunchKernelGGL(fn, dim3(8 * w), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

namespace {

// Kernel selection: the tensorwise and no-outer modes take their scale from
// tensor_scale (or have none), so they have no precomputed-outer variant; the
// bf16 dequantised output exists only for the rowwise-only uses (2D outer, and
// 16 x 16 inner tiles under any of none / tensorwise / 2D outer).
// Launches of grouped cast-transposes (both directions, no dequantised
// output) with more than one group, or with one group that does not start at
// row 0 (the last launch of a split call), take the kernel with the group
// bookkeeping.
template <int B, int O, bool S, bool C, bool E, bool GV, bool Y, bool I, bool ST>
hipError_t launch_kt(const TileArgs& a, hipStream_t s)
{
    if constexpr (C && !Y) {
        if (a.ngroups > 1 || a.row0[0] != 0)
            return launch_persistent(k_tile<B, O, S, C, E, GV, Y, I, ST, true>, a, s);
    }
    return launch_persistent(k_tile<B, O, S, C, E, GV, Y, I, ST, false>, a, s);
}

template <int B, int O, bool S, bool C, bool E, bool I>
hipError_t pick_given_y(const TileArgs& a, hipStream_t s)
{
    const bool given = a.outer_given != 0;
    const bool y = a.y != nullptr;
    if constexpr (C && !I && !tile_unrolled<O, S, E>()) {
        if (a.stage) {
            if constexpr (O == kOuterNone || O == kOuterTensor)
                return launch_kt<B, O, S, C, E, false, false, I, true>(a, s);
            else
                return given ? launch_kt<B, O, S, C, E, true, false, I, true>(a, s)
                             : launch_kt<B, O, S, C, E, false, false, I, true>(a, s);
        }
    }
    if constexpr (C) {
        if constexpr (O == kOuterNone || O == kOuterTensor) {
            return launch_kt<B, O, S, C, E, false, false, I, false>(a, s);
        } else {
            return given ? launch_kt<B, O, S, C, E, true, false, I, false>(a, s)
                         : launch_kt<B, O, S, C, E, false, false, I, false>(a, s);
        }
    } else if constexpr (O == kOuterNone || O == kOuterTensor) {
        return y ? launch_kt<B, O, S, C, E, false, true, I, false>(a, s)
                 : launch_kt<B, O, S, C, E, false, false, I, false>(a, s);
    } else {
        if (given) return y ? launch_kt<B, O, S, C, E, true, true, I, false>(a, s)
                            : launch_kt<B, O, S, C, E, true, false, I, false>(a, s);
        return y ? launch_kt<B, O, S, C, E, false, true, I, false>(a, s)
                 : launch_kt<B, O, S, C, E, false, false, I, false>(a, s);
    }
}

template <int B, int O, bool C, bool I>
hipError_t pick_sr_ef(bool sr, bool ef, const TileArgs& a, hipStream_t s)
{
    if (sr) return ef ? pick_given_y<B, O, true, C, true, I>(a, s) : pick_given_y<B, O, true, C, false, I>(a, s);
    return ef ? pick_given_y<B, O, false, C, true, I>(a, s) : pick_given_y<B, O, false, C, false, I>(a, s);
}

template <int B>
hipError_t pick_outer(int outer_kind, bool sr, const TileArgs& a, hipStream_t s)
{
    const bool ef = a.residual != nullptr;
    const bool i2d = a.inner_2d != 0;
    if (a.col_codes == nullptr) {
        // rowwise only: the 2D outer mode, or 16 x 16 inner tiles
        if (!i2d) return pick_sr_ef<B, kOuter2D, false, false>(sr, ef, a, s);
        switch (outer_kind) {
        case kOuterNone: return pick_sr_ef<B, kOuterNone, false, true>(sr, ef, a, s);
        case kOuterTensor: return pick_sr_ef<B, kOuterTensor, false, true>(sr, ef, a, s);
        default: return pick_sr_ef<B, kOuter2D, false, true>(sr, ef, a, s);
        }
    }
    switch (outer_kind) {
    case kOuterNone:
        return i2d ? pick_sr_ef<B, kOuterNone, true, true>(sr, ef, a, s)
                   : pick_sr_ef<B, kOuterNone, true, false>(sr, ef, a, s);
    case kOuterTensor:
        return i2d ? pick_sr_ef<B, kOuterTensor, true, true>(sr, ef, a, s)
                   : pick_sr_ef<B, kOuterTensor, true, false>(sr, ef, a, s);
    case kOuter1D: return pick_sr_ef<B, kOuter1D, true, false>(sr, ef, a, s);   // no 16 x 16 inner tiles
    default:
        return i2d ? pick_sr_ef<B, kOuter2D, true, true>(sr, ef, a, s)
                   : pick_sr_ef<B, kOuter2D, true, false>(sr, ef, a, s);
    }
}

}  // namespace

hipError_t launch_tiles(int bias, int outer_kind, bool sr, const TileArgs& a, hipStream_t s)
{
    return bias == 7 ? pick_outer<7>(outer_kind, sr, a, s) : pick_outer<15>(outer_kind, sr, a, s);
}

}  // namespace fp4q
