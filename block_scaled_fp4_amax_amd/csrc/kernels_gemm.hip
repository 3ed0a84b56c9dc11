// kernels_gemm.hip -- the FP4 GEMM consumer: C = A . B^T with MXFP4 operands
// on gfx950's block-scaled matrix cores.
//
// "fp4-train" README, API: fp4_mm(a, b) computes a @ b^T on FP4 operands with
// the hardware's FP4 matrix instructions; Correctness: the result equals the
// dequantise-then-multiply path.  On gfx950 the FP4 matrix instruction is
// v_mfma_scale_f32_32x32x64_f8f6f4, which takes one UE8M0 scale per 32
// K-values of each operand row: exactly the MXFP4 rowwise layout the quantiser
// writes (codes [rows, K/2], low nibble first; scales [rows, K/32]).  Both
// operands are K-major (A [M, K], B [N, K]), so no transpose is needed.
//
// Operand layout of the instruction (checked on the device): lane l supplies
// row l % 32 of its 32 x 64 operand, 32 FP4 values (16 bytes, the low four of
// its eight operand dwords) that all take lane l's scale byte, and the two
// lanes l and l + 32 together cover the 64 K-values; A and B lanes pair
// position by position.  Accumulator register r of lane l holds
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  So lane l's operand is one MX
// block: 16 contiguous bytes of a row, with that block's scale byte.
//
// Work decomposition: one workgroup of 512 lanes (8 waves, 2 x 4, two per
// SIMD so that one wave's loads and LDS traffic overlap the other's matrix
// instructions) per 256 x 256 tile of C; each wave owns 128 x 64 (4 x 2
// instructions, 128 accumulators).
// K advances in tiles of 256 values (128 bytes of codes per row) staged in LDS
// through registers, double-buffered: the next tile's global loads are issued
// before the current tile's 32 instructions per wave, and written to the other
// LDS buffer after them (one barrier per K-tile).  In LDS a row's eight 16-byte
// chunks are XOR-swizzled by the row (chunk ^ ((row / 2) & 7)), so the rows a
// wave reads for one operand spread over all banks.  Rows beyond M or N and
// K-values beyond K load as zero codes with scale byte 0 (2^-127), adding
// exact zeros.  Workgroup ids are remapped so each XCD (ids dealt round-robin)
// works on a contiguous run of tiles that share operand panels in its L2.
#include <mutex>

#include "fp4q_device.h"
#include "launch.h"

namespace fp4q {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;                  // 8 waves, two per SIMD
constexpr int kWaveM = 2, kWaveN = 4;          // wave grid over the tile
constexpr int kTM = 4, kTN = 2;                // 32 x 32 blocks per wave: 128 x 64
constexpr int kBM = 256;                       // tile rows (A) = tile columns (B)
constexpr int kBK = 256;                       // K-values per K-tile
constexpr int kRowB = kBK / 2;                 // code bytes per row and K-tile (128)
constexpr int kChunks = kBM * kRowB / 16;      // 16-byte chunks per operand tile (2048)
constexpr int kScB = kBK / 32;                 // scale bytes per row and K-tile (8)

struct Smem {
    uint4 code[2][2][kChunks];                 // [buffer][A, B][chunk]   128 KiB
    uint2 scale[2][2][kBM];                    // [buffer][A, B][row]       8 KiB
};

// 16-byte chunk c of a row lives at chunk c ^ ((row / 2) & 7): the 16 rows one
// quarter-wave reads (two rows per 256-byte bank window) land on distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Scale layouts the kernel reads (SL):
//   kScaleRowBytes   rowwise [rows, K/32] as the quantiser writes it, any K:
//                    one byte load per scale;
//   kScaleRow8       the same when K % 256 == 0 and the base is 8-byte aligned:
//                    one 8-byte load per row and K-tile;
//   kScaleTiled      the GEMM-ready layout [ceil(rows/256)][ceil(K/256)][256][8]
//                    (zero-padded): a workgroup's 2 KiB of scales for one K-tile
//                    are contiguous, one coalesced 8-byte load per lane.
enum { kScaleRowBytes = 0, kScaleRow8 = 1, kScaleTiled = 2 };

// The main loop moves a K-tile in quarters so that its global loads and LDS
// writes interleave with the matrix instructions.  A K-tile at or beyond the
// end of K loads zeros.
struct Stage {
    uint4 a[4], b[4];
    uint32_t sc[8];                            // scale bytes (or two words) of the lane's scale row
};

// Quarter Q of a K-tile: code chunk Q of A and of B per lane (rows q / 8,
// chunk q % 8 for q = Q * 512 + lane: eight lanes read one row's 128 bytes);
// with the last quarter, lanes 0..255 fetch the scale row of A row `lane`,
// lanes 256..511 that of B row `lane - 256`.
template <int SL>
__device__ __forceinline__ void load_quarter(const GemmArgs& g, const rsrc_t& ra, const rsrc_t& rb, const rsrc_t& ras,
                                             const rsrc_t& rbs, int kt, int rows_a, int rows_b, int Q, Stage& st)
{
    const int tid = (int)threadIdx.x;
    const int kb0 = kt * kRowB;                // byte offset of the K-tile in a code row
    const int kb_end = g.K / 2;
    {
        const int q = Q * kThreads + tid;
        const int row = q >> 3, c = q & 7;
        const int kb = kb0 + 16 * c;
        const bool kin = kb < kb_end;
        st.a[Q] = buf_load16<0>(ra, (row < rows_a && kin) ? (uint32_t)(row * kb_end + kb) : kOff);
        st.b[Q] = buf_load16<0>(rb, (row < rows_b && kin) ? (uint32_t)(row * kb_end + kb) : kOff);
    }
    if (Q != 3) return;
    const int sb0 = kt * kScB, sb_end = g.K / 32;
    const bool is_b = tid >= kBM;
    const int srow = is_b ? tid - kBM : tid;
    const int srows = is_b ? rows_b : rows_a;
    const rsrc_t rs = is_b ? rbs : ras;
    if (SL == kScaleRowBytes) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool kin = sb0 + j < sb_end;
            st.sc[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, (srow < srows && kin) ? (uint32_t)(srow * sb_end + sb0 + j)
                                                                                      : kOff, 0, 0);
        }
    } else {
        // 8 bytes of the lane's row: rowwise (K % 256 == 0, so a K-tile is
        // whole or beyond K) or the tiled block of this K-tile (padded)
        const bool kin = sb0 < sb_end;
        const uint32_t o = !kin ? kOff : SL == kScaleRow8 ? (srow < srows ? (uint32_t)(srow * sb_end + sb0) : kOff)
                                                           : (uint32_t)((kt * kBM + srow) * 8);
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
        st.sc[0] = v[0];
        st.sc[1] = v[1];
    }
}

template <int SL>
__device__ __forceinline__ void store_quarter(Smem& sm, int buf, const Stage& st, int Q)
{
    const int tid = (int)threadIdx.x;
    {
        const int q = Q * kThreads + tid;
        const int row = q >> 3, c = q & 7;
        sm.code[buf][0][swz(row, c)] = st.a[Q];
        sm.code[buf][1][swz(row, c)] = st.b[Q];
    }
    if (Q != 3) return;
    uint2 w;
    if (SL == kScaleRowBytes) {
        w.x = st.sc[0] | (st.sc[1] << 8) | (st.sc[2] << 16) | (st.sc[3] << 24);
        w.y = st.sc[4] | (st.sc[5] << 8) | (st.sc[6] << 16) | (st.sc[7] << 24);
    } else {
        w = make_uint2(st.sc[0], st.sc[1]);
    }
    const bool is_b = tid >= kBM;
    sm.scale[buf][is_b ? 1 : 0][is_b ? tid - kBM : tid] = w;
}

__device__ __forceinline__ uint32_t scale_byte(uint2 s, int idx)
{
    // byte idx (0..7) of the row's K-tile scales
    const uint32_t w = idx < 4 ? s.x : s.y;
    return (w >> (8 * (idx & 3))) & 0xFFu;
}

// Tile of this workgroup: XCD x takes the contiguous run x * T/8 .. of the
// tile order when T % 8 == 0 (ids are dealt round-robin to the 8 XCDs); within
// the order, groups of 4 tile rows are walked column by column.
__device__ __forceinline__ void tile_of_workgroup(const GemmArgs& g, int& tm, int& tn)
{
    const int T = g.tiles_m * g.tiles_n;
    int t = (int)blockIdx.x;
    if (T % 8 == 0) t = (t & 7) * (T >> 3) + (t >> 3);
    const int gm = 4;
    const int group = t / (gm * g.tiles_n);
    const int first_m = group * gm;
    const int rows_in_group = min(gm, g.tiles_m - first_m);
    const int in_group = t - group * gm * g.tiles_n;
    tm = first_m + in_group % rows_in_group;
    tn = in_group / rows_in_group;
}

// C tile: accumulator r of lane l of wave (wm, wn) holds
// C[m0 + 128 wm + 32 i + 8 (r / 4) + 4 (l / 32) + r % 4][n0 + 64 wn + 32 j + l % 32].
template <bool CF32>
__device__ __forceinline__ void store_c(const GemmArgs& g, const v16f_t (&acc)[kTM][kTN], int m0, int n0,
                                        unsigned char* smem_raw)
{
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / kWaveN, wn = wave % kWaveN;
    const int lr = lane & 31, lh = lane >> 5;
    const int64_t ldc = g.ldc;
    constexpr int kES = CF32 ? 4 : 2;                  // bytes per element of C
    const bool whole = m0 + kBM <= g.M && n0 + kBM <= g.N && ((uint64_t)ldc * kES) % 16 == 0 &&
                       (reinterpret_cast<uintptr_t>(g.c) & 15) == 0;
    if (whole) {
        // a whole tile and 16-byte aligned rows of C (uniform over the
        // workgroup): each wave stages its block in its own 16 KiB of the now
        // idle LDS (bf16: all 128 rows; FP32: 64 rows at a time), rows of 64
        // elements with the 16-byte chunk index XOR-swizzled by the row, then
        // writes 16-byte chunks, eight or sixteen lanes per row of C
        constexpr int kRowB = 64 * kES;                // staged row bytes
        constexpr int kCpr = kRowB / 16;               // chunks per staged row
        constexpr int kHalves = CF32 ? 2 : 1;
        constexpr int kTMh = kTM / kHalves;
        unsigned char* stage = smem_raw + wave * 16384;
#pragma unroll
        for (int h = 0; h < kHalves; ++h) {
            __syncthreads();                           // the LDS is free (operands, previous half)
#pragma unroll
            for (int ii = 0; ii < kTMh; ++ii)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int lrow = ii * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                        const int cb = (j * 32 + lr) * kES;
                        unsigned char* dst = stage + lrow * kRowB + (((cb >> 4) ^ (lrow & (kCpr - 1))) << 4) + (cb & 15);
                        const float v = acc[h * kTMh + ii][j][r];
                        if (CF32) *reinterpret_cast<float*>(dst) = v;
                        else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f32_to_bf16(v);
                    }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int ch = q * 64 + lane;
                const int lrow = ch / kCpr, c = ch % kCpr;
                const uint4 v = *reinterpret_cast<const uint4*>(stage + lrow * kRowB + ((c ^ (lrow & (kCpr - 1))) << 4));
                const int64_t grow = m0 + wm * 32 * kTM + h * kTMh * 32 + lrow;
                const int64_t gcol = n0 + wn * 32 * kTN + c * (16 / kES);
                st_nt16(static_cast<unsigned char*>(g.c) + (grow * ldc + gcol) * kES, v);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int col = n0 + wn * 32 * kTN + j * 32 + lr;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 32 * kTM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (row < g.M && col < g.N) {
                    const float v = acc[i][j][r];
                    if (CF32) static_cast<float*>(g.c)[(int64_t)row * ldc + col] = v;
                    else static_cast<uint16_t*>(g.c)[(int64_t)row * ldc + col] = (uint16_t)f32_to_bf16(v);
                }
            }
        }
}

template <bool CF32, int SL>
__global__ __launch_bounds__(kThreads) void k_mx_gemm(GemmArgs g)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

    int tm, tn;
    tile_of_workgroup(g, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBM;
    const int rows_a = min(kBM, g.M - m0), rows_b = min(kBM, g.N - n0);
    const int64_t lda = g.K / 2;
    const rsrc_t ra = make_rsrc(g.a + (int64_t)m0 * lda);
    const rsrc_t rb = make_rsrc(g.b + (int64_t)n0 * lda);
    // tiled scales: the workgroup's row tile is block tm (tn) of ceil(K/256) K-tiles
    const int kts = (g.K + kBK - 1) / kBK;
    const rsrc_t ras = make_rsrc(SL == kScaleTiled ? g.as + (int64_t)tm * kts * kBM * 8 : g.as + (int64_t)m0 * (g.K / 32));
    const rsrc_t rbs = make_rsrc(SL == kScaleTiled ? g.bs + (int64_t)tn * kts * kBM * 8 : g.bs + (int64_t)n0 * (g.K / 32));

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / kWaveN, wn = wave % kWaveN;   // wave rows 128 wm.., columns 64 wn..
    const int lr = lane & 31, lh = lane >> 5;

    v16f_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = v16f_t{};

    const int nk = (g.K + kBK - 1) / kBK;
    Stage st;
    // prologue: tile 0 into LDS buffer 0, tile 1 in flight into the registers
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) load_quarter<SL>(g, ra, rb, ras, rbs, 0, rows_a, rows_b, Q, st);
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) store_quarter<SL>(sm, 0, st, Q);
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) load_quarter<SL>(g, ra, rb, ras, rbs, 1, rows_a, rows_b, Q, st);
    __syncthreads();

    // iteration kt: LDS buffer kt % 2 holds tile kt, the registers receive
    // tile kt + 1; during the 64 instructions of each wave, tile kt + 1 goes
    // to the other buffer and tile kt + 2 is requested, a quarter per K-step
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1, nxt = cur ^ 1;
        const int ksteps = min(kBK / 64, (g.K - kt * kBK) >> 6);   // K-steps inside K (K % 64 == 0)
        uint2 sa[kTM], sb[kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i) sa[i] = sm.scale[cur][0][wm * 32 * kTM + i * 32 + lr];
#pragma unroll
        for (int j = 0; j < kTN; ++j) sb[j] = sm.scale[cur][1][wn * 32 * kTN + j * 32 + lr];
        v8i_t av[2][kTM], bv[2][kTN];
        auto read_ops = [&](int ks, int p) __attribute__((always_inline)) {
            const int chunk = 2 * ks + lh;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const uint4 x = sm.code[cur][0][swz(wm * 32 * kTM + i * 32 + lr, chunk)];
                av[p][i] = v8i_t{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const uint4 y = sm.code[cur][1][swz(wn * 32 * kTN + j * 32 + lr, chunk)];
                bv[p][j] = v8i_t{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
            }
        };
        read_ops(0, 0);
#pragma unroll
        for (int ks = 0; ks < kBK / 64; ++ks) {
            const int p = ks & 1;
            // the next K-step's operand reads go out a whole K-step (16
            // instructions) before their use; the fences keep the scheduler
            // from moving them next to their consumers
            if (ks + 1 < ksteps) read_ops(ks + 1, p ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            const int chunk = 2 * ks + lh;
            // a K-tile's K-steps beyond K hold only zero codes: skipped
            if (ks < ksteps) {
#pragma unroll
                for (int i = 0; i < kTM; ++i) {
                    const int sai = (int)scale_byte(sa[i], chunk);
#pragma unroll
                    for (int j = 0; j < kTN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            av[p][i], bv[p][j], acc[i][j], 4, 4, 0, sai, 0, (int)scale_byte(sb[j], chunk));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            store_quarter<SL>(sm, nxt, st, ks);
            load_quarter<SL>(g, ra, rb, ras, rbs, kt + 2, rows_a, rows_b, ks, st);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }

    store_c<CF32>(g, acc, m0, n0, smem_raw);
}

// Direct-to-LDS variant for the GEMM-ready scale layout.  gfx950's buffer loads
// with the LDS flag write a wave's 64 results (16 bytes each here) to 64
// consecutive LDS slots at a wave-uniform base, bypassing registers, so a
// K-tile moves into LDS without register staging or LDS write instructions.
// Two buffers: K-tile kt + 1 is requested right after the barrier that opens
// K-tile kt (the barrier also retires every wave's reads of the buffer it
// overwrites); the first two K-tiles are requested before the loop.  Slot l of
// code block b (1 KiB, rows 8 b .. 8 b + 7) receives row 8 b + l / 8, stored
// chunk l % 8, i.e. K-chunk (l % 8) ^ ((row / 2) & 7) of the row: the same
// swizzled layout the register-staged kernel writes.  Scale rows (eight bytes
// each) arrive two per lane: issuing a load costs about the same whatever its
// width, and four 4-byte scale loads per loading wave took 2% longer (8192^3:
// 285 against 279 us).  The loads are issued from inline assembly with
// explicit waits: the compiler's own wait insertion cannot tell the two
// buffers apart and would wait for the next K-tile's loads before every read
// of the current one.  Only waves 0..3 (one per SIMD) load.  A
// burst of load instructions issues slowly (the K-tile's 68 KiB enter the CU at
// the rate its memory path accepts them), and a wave that is issuing loads
// issues no matrix instructions: with the loads on one wave of each SIMD, the
// SIMD's other wave keeps the matrix pipe fed meanwhile.
struct SmemLds {
    uint4 code[2][2][kChunks];                 // [buffer][A, B][chunk]         128 KiB
    uint2 scale[2][2][kBM];                    // [buffer][A, B][row]  8 KiB
};

// The loads set m0 (the LDS base) themselves; no other instruction of these
// kernels reads m0, so the reserved-register clobber warning is silenced.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t voff, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :
                 : "v"(voff), "s"(lds_base), "s"(r)
                 : "memory", "m0");
}

#pragma clang diagnostic pop

// wait until at most N of this wave's vector-memory loads are outstanding
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// The seventeen loads of K-tile kt into buffer buf issued by wave w < 4: code
// blocks 8 w .. 8 w + 7 of A and of B, and one 1 KiB block of scale rows.
// Waves 4..7 load nothing.  Codes beyond the rows or
// K load as zeros; the tiled scales are zero-padded.
__device__ __forceinline__ void lds_tile(const GemmArgs& g, SmemLds& sm, const rsrc_t& ra, const rsrc_t& rb,
                                         const rsrc_t& ras, const rsrc_t& rbs, int kt, int rows_a, int rows_b,
                                         int buf, int wave, int lane)
{
    if (wave >= 4) return;                     // uniform
    const int kb_end = g.K / 2;
#pragma unroll
    for (int o = 0; o < 2; ++o) {
        const int rows = o ? rows_b : rows_a;
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int b = 8 * wave + h;
            const int row = 8 * b + (lane >> 3);
            const int c = (lane & 7) ^ ((row >> 1) & 7);
            const int kb = kt * kRowB + 16 * c;
            const uint32_t off = (row < rows && kb < kb_end) ? (uint32_t)(row * kb_end + kb) : kOff;
            lds_load16(o ? rb : ra, off, lds_addr(&sm.code[buf][o][b * 64]));
        }
    }
    // scale rows: wave w takes rows 128 (w & 1) .. + 127 of operand w >> 1,
    // two 8-byte rows per lane
    const int o = wave >> 1, r0 = 128 * (wave & 1);
    lds_load16(o ? rbs : ras, (uint32_t)((kt * kBM + r0) * 8 + 16 * lane), lds_addr(&sm.scale[buf][o][r0]));
}

constexpr int kLdsLoadsPerTile = 17;           // per loading wave

template <bool CF32>
__global__ __launch_bounds__(kThreads) void k_mx_gemm_lds(GemmArgs g)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    SmemLds& sm = *reinterpret_cast<SmemLds*>(smem_raw);

    int tm, tn;
    tile_of_workgroup(g, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBM;
    const int rows_a = min(kBM, g.M - m0), rows_b = min(kBM, g.N - n0);
    const int64_t lda = g.K / 2;
    const rsrc_t ra = make_rsrc(g.a + (int64_t)m0 * lda);
    const rsrc_t rb = make_rsrc(g.b + (int64_t)n0 * lda);
    const int nk = (g.K + kBK - 1) / kBK;
    const rsrc_t ras = make_rsrc(g.as + (int64_t)tm * nk * kBM * 8);
    const rsrc_t rbs = make_rsrc(g.bs + (int64_t)tn * nk * kBM * 8);

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wm = wave / kWaveN, wn = wave % kWaveN;
    const int lr = lane & 31, lh = lane >> 5;

    v16f_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = v16f_t{};

    lds_tile(g, sm, ra, rb, ras, rbs, 0, rows_a, rows_b, 0, wave_u, lane);
    if (nk > 1) lds_tile(g, sm, ra, rb, ras, rbs, 1, rows_a, rows_b, 1, wave_u, lane);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        // this wave's part of K-tile kt has landed (K-tile 1 may still be in
        // flight at kt = 0; waves that load nothing wait for nothing); the
        // barrier makes every wave's part visible
        if (kt == 0) wait_vm<kLdsLoadsPerTile>();
        else wait_vm<0>();
        __syncthreads();
        if (kt >= 1 && kt + 1 < nk) lds_tile(g, sm, ra, rb, ras, rbs, kt + 1, rows_a, rows_b, cur ^ 1, wave_u, lane);
        uint2 sa[kTM], sb[kTN];
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int r = wm * 32 * kTM + i * 32 + lr;
            sa[i] = sm.scale[cur][0][r];
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int r = wn * 32 * kTN + j * 32 + lr;
            sb[j] = sm.scale[cur][1][r];
        }
        v8i_t av[2][kTM], bv[2][kTN];
        auto read_ops = [&](int ks, int p) __attribute__((always_inline)) {
            const int chunk = 2 * ks + lh;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const uint4 x = sm.code[cur][0][swz(wm * 32 * kTM + i * 32 + lr, chunk)];
                av[p][i] = v8i_t{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const uint4 y = sm.code[cur][1][swz(wn * 32 * kTN + j * 32 + lr, chunk)];
                bv[p][j] = v8i_t{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
            }
        };
        read_ops(0, 0);
#pragma unroll
        for (int ks = 0; ks < kBK / 64; ++ks) {
            const int p = ks & 1;
            if (ks + 1 < kBK / 64) read_ops(ks + 1, p ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            const int chunk = 2 * ks + lh;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int sai = (int)scale_byte(sa[i], chunk);
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        av[p][i], bv[p][j], acc[i][j], 4, 4, 0, sai, 0, (int)scale_byte(sb[j], chunk));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // no load is in flight here: the last K-tile's loads were waited for
    store_c<CF32>(g, acc, m0, n0, smem_raw);
}

// GEMM-ready scales: out[(t * kts + kt) * 256 + r][j] = in[t * 256 + r][kt * 8 + j],
// zero outside [rows, K/32].  One lane per 8 output bytes.
__global__ __launch_bounds__(256) void k_mx_scales_tiled(const uint8_t* __restrict__ in, int32_t rows, int32_t nsb,
                                                         int32_t kts, int64_t total, uint8_t* __restrict__ out)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-byte group
    if (q >= total) return;
    const int r = (int)(q % kBM);
    const int64_t tk = q / kBM;
    const int kt = (int)(tk % kts);
    const int t = (int)(tk / kts);
    const int row = t * kBM + r;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int col = kt * 8 + j;
        const uint32_t v = (row < rows && col < nsb) ? (uint32_t)in[(int64_t)row * nsb + col] : 0u;
        w[j >> 2] |= v << (8 * (j & 3));
    }
    *reinterpret_cast<uint2*>(out + q * 8) = make_uint2(w[0], w[1]);
}

}  // namespace

hipError_t launch_mx_scales_tiled(const uint8_t* in, int64_t rows, int64_t K, uint8_t* out, hipStream_t s)
{
    const int32_t kts = (int32_t)((K + kBK - 1) / kBK);
    const int64_t tiles = (rows + kBM - 1) / kBM;
    const int64_t total = tiles * kts * kBM;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(k_mx_scales_tiled, dim3((uint32_t)grid), dim3(256), 0, s, in, (int32_t)rows, (int32_t)(K / 32),
                       kts, total, out);
    return hipGetLastError();
}

hipError_t launch_mx_gemm(const GemmArgs& g, hipStream_t s)
{
    const int T = g.tiles_m * g.tiles_n;
    static_assert(sizeof(Smem) == sizeof(SmemLds), "both kernels take 136 KiB of the CU's 160 KiB");
    const size_t lds = sizeof(Smem);
    // GEMM-ready scales take the direct-to-LDS kernel from three K-tiles on:
    // measured on uniformly random operands it was ahead of the register-
    // staged one by 4-14% on 17 of 18 shapes (K from 768 to 16384, M and N
    // from 1024 to 16384), and even at 8192^2 x 2880, whose K tail the
    // register-staged kernel skips.  Its wait for K-tile 0 needs two K-tiles.
    const bool direct = g.scale_layout == kScaleTiled && g.K >= 3 * kBK;
    const int variant = direct ? 6 + (g.c_f32 ? 1 : 0)
                               : (g.scale_layout == kScaleTiled ? 4 : g.scale_layout == kScaleRow8 ? 2 : 0) +
                                     (g.c_f32 ? 1 : 0);
    static void (*const fns[8])(GemmArgs) = {
        k_mx_gemm<false, kScaleRowBytes>, k_mx_gemm<true, kScaleRowBytes>, k_mx_gemm<false, kScaleRow8>,
        k_mx_gemm<true, kScaleRow8>,      k_mx_gemm<false, kScaleTiled>,   k_mx_gemm<true, kScaleTiled>,
        k_mx_gemm_lds<false>,             k_mx_gemm_lds<true>};
    // the dynamic-LDS limit is a property of the kernel function: raise it once
    // per variant (not per launch, so launches stay capturable in a HIP graph)
    static std::once_flag once[8];
    static hipError_t attr_status[8];
    std::call_once(once[variant], [&] {
        attr_status[variant] = hipFuncSetAttribute(reinterpret_cast<const void*>(fns[variant]),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    });
    if (attr_status[variant] != hipSuccess) return attr_status[variant];
    hipLaunchKernelGGL(fns[variant], dim3(T), dim3(kThreads), lds, s, g);
    return hipGetLastError();
}

}  // namespace fp4q
