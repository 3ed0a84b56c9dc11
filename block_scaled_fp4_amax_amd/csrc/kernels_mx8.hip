// kernels_mx8.hip -- the MXFP4 projection of a bf16 weight and its FP8
// re-encodings in one pass, for gfx950.
//
// "MXFP4 weight QAT recipes on MXFP8 and FP8 block-scaling hosts", Overview,
// Design and Correctness: the projected weight y (MXFP4 1x32 fake-quant, exact
// in bf16) feeds MXFP8 (1x32 UE8M0 scale, E4M3 payload) and Float8 128x128
// block-scaling hosts; the rowwise MXFP8 encoding of y is bitwise lossless,
// the 128x128 encoding lossless within each tile's E4M3 headroom, the
// columnwise (32x1) MXFP8 encoding a bounded re-quantisation.  Here one read
// of the weight produces y and all of them:
//   MXFP8 rowwise   scale 2^E, E = floor(log2 amax) - 8 (the OCP MX rule for
//                   E4M3), clamped to [-127, 127], amax over finite values;
//   MXFP8 colwise   the same on 32 x 1 blocks, stored as the rowwise layout of y^T;
//   128 x 128       one power-of-two FP32 scale per tile, the smallest with
//                   amax / s <= 448, and the payload also stored transposed.
// Every y = +-G[m] 2^k has a significand of 1 or 1.5, so for a block (tile)
// whose largest finite magnitude is G[M] 2^K both exponents are
// K + floor(log2 G[M]) - 8: the row and tile scales come from integer work on
// the MXFP4 exponent and the largest code, never from a division.
//
// Work decomposition: one workgroup (256 lanes) per 128 x 128 tile.
//   row pass     lane chunk = 8 consecutive bf16 of a row (one 16-byte load),
//                4 lanes = one 1x32 block (DPP maxima), 8 chunks per lane
//                issued before any arithmetic; MXFP4 codes and y through the
//                scaled FP4 conversions (as in the MXFP4 fake-quant kernel),
//                the MXFP8 payload through gfx950's scaled FP8 conversion,
//                which equals RNE onto E4M3 with subnormals for every
//                projected value and every scale 2^-127 .. 2^127 (checked on
//                the device) and gives 0xFF for NaN; y stays packed in
//                registers and is staged in LDS;
//   tile scale   maximum of K + floor(log2 G[M]) over the tile's blocks
//                (DPP, then LDS across the four waves);
//   row pass 2   the 128 x 128 payload of the lane's chunks from registers;
//   column pass  lane = 2 columns x 8 rows (eight 32-bit LDS reads), 4 lanes =
//                one 32 x 1 block per column: MXFP8 column payload and scale,
//                128 x 128 transposed payload.
// Stores cover whole 128-byte lines per wave instruction wherever the layout
// allows (row payloads: 4 rows x 128 B; column payloads: 4 columns x 128 B),
// with the non-temporal policy: nothing here is read back (8192^2 with every
// output: 0.115-0.118 -> 0.112 ms).
#include "fp4q_device.h"
#include "launch.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kT = 128;                     // tile edge
constexpr int kChunks = kT * kT / 8 / kThreads;   // 8-element chunks per lane and pass (8)

__device__ __forceinline__ int mx4_exponent(uint32_t abits)
{
    // k = ceil(log2(amax / 6)) from the bf16 bits of amax, floor -126, cap 125
    int e = (int)(abits >> 7);
    int k = e - 129 + (int)((abits & 0x7Fu) > 0x40u);
    k = e == 0 ? -126 : k;
    k = k < -126 ? -126 : k;
    return k > 125 ? 125 : k;
}

__device__ __forceinline__ float pow2f(int e)
{
    // 2^e for e in [-127, 127] (2^-127 is the subnormal 0x00400000)
    return e == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 + e) << 23);
}

template <int Q>
__device__ __forceinline__ void decode_pair(uint32_t codes, float scale, float& a, float& b)
{
    auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, scale, Q);
    a = f[0];
    b = f[1];
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// E4M3 payload bytes of v[0..3] / s (s a power of two) in one 32-bit word,
// byte i from v[i]: two conversions into the low and the high half.
typedef short s16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fp8x4(float v0, float v1, float v2, float v3, float s)
{
    s16x2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v0, v1, s, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, v2, v3, s, true);
    return __builtin_bit_cast(uint32_t, r);
}

// Eight payload bytes of eight floats (one 64-bit word).
__device__ __forceinline__ uint2 fp8x8(const float (&v)[8], float s)
{
    return make_uint2(fp8x4(v[0], v[1], v[2], v[3], s), fp8x4(v[4], v[5], v[6], v[7], s));
}

// LDS tile of y as bf16: [row][64 dwords], the dword index XOR 4 * (row / 8),
// which keeps a row chunk's four dwords contiguous (one 128-bit write) and
// spreads the column pass's reads (4 dword-columns x 16 row groups per wave
// instruction) over distinct banks.
__device__ __forceinline__ int lds_dword(int row, int dcol)
{
    return row * 64 + (dcol ^ (4 * ((row >> 3) & 15)));
}

template <bool WY, bool ROW8, bool COL8, bool BLK>
__global__ __launch_bounds__(kThreads) void k_mx_fp8(Mx8Args a)
{
    __shared__ uint32_t lds_y[kT * 64];
    __shared__ int red[kThreads / 64];

    const int tid = (int)threadIdx.x;
    const int tiles_c = (int)((a.cols + kT - 1) / kT);
    const int ti = (int)blockIdx.x / tiles_c, tj = (int)blockIdx.x - ti * tiles_c;
    const int r0 = ti * kT, c0 = tj * kT;
    const int rows_valid = min(kT, (int)a.rows - r0);   // multiples of 32
    const int cols_valid = min(kT, (int)a.cols - c0);

    // ---------------- row pass: loads
    uint4 in[kChunks];
    const rsrc_t rx = make_rsrc(a.x + (int64_t)r0 * a.ld + c0);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const int ch = j * kThreads + tid;
        const int row = ch >> 4, cc = ch & 15;   // 16 chunks per tile row
        const bool act = row < rows_valid && 8 * cc < cols_valid;
        in[j] = buf_load16(rx, act ? (uint32_t)(row * (int)a.ld + 8 * cc) * 2u : kOff);
    }

    uint4 ypk[kChunks];   // y of the lane's chunks, packed bf16
    int lmax = -1000;     // largest K + floor(log2 G[M]) of the lane's finite nonzero blocks
    const rsrc_t ry = make_rsrc(a.y ? a.y + (int64_t)r0 * a.cols + c0 : nullptr);
    const rsrc_t rp = make_rsrc(a.mx8_row ? a.mx8_row + (int64_t)r0 * a.cols + c0 : nullptr);
    const rsrc_t rps = make_rsrc(a.mx8_row_sc ? a.mx8_row_sc + (int64_t)r0 * (a.cols / 32) + c0 / 32 : nullptr);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const int ch = j * kThreads + tid;
        const int row = ch >> 4, cc = ch & 15;
        const bool act = row < rows_valid && 8 * cc < cols_valid;
        const uint32_t w[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
        const uint32_t am = quad_max_u32(bf16_absmax_bits(w), 4);   // block amax, bf16 bits
        const bool poisoned = am >= 0x7F80u;
        const int k = mx4_exponent(am);
        const float sk = __uint_as_float((uint32_t)(127 + k) << 23);
        uint32_t cw = 0;
        cw = fp4x2_rne_scaled<0>(cw, bf16_lo(w[0]), bf16_hi(w[0]), sk);
        cw = fp4x2_rne_scaled<1>(cw, bf16_lo(w[1]), bf16_hi(w[1]), sk);
        cw = fp4x2_rne_scaled<2>(cw, bf16_lo(w[2]), bf16_hi(w[2]), sk);
        cw = fp4x2_rne_scaled<3>(cw, bf16_lo(w[3]), bf16_hi(w[3]), sk);
        float yv[8];   // exact +-G[m] 2^k
        decode_pair<0>(cw, sk, yv[0], yv[1]);
        decode_pair<1>(cw, sk, yv[2], yv[3]);
        decode_pair<2>(cw, sk, yv[4], yv[5]);
        decode_pair<3>(cw, sk, yv[6], yv[7]);
        if (poisoned) {
#pragma unroll
            for (int q = 0; q < 8; ++q) yv[q] = __uint_as_float(0x7FC00000u);
        }
        uint4 yp;
        yp.x = pack_bf16x2(yv[0], yv[1]);
        yp.y = pack_bf16x2(yv[2], yv[3]);
        yp.z = pack_bf16x2(yv[4], yv[5]);
        yp.w = pack_bf16x2(yv[6], yv[7]);
        ypk[j] = yp;
        // largest code of the block: the code of amax / 2^k (RNE is monotone)
        const uint32_t mcode = fp4x2_rne_scaled<0>(0u, __uint_as_float(am << 16), 0.0f, sk) & 7u;
        const int L = (poisoned || mcode == 0u) ? -1000 : k + (int)(mcode >> 1) - 1;
        if (act) lmax = max(lmax, L);
        if (WY) buf_store16<kNT>(ry, act ? (uint32_t)(row * (int)a.cols + 8 * cc) * 2u : kOff, yp);
        if (ROW8) {
            const int E = max(-127, L - 8);
            buf_store8<kNT>(rp, act ? (uint32_t)(row * (int)a.cols + 8 * cc) : kOff, fp8x8(yv, pow2f(E)));
            buf_store_u8(rps, (act && (cc & 3) == 0) ? (uint32_t)(row * ((int)a.cols / 32) + cc / 4) : kOff,
                         (uint32_t)(E + 127));
        }
        if (COL8 || BLK) {
            const int d = lds_dword(row, 4 * cc);
            *reinterpret_cast<uint4*>(&lds_y[d]) = yp;
        }
    }
    if (!(COL8 || BLK)) return;

    // ---------------- tile scale: the largest block exponent of the tile
    int e_s = 0;
    if (BLK) {
        uint32_t m = (uint32_t)(lmax + 1024);   // non-negative
        m = wave_max_u32(m);
        if ((tid & 63) == 0) red[tid >> 6] = (int)m;
    }
    lds_barrier();
    if (BLK) {
        const int lt = max(max(red[0], red[1]), max(red[2], red[3])) - 1024;
        e_s = lt < -900 ? 0 : lt - 8;   // no finite nonzero value: scale 1
        const rsrc_t rbs = make_rsrc(a.blk_sc ? a.blk_sc + (int64_t)ti * (a.cols / kT) + tj : nullptr);
        buf_store_u32(rbs, tid == 0 ? 0u : kOff,
                      e_s >= -126 ? (uint32_t)(127 + e_s) << 23 : 0x00400000u >> (-127 - e_s));
    }
    // scaled conversions take a power-of-two scale down to 2^-127; below that
    // (a tile of tiny values only) the values are first multiplied by 2^32,
    // exactly, on a uniform branch
    const bool pre = e_s < -127;
    const float sblk = pow2f(pre ? e_s + 32 : e_s);
    auto prescale = [&](float (&v)[8]) __attribute__((always_inline)) {
        if (__builtin_expect(pre, 0)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] *= 0x1p32f;
        }
    };

    // ---------------- row pass 2: 128 x 128 payload, rowwise
    if (BLK) {
        const rsrc_t rb = make_rsrc(a.blk ? a.blk + (int64_t)r0 * a.cols + c0 : nullptr);
#pragma unroll
        for (int j = 0; j < kChunks; ++j) {
            const int ch = j * kThreads + tid;
            const int row = ch >> 4, cc = ch & 15;
            const bool act = row < rows_valid && 8 * cc < cols_valid;
            const uint32_t w[4] = {ypk[j].x, ypk[j].y, ypk[j].z, ypk[j].w};
            float yv[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                yv[2 * q] = bf16_lo(w[q]);
                yv[2 * q + 1] = bf16_hi(w[q]);
            }
            prescale(yv);
            buf_store8<kNT>(rb, act ? (uint32_t)(row * (int)a.cols + 8 * cc) : kOff, fp8x8(yv, sblk));
        }
    }

    // ---------------- column pass: lane = dword-column dc (columns 2 dc, 2 dc + 1) x 8 rows
    const int rows_c = (int)a.rows;
    const rsrc_t rc = make_rsrc(a.mx8_col ? a.mx8_col + (int64_t)c0 * rows_c + r0 : nullptr);
    const rsrc_t rcs = make_rsrc(a.mx8_col_sc ? a.mx8_col_sc + (int64_t)c0 * (rows_c / 32) + r0 / 32 : nullptr);
    const rsrc_t rbt = make_rsrc(a.blk_t ? a.blk_t + (int64_t)c0 * rows_c + r0 : nullptr);
#pragma unroll
    for (int j = 0; j < kChunks / 2; ++j) {
        const int ch = j * kThreads + tid;
        const int dc = ch >> 4, rg = ch & 15;   // 64 dword-columns x 16 groups of 8 rows
        const bool act = 2 * dc < cols_valid && 8 * rg < rows_valid;
        float lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t v = lds_y[lds_dword(8 * rg + i, dc)];
            lo[i] = bf16_lo(v);
            hi[i] = bf16_hi(v);
        }
        if (COL8) {
            // column maxima over finite values (IEEE maximum ignores a NaN operand)
            float ml = 0.0f, mh = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ml = fmaxf(ml, __builtin_fabsf(lo[i]));
                mh = fmaxf(mh, __builtin_fabsf(hi[i]));
            }
            const uint32_t bl = quad_max_u32(__float_as_uint(ml), 4);
            const uint32_t bh = quad_max_u32(__float_as_uint(mh), 4);
            // E = floor(log2 max) - 8 from the exponent field; zero and the one
            // subnormal projected value (2^-127) fall to the clamp
            const int El = max(-127, (int)(bl >> 23) - 127 - 8);
            const int Eh = max(-127, (int)(bh >> 23) - 127 - 8);
            const uint32_t ocol = (uint32_t)(2 * dc * rows_c + 8 * rg);
            buf_store8<kNT>(rc, act ? ocol : kOff, fp8x8(lo, pow2f(El)));
            buf_store8<kNT>(rc, act ? ocol + (uint32_t)rows_c : kOff, fp8x8(hi, pow2f(Eh)));
            const uint32_t osc = (uint32_t)(2 * dc * (rows_c / 32) + rg / 4);
            buf_store_u8(rcs, (act && (rg & 3) == 0) ? osc : kOff, (uint32_t)(El + 127));
            buf_store_u8(rcs, (act && (rg & 3) == 0) ? osc + (uint32_t)(rows_c / 32) : kOff, (uint32_t)(Eh + 127));
        }
        if (BLK) {
            prescale(lo);
            prescale(hi);
            const uint32_t ocol = (uint32_t)(2 * dc * rows_c + 8 * rg);
            buf_store8<kNT>(rbt, act ? ocol : kOff, fp8x8(lo, sblk));
            buf_store8<kNT>(rbt, act ? ocol + (uint32_t)rows_c : kOff, fp8x8(hi, sblk));
        }
    }
}

}  // namespace

hipError_t launch_mx_fp8(const Mx8Args& a, hipStream_t s)
{
    const int tiles = (int)(((a.rows + kT - 1) / kT) * ((a.cols + kT - 1) / kT));
    const bool wy = a.y != nullptr, row8 = a.mx8_row != nullptr || a.mx8_row_sc != nullptr;
    const bool col8 = a.mx8_col != nullptr || a.mx8_col_sc != nullptr;
    const bool blk = a.blk != nullptr || a.blk_t != nullptr || a.blk_sc != nullptr;
    const int key = (wy ? 8 : 0) | (row8 ? 4 : 0) | (col8 ? 2 : 0) | (blk ? 1 : 0);
    void (*fn)(Mx8Args) = nullptr;
    switch (key) {
#define FP4Q_MX8(K) case K: fn = k_mx_fp8<(K & 8) != 0, (K & 4) != 0, (K & 2) != 0, (K & 1) != 0>; break;
        FP4Q_MX8(0) FP4Q_MX8(1) FP4Q_MX8(2) FP4Q_MX8(3) FP4Q_MX8(4) FP4Q_MX8(5) FP4Q_MX8(6) FP4Q_MX8(7)
        FP4Q_MX8(8) FP4Q_MX8(9) FP4Q_MX8(10) FP4Q_MX8(11) FP4Q_MX8(12) FP4Q_MX8(13) FP4Q_MX8(14) FP4Q_MX8(15)
#undef FP4Q_MX8
    }
    hipLaunchKernelGGL(fn, dim3(tiles), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace fp4q
