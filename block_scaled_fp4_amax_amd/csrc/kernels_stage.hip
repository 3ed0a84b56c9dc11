// kernels_stage.hip -- the gather pass of the staged cast-transpose: moves the
// tile-major blocks written by the tile kernel into the row-major rowwise and
// columnwise buffers.
//
// Why: the rowwise and columnwise buffers of a cast-transpose are the
// rowwise layouts of X and X^T ("Block-Scaled FP8 and FP4 Weight
// Quantization", sections 1-3), so a 64 x 64 tile owns 32-byte pieces of 64
// code rows in each and 4-byte pieces of 64 scale rows.  On MI355X a store
// that leaves part of a 128-byte line unwritten costs far more HBM time than
// its bytes (measured on a copy of the grouped 32 x 2880^2 step's traffic:
// adding its codes and scale bytes as pieces of 32 or 64 bytes from different
// workgroups takes it from 0.48 to 0.82 ms, as whole lines to 0.53 ms).  The tile kernel
// therefore writes whole lines of a tile-major scratch, and this pass writes
// whole lines of the final buffers.  A work unit is a slice of up to 64 lines
// (rows of a rowwise buffer, columns of a columnwise one) of one 64-line band
// and one output kind; its bytes are one contiguous range of the buffer.  The
// workgroup reads the slice's part of every tile block along the band (one
// contiguous run per tile), places the pieces in LDS in output order and
// writes the range as 16-byte stores (staged layout in launch.h).
#include <algorithm>

#include "launch.h"

namespace fp4q {

namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 4;    // 16-byte chunks per lane issued before any store (fallback paths)

// One output range [dst, dst + nbytes) filled from staged blocks, by the
// whole workgroup.  LOC(off) gives the staged address of the G bytes at range
// offset off (off a multiple of G; G divides 16 and the range's start address
// is G-aligned).  Lanes take the 16-byte aligned chunks of the range in turn,
// kBatch of them per lane with every load issued before any store; a chunk
// wholly inside the range is one 16-byte store, the (at most two) edge chunks
// are stored G bytes at a time.
template <int G, class Loc>
__device__ __forceinline__ void gather_range(uint8_t* dst, int64_t nbytes, Loc loc)
{
    if (nbytes <= 0) return;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t c0 = a0 & ~(uintptr_t)15;
    const int64_t nchunks = (int64_t)((a0 + nbytes + 15 - c0) >> 4);
    for (int64_t base = 0; base < nchunks; base += (int64_t)kThreads * kBatch) {
        uint32_t v[kBatch][4];
        bool inb[kBatch][16 / G];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int64_t ch = base + (int64_t)k * kThreads + threadIdx.x;
            const int64_t rel0 = (int64_t)(c0 + 16 * ch) - (int64_t)a0;    // range offset of the chunk's first byte
#pragma unroll
            for (int j = 0; j < 16 / G; ++j) {
                const int64_t rel = rel0 + G * j;
                inb[k][j] = ch < nchunks && rel >= 0 && rel < nbytes;
                const int64_t r = inb[k][j] ? rel : 0;
                if (G == 16) {
                    const uint4 w = *reinterpret_cast<const uint4*>(loc(r));
                    v[k][0] = w.x; v[k][1] = w.y; v[k][2] = w.z; v[k][3] = w.w;
                } else if (G == 8) {
                    const uint2 w = *reinterpret_cast<const uint2*>(loc(r));
                    v[k][2 * j] = w.x;
                    v[k][2 * j + 1] = w.y;
                } else if (G == 4) {
                    v[k][j] = *reinterpret_cast<const uint32_t*>(loc(r));
                } else {
                    const uint32_t w = *loc(r);
                    const uint32_t sh = 8u * (uint32_t)(j & 3);
                    if ((j & 3) == 0) v[k][j >> 2] = 0u;
                    v[k][j >> 2] |= w << sh;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int64_t ch = base + (int64_t)k * kThreads + threadIdx.x;
            if (ch >= nchunks) continue;
            uint8_t* p = reinterpret_cast<uint8_t*>(c0 + 16 * (uintptr_t)ch);
            bool all = true;
#pragma unroll
            for (int j = 0; j < 16 / G; ++j) all = all && inb[k][j];
            if (all) {
                *reinterpret_cast<uint4*>(p) = make_uint4(v[k][0], v[k][1], v[k][2], v[k][3]);
            } else {
#pragma unroll
                for (int j = 0; j < 16 / G; ++j) {
                    if (!inb[k][j]) continue;
                    if (G == 8) *reinterpret_cast<uint2*>(p + 8 * j) = make_uint2(v[k][2 * j], v[k][2 * j + 1]);
                    else if (G == 4) *reinterpret_cast<uint32_t*>(p + 4 * j) = v[k][j];
                    else if (G == 1) p[j] = (uint8_t)(v[k][j >> 2] >> (8 * (j & 3)));
                }
            }
        }
    }
}

// q = o / d and the remainder for o / d <= 64 (a row or column of one band):
// a binary32 reciprocal estimate, off by at most one at that size, then one
// exact correction.
struct DivSmall {
    uint32_t d;
    float inv;
    __device__ __forceinline__ explicit DivSmall(uint32_t dd) : d(dd), inv(1.0f / (float)dd) {}
    __device__ __forceinline__ uint32_t quot(uint32_t o, uint32_t& rem) const
    {
        uint32_t q = (uint32_t)((float)o * inv);
        int32_t r = (int32_t)(o - q * d);
        if (r < 0) {
            --q;
            r += (int32_t)d;
        } else if (r >= (int32_t)d) {
            ++q;
            r -= (int32_t)d;
        }
        rem = (uint32_t)r;
        return q;
    }
};

// One band of one output kind: `lines` rows (or columns) of P bytes at dst,
// line l's bytes [t U, t U + U) coming from tile t's block (T tiles, the last
// one contributing only Ulast = P - (T - 1) U bytes) at in + t * tstride + l * U.
struct Band {
    uint8_t* dst;
    const uint8_t* in;
    int64_t tstride;
    int32_t P, U, Ulast, T, lines;
};

constexpr int kLdsBytes = 32768;

// Lines [l0, l0 + cnt) of a band through LDS: the inputs are read as runs of
// cnt * U contiguous bytes per tile (pieces of G bytes), placed in LDS in
// output order, and written out as 16-byte chunks of one contiguous range.
// Needs cnt * P <= kLdsBytes, dst + l0 * P 16-byte aligned, cnt * P % 16 == 0,
// and G dividing U, Ulast and P.
template <int G>
__device__ __forceinline__ void band_lds(const Band& b, int l0, int cnt, uint8_t* lds)
{
    const int per_tile = cnt * (b.U / G);              // pieces per tile run
    const int npieces = b.T * per_tile;
    const DivSmall dtile((uint32_t)per_tile), dunit((uint32_t)(b.U / G));
    for (int base = 0; base < npieces; base += kThreads * kBatch) {
        uint32_t v[kBatch][G >= 4 ? G / 4 : 1];
        int dsto[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int p = base + k * kThreads + (int)threadIdx.x;
            uint32_t rem, ub;
            const uint32_t t = dtile.quot((uint32_t)min(p, npieces - 1), rem);
            const uint32_t l = dunit.quot(rem, ub);
            ub *= G;
            const bool ok = p < npieces && !(t == (uint32_t)(b.T - 1) && (int)ub >= b.Ulast);
            dsto[k] = ok ? (int)(l * b.P + t * b.U + ub) : -1;
            const uint8_t* src = b.in + (int64_t)t * b.tstride + (int64_t)(l0 + (int)l) * b.U + ub;
            if (!ok) src = b.in;
            if (G == 16) {
                const uint4 w = *reinterpret_cast<const uint4*>(src);
                v[k][0] = w.x; v[k][1] = w.y; v[k][2] = w.z; v[k][3] = w.w;
            } else if (G == 8) {
                const uint2 w = *reinterpret_cast<const uint2*>(src);
                v[k][0] = w.x; v[k][1] = w.y;
            } else if (G == 4) {
                v[k][0] = *reinterpret_cast<const uint32_t*>(src);
            } else {
                v[k][0] = *src;
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (dsto[k] < 0) continue;
            uint8_t* q = lds + dsto[k];
            if (G == 16) *reinterpret_cast<uint4*>(q) = make_uint4(v[k][0], v[k][1], v[k][2], v[k][3]);
            else if (G == 8) *reinterpret_cast<uint2*>(q) = make_uint2(v[k][0], v[k][1]);
            else if (G == 4) *reinterpret_cast<uint32_t*>(q) = v[k][0];
            else *q = (uint8_t)v[k][0];
        }
    }
    __syncthreads();
    const int nchunks = cnt * b.P / 16;
    uint4* out = reinterpret_cast<uint4*>(b.dst + (int64_t)l0 * b.P);
    for (int c = (int)threadIdx.x; c < nchunks; c += kThreads) out[c] = reinterpret_cast<const uint4*>(lds)[c];
    __syncthreads();
}

// band_lds for the common shapes, with no division per piece: each tile's run
// (cnt * U contiguous bytes, 16-byte aligned) is read as 16-byte chunks by R =
// cnt * U / 16 neighbouring lanes, 256 / R runs per instruction, so a lane's
// chunk offset within a run, and with it the chunk's line and LDS position,
// is fixed for the whole unit and only the tile index advances.  W = min(U,
// 16) is the LDS write width: a chunk holds 16 / W lines (U <= 16) or part of
// one line (U = 32).  Needs cnt * U % 16 == 0, cnt * U <= 4096, the run start
// 16-byte aligned, P % W == 0, and the last tile whole (Ulast == U).
constexpr int kRunBatch = 12;
// Staged bytes are read once and the outputs are not read again by this
// pass, so both go with the non-temporal policy (measured on the grouped
// 32 x 2880^2 step: the gather 133 -> 110 us; the same policy on the tile
// pass's block and residual stores changed nothing, and on its residual
// loads cost 12%).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));

template <int W>
__device__ __forceinline__ void band_runs(const Band& b, int l0, int cnt, uint8_t* lds)
{
    const int R = cnt * b.U / 16;
    const int per_it = kThreads / R;
    const int tid = (int)threadIdx.x;
    const int ts = tid / R;
    const int o = (tid - ts * R) * 16;            // chunk offset in the run
    const bool lane_ok = ts < per_it;
    const int l = o / b.U;                         // first line of the chunk
    const int dst0 = l * b.P + (o - l * b.U);      // LDS offset for tile 0
    const uint8_t* src0 = b.in + (int64_t)l0 * b.U + o;
    for (int t0 = 0; t0 < b.T; t0 += per_it * kRunBatch) {
        uint32_t v[kRunBatch][4];    // plain words: an array of uint4 would live in scratch
#pragma unroll
        for (int k = 0; k < kRunBatch; ++k) {
            const int t = t0 + k * per_it + ts;
            const bool ok = lane_ok && t < b.T;
            const nt_u32x4 w = __builtin_nontemporal_load(
                reinterpret_cast<const nt_u32x4*>(ok ? src0 + (int64_t)t * b.tstride : b.in));
            v[k][0] = w[0]; v[k][1] = w[1]; v[k][2] = w[2]; v[k][3] = w[3];
        }
#pragma unroll
        for (int k = 0; k < kRunBatch; ++k) {
            const int t = t0 + k * per_it + ts;
            if (!(lane_ok && t < b.T)) continue;
            uint8_t* q = lds + dst0 + t * b.U;
            if (W == 16) {
                *reinterpret_cast<uint4*>(q) = make_uint4(v[k][0], v[k][1], v[k][2], v[k][3]);
            } else if (W == 8) {
                *reinterpret_cast<uint2*>(q) = make_uint2(v[k][0], v[k][1]);
                *reinterpret_cast<uint2*>(q + b.P) = make_uint2(v[k][2], v[k][3]);
            } else {
                *reinterpret_cast<uint32_t*>(q) = v[k][0];
                *reinterpret_cast<uint32_t*>(q + b.P) = v[k][1];
                *reinterpret_cast<uint32_t*>(q + 2 * b.P) = v[k][2];
                *reinterpret_cast<uint32_t*>(q + 3 * b.P) = v[k][3];
            }
        }
    }
    __syncthreads();
    const int nchunks = cnt * b.P / 16;
    nt_u32x4* out = reinterpret_cast<nt_u32x4*>(b.dst + (int64_t)l0 * b.P);
    for (int c = tid; c < nchunks; c += kThreads) {
        const uint4 q = reinterpret_cast<const uint4*>(lds)[c];
        const nt_u32x4 w = {q.x, q.y, q.z, q.w};
        __builtin_nontemporal_store(w, out + c);
    }
    __syncthreads();
}

// Lines [l0, l0 + cnt) of a band without LDS: each 16-byte output chunk
// gathered from the blocks directly (shapes the LDS path does not take).
__device__ __forceinline__ void band_direct(const Band& b, int l0, int cnt)
{
    const DivSmall dline((uint32_t)b.P);
    auto loc = [&](int64_t o) {
        uint32_t byte;
        const uint32_t l = dline.quot((uint32_t)o, byte);
        const uint32_t t = byte / (uint32_t)b.U;
        return b.in + (int64_t)t * b.tstride + (int64_t)(l0 + (int)l) * b.U + (byte - t * (uint32_t)b.U);
    };
    gather_range<1>(b.dst + (int64_t)l0 * b.P, (int64_t)cnt * b.P, loc);
}

// Work units: for each output kind (rowwise codes, scale bytes, 1D outer
// scales, then the columnwise ones), every band in slices of a.lines[k] lines
// (a.kind_units[k] .. a.kind_units[k + 1]).
__global__ __launch_bounds__(kThreads) void k_gather(GatherArgs a)
{
    __shared__ uint4 lds4[kLdsBytes / 16];
    uint8_t* lds = reinterpret_cast<uint8_t*>(lds4);
    const int64_t C = a.cols;
    const int nrb = a.tile0[a.ngroups] / a.tiles_c;    // 64-row bands in the launch
    const int opr = a.obs ? 64 / a.obs : 0;           // 1D outer groups per tile row
    // staging regions (launch.h): row codes, column codes, then one tail of
    // tailB bytes per tile; `sb` below is where a tile's tail would start if
    // it followed 4096 bytes of codes, so the tail parts sit at sb +
    // kStageTail (scale bytes) and sb + kStageRowOuter (1D outer scales)
    const int64_t blk = a.stage_block;
    const int64_t ntiles = a.tile0[a.ngroups];
    const int64_t tailB = blk - kStageTail;
    const uint8_t* const tails = a.stage + 2 * ntiles * kStageCodes;
    const int units = a.kind_units[6];
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int kind = 0;
        while (kind < 5 && a.kind_units[kind + 1] <= u) ++kind;
        const int w = u - a.kind_units[kind];
        const int per_band = (64 + a.lines[kind] - 1) / a.lines[kind];
        const int band = w / per_band;
        const int l0 = (w - band * per_band) * a.lines[kind];
        Band b;
        if (kind < 3) {
            // rowwise: band ti of group g, rows grow .. grow + nr - 1
            int g = 0;
            {
                int lo = 0, hi = a.ngroups - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (a.tile0[mid] / a.tiles_c <= band) lo = mid;
                    else hi = mid - 1;
                }
                g = lo;
            }
            const int ti = band - a.tile0[g] / a.tiles_c;
            const int Rg = a.row0[g + 1] - a.row0[g];
            const int64_t grow = a.row0[g] + 64 * ti;
            const int64_t f = a.tile0[g] + ti * a.tiles_c;                       // tile (ti, 0)
            const uint8_t* sb = tails + f * tailB - kStageTail;
            b.lines = min(64, Rg - 64 * ti);
            b.T = a.tiles_c;
            b.tstride = tailB;
            if (kind == 0) {
                b.P = (int32_t)(C / 2);
                b.U = 32;
                b.in = a.stage + f * kStageCodes;                                  // band's run of row codes
                b.tstride = kStageCodes;
                b.dst = a.row_codes + grow * b.P;
            } else if (kind == 1) {
                b.P = (int32_t)(C / 16);
                b.U = 4;
                b.in = sb + kStageTail;
                b.dst = a.row_scales + grow * b.P;
            } else {
                b.P = (int32_t)(C / a.obs) * 4;
                b.U = opr * 4;
                b.in = sb + kStageRowOuter;
                b.dst = reinterpret_cast<uint8_t*>(a.row_outer) + grow * b.P;
            }
        } else {
            // columnwise: band tj of group g, columns 64 tj .. 64 tj + nc - 1
            const int g = band / a.tiles_c;
            const int tj = band - g * a.tiles_c;
            const int64_t Rg = a.row0[g + 1] - a.row0[g];
            const uint8_t* sb = tails + (int64_t)(a.tile0[g] + tj) * tailB - kStageTail;   // tile (0, tj)
            const int64_t c0 = 64 * (int64_t)tj;
            b.lines = (int)min((int64_t)64, C - c0);
            b.T = (int32_t)((Rg + 63) / 64);
            b.tstride = (int64_t)a.tiles_c * tailB;
            if (kind == 3) {
                b.P = (int32_t)(Rg / 2);
                b.U = 32;
                b.in = a.stage + (ntiles + a.tile0[g] + (int64_t)tj * b.T) * kStageCodes;   // band's run
                b.tstride = kStageCodes;
                b.dst = a.col_codes + a.row0[g] * (C / 2) + c0 * b.P;
            } else if (kind == 4) {
                b.P = (int32_t)(Rg / 16);
                b.U = 4;
                b.in = sb + kStageTail + 256;
                b.dst = a.col_scales + a.row0[g] * (C / 16) + c0 * b.P;
            } else {
                b.P = (int32_t)(Rg / a.obs) * 4;
                b.U = opr * 4;
                b.in = sb + kStageRowOuter + 64 * opr * 4;
                b.dst = reinterpret_cast<uint8_t*>(a.col_outer) + (a.row0[g] * (C / a.obs) + c0 * (Rg / a.obs)) * 4;
            }
        }
        if (b.P <= 0 || l0 >= b.lines) continue;                  // uniform per workgroup
        b.Ulast = b.P - (b.T - 1) * b.U;
        const int cnt = min(a.lines[kind], b.lines - l0);
        const bool lds_ok = cnt * b.P <= kLdsBytes && (reinterpret_cast<uintptr_t>(b.dst + (int64_t)l0 * b.P) & 15) == 0 &&
                            (cnt * b.P) % 16 == 0;
        const int run = cnt * b.U;
        const bool runs_ok = lds_ok && b.Ulast == b.U && run % 16 == 0 && run <= 16 * kThreads &&
                             ((reinterpret_cast<uintptr_t>(b.in) + (uintptr_t)l0 * b.U) & 15) == 0 && b.tstride % 16 == 0;
        if (!lds_ok) {
            band_direct(b, l0, cnt);
        } else if (runs_ok && b.U % 16 == 0 && b.P % 16 == 0) {
            band_runs<16>(b, l0, cnt, lds);
        } else if (runs_ok && b.U == 8 && b.P % 8 == 0) {
            band_runs<8>(b, l0, cnt, lds);
        } else if (runs_ok && b.U == 4 && b.P % 4 == 0) {
            band_runs<4>(b, l0, cnt, lds);
        } else if (b.U % 16 == 0 && b.Ulast % 16 == 0 && b.P % 16 == 0) {
            band_lds<16>(b, l0, cnt, lds);
        } else if (b.U % 8 == 0 && b.Ulast % 8 == 0 && b.P % 8 == 0) {
            band_lds<8>(b, l0, cnt, lds);
        } else if (b.U % 4 == 0 && b.Ulast % 4 == 0 && b.P % 4 == 0) {
            band_lds<4>(b, l0, cnt, lds);
        } else {
            band_lds<1>(b, l0, cnt, lds);
        }
    }
}

}  // namespace

hipError_t launch_gather(GatherArgs a, hipStream_t s)
{
    // per kind: lines per work unit (the most that fit the LDS stage with a
    // byte count that is a multiple of 16 for every group), and the units
    const int nrb = a.tile0[a.ngroups] / a.tiles_c;
    const int ncb = a.ngroups * a.tiles_c;
    const int64_t C = a.cols;
    const bool have[6] = {a.row_codes != nullptr, a.row_scales != nullptr, a.row_outer != nullptr,
                          a.col_codes != nullptr, a.col_scales != nullptr, a.col_outer != nullptr};
    a.kind_units[0] = 0;
    for (int k = 0; k < 6; ++k) {
        int64_t pmax = 0;
        int m = 1;   // lines per unit must be a multiple of m
        auto pitch = [&](int64_t len) -> int64_t {
            const int kk = k % 3;
            if (kk == 0) return len / 2;
            if (kk == 1) return len / 16;
            return a.obs ? (len / a.obs) * 4 : 0;
        };
        if (k < 3) {
            pmax = pitch(C);
        } else {
            for (int g = 0; g < a.ngroups; ++g) pmax = std::max<int64_t>(pmax, pitch(a.row0[g + 1] - a.row0[g]));
        }
        for (int g = 0; g < (k < 3 ? 1 : a.ngroups); ++g) {
            const int64_t P = k < 3 ? pmax : pitch(a.row0[g + 1] - a.row0[g]);
            if (P <= 0) continue;
            int mg = 1;   // smallest m with m * P % 16 == 0
            while ((P * mg) % 16) mg *= 2;
            m = std::max(m, mg);
        }
        int lines = pmax > 0 ? (int)std::min<int64_t>(64, kLdsBytes / pmax) : 64;
        lines -= lines % m;
        if (lines < 16) lines = lines > 0 ? lines : 16;   // too wide for the LDS stage: the direct path
        a.lines[k] = lines;
        const int bands = k < 3 ? nrb : ncb;
        const int per_band = (64 + lines - 1) / lines;
        a.kind_units[k + 1] = a.kind_units[k] + ((have[k] && pmax > 0) ? bands * per_band : 0);
    }
    const int units = a.kind_units[6];
    if (units <= 0) return hipSuccess;
    const int grid = units < 8192 ? units : 8192;
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace fp4q
