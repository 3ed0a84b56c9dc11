/*
 * fp4_oracle.c -- plain CPU oracle for block-scaled FP4 quantisation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test-suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or constant generator with the HIP
 * library under block_scaled_fp4_amax_amd/.
 *
 * Sources (cited by page title and section):
 *   [ALTO]  "NVFP4 / AMD-FP4 outer-block (two-level) scaling for FP4 training"
 *           -- Background, Technical design, Implementation, Op-level tests.
 *   [FP4T]  "fp4-train" README -- Method, API, Correctness, Requirements.
 *   [TEQAT] "MXFP4 weight QAT recipes on MXFP8 and FP8 block-scaling hosts"
 *           -- Design, Correctness, Guards, Known limitations.
 *   [BSWQ]  "Block-Scaled FP8 and FP4 Weight Quantization" -- sections 1-4.
 *
 * Arithmetic: every named floating-point step is ONE IEEE-754 binary32
 * operation rounded to nearest-even (the pages hold the outer scale and the
 * error-feedback residual in FP32, so decisions are taken in binary32).  This
 * file must be compiled with -O2 -fno-fast-math -ffp-contract=off on x86-64
 * (SSE scalar float, no FMA contraction, subnormals honoured).  Where a value
 * is exact in any precision (decoded grids, powers of two) double is used only
 * to hold it.
 *
 * Everything is written as the plain definition: nearest-value searches over
 * whole code tables, one RNG call per element, explicit transposes.  It is
 * slow on purpose; OpenMP only splits independent rows/blocks.
 *
 * Readings of points the pages leave open are listed in the design notes; the
 * ones that change bits are repeated at the function that applies them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Format primitives                                                         */
/* ------------------------------------------------------------------------ */

static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32: a bf16 is the upper half of a binary32, so widening is exact. */
float orc_bf16_to_f32(uint16_t b) { return f_from_bits((uint32_t)b << 16); }

/* fp32 -> bf16, round to nearest even on bit 16; any NaN becomes the canonical
 * quiet NaN 0x7FC0.  (Plain definition of RNE to 8 significant bits.) */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = bits_from_f(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
    return (uint16_t)upper;
}

int orc_abi_version(void) { return 1; }

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count for the parallel loops that follow (timing only: the loops
 * split independent rows, so results do not depend on it). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* E2M1 magnitude grid, [FP4T] Method: {0, .5, 1, 1.5, 2, 3, 4, 6}; the 3-bit
 * magnitude code m indexes it and the sign is a separate bit (code = s*8+m). */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int m) { return E2M1_GRID[m & 7]; }

/* Round-to-nearest-even onto the E2M1 magnitude grid, saturating at 6
 * ([TEQAT] Correctness: RTNE midpoints, satfinite cap).  "Even" is the even
 * code index.  a >= 0.  Plain nearest search over the 8 grid points. */
int orc_e2m1_rne(double a)
{
    /* satfinite: at or above the largest grid point the code is 6's.  (Stated
     * first so the distance search below only sees a < 6, where every
     * difference is exact in double.) */
    if (a >= 6.0) return 7;
    int best = 0;
    double bestd = fabs(a - E2M1_GRID[0]);
    for (int m = 1; m < 8; ++m) {
        double d = fabs(a - E2M1_GRID[m]);
        if (d < bestd || (d == bestd && (m % 2 == 0))) { best = m; bestd = d; }
    }
    return best;
}

/* Stochastic rounding onto the E2M1 grid, [FP4T] Method: for a value between
 * two grid points the higher one is chosen with probability equal to the
 * fractional distance.  Realisation: with u16 uniform on [0, 2^16), round up
 * iff u16 < frac * 2^16 (exact comparison).  Values on a grid point and values
 * at or above 6 are not randomised (6 is the saturation cap).  a >= 0. */
int orc_e2m1_sr(double a, uint32_t u16)
{
    if (a >= 6.0) return 7;
    int lo = 0;
    for (int m = 0; m < 8; ++m) if (E2M1_GRID[m] <= a) lo = m;
    if (E2M1_GRID[lo] == a) return lo;
    double frac = (a - E2M1_GRID[lo]) / (E2M1_GRID[lo + 1] - E2M1_GRID[lo]);
    return ((double)u16 < frac * 65536.0) ? lo + 1 : lo;
}

/* Inner-scale grids.
 * E4M3 ([ALTO] Technical design: NVFP4 inner grid max 448): OCP E4M3FN, bias 7,
 *   subnormals m/8*2^-6, 0x7F is NaN, largest finite 0x7E = 448.
 * UE5M3 ([ALTO] Background/Technical design: AMD-FP4 inner grid max 114688):
 *   unsigned, 5 exponent bits, 3 mantissa bits, bias 15, subnormals
 *   m/8*2^-14, 0xFF is NaN, largest finite 0xFE = 1.75*2^16 = 114688.
 * sfmt: 1 = E4M3, 2 = UE5M3. */
double orc_scale_decode(int sfmt, int c)
{
    c &= 0xFF;
    int ebits = (sfmt == 1) ? 4 : 5;
    int bias = (sfmt == 1) ? 7 : 15;
    int maxcode = (sfmt == 1) ? 0x7E : 0xFE;
    if (c > maxcode) return NAN;
    int e = c >> 3, m = c & 7;
    (void)ebits;
    if (e == 0) return ldexp((double)m / 8.0, 1 - bias);
    return ldexp(1.0 + (double)m / 8.0, e - bias);
}

static int scale_maxcode(int sfmt) { return (sfmt == 1) ? 0x7E : 0xFE; }

/* RNE of y >= 0 onto the inner-scale grid, satfinite (anything above the
 * largest finite value encodes to it), underflow to code 0 ([FP4T]
 * Requirements: blocks below the scale range quantise to zero).  Plain
 * nearest search over every finite code; ties go to the even code. */
int orc_scale_encode(int sfmt, float y)
{
    int maxc = scale_maxcode(sfmt);
    double yd = (double)y;
    /* satfinite: above the largest finite value the code is the largest
     * finite code (stated first so the search only sees y <= max, where the
     * double differences are exact). */
    if (yd >= orc_scale_decode(sfmt, maxc)) return maxc;
    int best = 0;
    double bestd = fabs(yd - orc_scale_decode(sfmt, 0));
    for (int c = 1; c <= maxc; ++c) {
        double d = fabs(yd - orc_scale_decode(sfmt, c));
        if (d < bestd || (d == bestd && (c % 2 == 0))) { best = c; bestd = d; }
    }
    return best;
}

/* UE8M0 decode ([TEQAT] Design/Guards): code c -> 2^(c-127) for c in [0,254],
 * code 0 is 2^-127 (not flushed), code 255 is NaN. */
double orc_ue8m0_decode(int c)
{
    c &= 0xFF;
    if (c == 255) return NAN;
    return ldexp(1.0, c - 127);
}

/* ------------------------------------------------------------------------ */
/* Counter-based RNG: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel    */
/* random numbers: as easy as 1, 2, 3", SC'11).  [FP4T] Method keys the SR     */
/* draw on (seed, step, global index); the key/counter mapping is a reading.  */
/* ------------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16-bit uniform variate of element idx:
 *   key = (lo32 seed, hi32 seed), counter = (lo32(idx>>3), hi32(idx>>3),
 *   lo32 step, hi32 step); lane = idx & 7 selects 16-bit half (lane & 1) of
 *   output word (lane >> 1). */
uint32_t orc_sr_u16(uint64_t seed, uint64_t step, uint64_t idx)
{
    uint64_t blk = idx >> 3;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)step, (uint32_t)(step >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    unsigned lane = (unsigned)(idx & 7u);
    return (out[lane >> 1] >> (16u * (lane & 1u))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------ */
/* Array helpers used by the exhaustive pins                                 */
/* ------------------------------------------------------------------------ */

void orc_f32_to_bf16_array(const float* f, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(f[i]);
}

void orc_e2m1_rne_array(const float* a, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e2m1_rne((double)a[i]);
}

void orc_scale_encode_array(int sfmt, const float* y, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_scale_encode(sfmt, y[i]);
}

void orc_sr_u16_array(uint64_t seed, uint64_t step, uint64_t idx0, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint16_t)orc_sr_u16(seed, step, idx0 + (uint64_t)i);
}

void orc_div_array(const float* a, const float* b, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] / b[i];
}

/* ------------------------------------------------------------------------ */
/* NVFP4 / AMD-FP4 (per-16 E4M3 or UE5M3 inner scales, optional tensorwise   */
/* or outer-block FP32 level).                                               */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t scale_fmt;       /* 1 = E4M3 (NVFP4 default), 2 = UE5M3 (AMD-FP4, or NVFP4 scale_format="ue5m3") */
    int32_t two_level;       /* 0 none, 1 tensorwise, 2 outer block                 */
    int32_t obs;             /* outer block size (outer-block mode)                  */
    int32_t outer_2d;        /* 1: obs x obs tiles shared by both directions         */
    int32_t stochastic;      /* 0 RNE, 1 stochastic rounding                         */
    int32_t use_given_outer; /* 1: row_outer (and col_outer in 1D) are inputs        */
    int32_t inner_2d;        /* 1: 16 x 16 inner tiles share one scale               */
    uint64_t seed, step, index_base;
} orc_nv_params;

#define INNER 16

/* Outer denominator, [ALTO] Technical design: amax / (scale_max * 6) with
 * scale_max = 448 (E4M3) or 114688 (UE5M3). */
static float outer_denominator(int sfmt) { return (sfmt == 1) ? 448.0f * 6.0f : 114688.0f * 6.0f; }

/* NaN-input sanitisation ([ALTO] Op-level tests).  Reading: NaN -> +0,
 * +-inf -> +-(largest finite bf16), applied to the value being quantised. */
static float sanitize(float v)
{
    if (isnan(v)) return 0.0f;
    if (isinf(v)) return v > 0 ? f_from_bits(0x7F7F0000u) : -f_from_bits(0x7F7F0000u);
    return v;
}

/* Element e of a source held as bf16 bits or as binary32 ([FP4T] Requirements:
 * float32 or bfloat16 input; a bf16 value widens to binary32 exactly). */
static float load_x(const void* X, int x_f32, int64_t e)
{
    return x_f32 ? ((const float*)X)[e] : orc_bf16_to_f32(((const uint16_t*)X)[e]);
}

/* Store a binary32 result as bf16 (RNE) or as binary32 itself ([TEQAT]
 * Correctness: bf16 and fp32 fake-quant and dequantise targets). */
static void store_y(void* Y, int y_f32, int64_t e, float w)
{
    if (y_f32) ((float*)Y)[e] = w;
    else ((uint16_t*)Y)[e] = orc_f32_to_bf16(w);
}

/* Quantise the rows of an [R, C] fp32 matrix of normalised values vn with
 * per-16 inner blocks along each row ([FP4T] Method; [ALTO] Technical design
 * level 2 and 3).  u holds each element's SR variate (ignored for RNE).
 * Writes packed codes [R, C/2] (low nibble = even column), scale bytes
 * [R, C/16] and the signed inner-dequantised value p = +-G[m]*d (exact). */
static void quantize_rows(const float* vn, const uint16_t* u, int64_t R, int64_t C,
                          int sfmt, int stochastic, const float* tile_max,
                          uint8_t* codes, uint8_t* scales, float* p_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i) {
        for (int64_t j0 = 0; j0 < C; j0 += INNER) {
            const float* blk = vn + i * C + j0;
            /* block amax: of the 1 x 16 block, or (2D inner scaling) of the
             * 16 x 16 tile holding it */
            float b = 0.0f;
            if (tile_max) {
                b = tile_max[(i / INNER) * (C / INNER) + j0 / INNER];
            } else {
                for (int k = 0; k < INNER; ++k) {
                    float a = fabsf(blk[k]);
                    if (a > b) b = a;
                }
            }
            /* block_absmax / 6, encoded onto the scale grid; elements are then
             * divided by the DECODED scale ([FP4T] Method). */
            float y = b / 6.0f;
            int cs = orc_scale_encode(sfmt, y);
            float d = (float)orc_scale_decode(sfmt, cs);
            scales[i * (C / INNER) + j0 / INNER] = (uint8_t)cs;
            for (int k = 0; k < INNER; ++k) {
                float v = blk[k];
                float t = (d == 0.0f) ? 0.0f : fabsf(v) / d;
                int m = stochastic ? orc_e2m1_sr((double)t, u[i * C + j0 + k]) : orc_e2m1_rne((double)t);
                int s = signbit(v) ? 1 : 0;
                int code = (s << 3) | m;
                int64_t jj = j0 + k;
                uint8_t* byte = &codes[i * (C / 2) + jj / 2];
                if ((jj & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | code);
                else *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
                float p = (float)E2M1_GRID[m] * d; /* exact: <= 2 x 4 significant bits */
                p_out[i * C + jj] = s ? -p : p;
            }
        }
    }
}

/* outer scale lookup for element (i, j) of an [R, C] row-quantised matrix */
typedef struct {
    int mode;          /* 0 none, 1 tensorwise, 2 outer 1D, 3 outer 2D, 4 outer 2D transposed */
    int64_t obs;
    const float* s;
} outer_map;

static float outer_at(const outer_map* om, int64_t R, int64_t C, int64_t i, int64_t j)
{
    (void)R;
    switch (om->mode) {
    case 1: return om->s[0];
    case 2: return om->s[i * (C / om->obs) + j / om->obs];
    case 3: return om->s[(i / om->obs) * (C / om->obs) + j / om->obs];
    case 4: return om->s[(j / om->obs) * (R / om->obs) + i / om->obs];
    default: return 1.0f;
    }
}

/* Dequantise ([FP4T] API dequantize; [ALTO] Implementation convert_from):
 * w = p (no outer level) or RN(p * s_o); y = bf16(w) by RNE. */
static float dequant_value(float p, int has_outer, float so)
{
    return has_outer ? p * so : p;
}

/* Normalise by the outer scale ([ALTO] Background: each outer block is
 * normalised by its own amax/(inner_grid_max*6) before inner FP4
 * quantisation; Implementation: compute the outer scale, normalise, then run
 * the inner quantiser with tensorwise scaling disabled).
 * v_n = RN(v / s_o); a zero outer scale quantises its group to signed zero. */
static float normalize(float v, float so)
{
    if (so == 0.0f) return copysignf(0.0f, v);
    return v / so;
}

static int check_params(const orc_nv_params* p, int64_t R, int64_t C, int need_cols)
{
    if (p->scale_fmt != 1 && p->scale_fmt != 2) return -1;
    if (R < 0 || C < 0) return -2;
    if (C % INNER) return -2;
    if (need_cols && (R % INNER)) return -2;
    if (p->two_level == 2) {
        if (p->obs <= 0 || p->obs % INNER) return -3;
        if (C % p->obs) return -3;
        if ((p->outer_2d || need_cols) && (R % p->obs)) return -3;
    }
    if (p->inner_2d) {
        /* one quantisation decision per element shared by both directions:
         * a per-direction (1D) outer scale would make two */
        if (p->two_level == 2 && !p->outer_2d) return -4;
        if (R % INNER) return -2;
    }
    return 0;
}

/* Largest |vn| of every 16 x 16 tile of an [R, C] matrix ("Block-Scaled FP8
 * and FP4 Weight Quantization", section 6: a square tile shares one scale,
 * computed from all of its values). */
static void tile_maxima(const float* vn, int64_t R, int64_t C, float* tmax)
{
#pragma omp parallel for schedule(static)
    for (int64_t ti = 0; ti < R / INNER; ++ti)
        for (int64_t tj = 0; tj < C / INNER; ++tj) {
            float b = 0.0f;
            for (int64_t i = ti * INNER; i < (ti + 1) * INNER; ++i)
                for (int64_t j = tj * INNER; j < (tj + 1) * INNER; ++j) {
                    float a = fabsf(vn[i * C + j]);
                    if (a > b) b = a;
                }
            tmax[ti * (C / INNER) + tj] = b;
        }
}

/* Full NVFP4 / AMD-FP4 quantisation of X [R, C] (bf16 bits, row-major,
 * contiguous) in the rowwise direction and, if col_codes != NULL, in the
 * columnwise direction (the rowwise layout of X^T, [BSWQ] sections 1-3).
 *
 *  1. x = f32(X); with a residual Z: v = RN(x + Z)  ([FP4T] API, Method:
 *     error feedback adds the carried residual into the next quantisation);
 *     then v is sanitised (NaN -> +0, +-inf -> +-largest bf16), so a NaN x
 *     gives +0 and an infinite x or an overflowing sum the signed largest
 *     bf16 whatever the (finite) residual holds.
 *  2. outer groups ([ALTO] Technical design): tensorwise = the whole tensor;
 *     2D = obs x obs tiles shared by both directions; 1D = 1 x obs along the
 *     row for the rowwise direction and obs x 1 along the column for the
 *     columnwise direction ([BSWQ] section 4: 1D groups follow the active
 *     direction).  s_o = RN(A / (scale_max * 6)), A = max |v| of the group.
 *  3. v_n = RN(v / s_o).
 *  4. per-16 inner quantisation of v_n along the direction.
 *  5. y = bf16(RN(p * s_o)).
 *  6. residual Z' = RN(v - w_row) using the rowwise dequantised FP32 value
 *     ([FP4T] Method: residual x - dequant(quantize(x))).
 * SR draws: element (i, j) uses u16(seed, step, index_base + i*C + j) in both
 * directions.  Returns 0 or a negative error. */
static int nv_quantize_impl(const orc_nv_params* prm, const void* X, int x_f32, int64_t R, int64_t C,
                            float* residual,
                            uint8_t* row_codes, uint8_t* row_scales, float* row_outer, void* row_y,
                            uint8_t* col_codes, uint8_t* col_scales, float* col_outer, void* col_y, int y_f32)
{
    int want_cols = (col_codes != NULL);
    int rc = check_params(prm, R, C, want_cols);
    if (rc) return rc;
    const int64_t N = R * C;
    const int sfmt = prm->scale_fmt;
    const float D = outer_denominator(sfmt);
    const int64_t obs = prm->obs;

    float* v = (float*)malloc(sizeof(float) * (size_t)(N ? N : 1));
    uint16_t* u = (uint16_t*)calloc((size_t)(N ? N : 1), sizeof(uint16_t));
    float* vn_r = (float*)malloc(sizeof(float) * (size_t)(N ? N : 1));
    float* p_r = (float*)malloc(sizeof(float) * (size_t)(N ? N : 1));
    uint8_t* rc_codes = row_codes ? row_codes : (uint8_t*)malloc((size_t)(N / 2 + 1));
    uint8_t* rc_scales = row_scales ? row_scales : (uint8_t*)malloc((size_t)(N / INNER + 1));

    /* step 1 */
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < N; ++e) {
        float x = load_x(X, x_f32, e);
        float ve = residual ? x + residual[e] : x;
        v[e] = sanitize(ve);
    }
    if (prm->stochastic) {
#pragma omp parallel for schedule(static)
        for (int64_t e = 0; e < N; ++e) u[e] = (uint16_t)orc_sr_u16(prm->seed, prm->step, prm->index_base + (uint64_t)e);
    }

    /* step 2: outer scales */
    outer_map om_r = {0, obs, NULL}, om_c = {0, obs, NULL};
    float* so_row = NULL;
    float* so_col = NULL;
    float tensor_scale = 0.0f;
    if (prm->two_level == 1) {
        if (prm->use_given_outer) tensor_scale = row_outer[0];
        else {
            float A = 0.0f;
            for (int64_t e = 0; e < N; ++e) { float a = fabsf(v[e]); if (a > A) A = a; }
            tensor_scale = A / D;
            if (row_outer) row_outer[0] = tensor_scale;
            if (col_outer) col_outer[0] = tensor_scale;
        }
        so_row = &tensor_scale;
        om_r.mode = 1; om_r.s = so_row;
        om_c = om_r;
    } else if (prm->two_level == 2 && prm->outer_2d) {
        int64_t TR = R / obs, TC = C / obs;
        so_row = (float*)malloc(sizeof(float) * (size_t)(TR * TC + 1));
        if (prm->use_given_outer) memcpy(so_row, row_outer, sizeof(float) * (size_t)(TR * TC));
        else {
            for (int64_t ti = 0; ti < TR; ++ti)
                for (int64_t tj = 0; tj < TC; ++tj) {
                    float A = 0.0f;
                    for (int64_t i = ti * obs; i < (ti + 1) * obs; ++i)
                        for (int64_t j = tj * obs; j < (tj + 1) * obs; ++j) {
                            float a = fabsf(v[i * C + j]); if (a > A) A = a;
                        }
                    so_row[ti * TC + tj] = A / D;
                }
            if (row_outer) memcpy(row_outer, so_row, sizeof(float) * (size_t)(TR * TC));
            if (col_outer) memcpy(col_outer, so_row, sizeof(float) * (size_t)(TR * TC));
        }
        om_r.mode = 3; om_r.s = so_row;
        om_c.mode = 4; om_c.s = so_row;   /* the columnwise matrix is [C, R]: tile index transposed */
    } else if (prm->two_level == 2) {
        /* 1D: rowwise groups 1 x obs -> [R, C/obs]; columnwise groups obs x 1 -> [C, R/obs] */
        so_row = (float*)malloc(sizeof(float) * (size_t)(R * (C / obs) + 1));
        if (prm->use_given_outer) memcpy(so_row, row_outer, sizeof(float) * (size_t)(R * (C / obs)));
        else {
            for (int64_t i = 0; i < R; ++i)
                for (int64_t g = 0; g < C / obs; ++g) {
                    float A = 0.0f;
                    for (int64_t j = g * obs; j < (g + 1) * obs; ++j) { float a = fabsf(v[i * C + j]); if (a > A) A = a; }
                    so_row[i * (C / obs) + g] = A / D;
                }
            if (row_outer) memcpy(row_outer, so_row, sizeof(float) * (size_t)(R * (C / obs)));
        }
        om_r.mode = 2; om_r.s = so_row;
        if (want_cols) {
            so_col = (float*)malloc(sizeof(float) * (size_t)(C * (R / obs) + 1));
            if (prm->use_given_outer) memcpy(so_col, col_outer, sizeof(float) * (size_t)(C * (R / obs)));
            else {
                for (int64_t j = 0; j < C; ++j)
                    for (int64_t g = 0; g < R / obs; ++g) {
                        float A = 0.0f;
                        for (int64_t i = g * obs; i < (g + 1) * obs; ++i) { float a = fabsf(v[i * C + j]); if (a > A) A = a; }
                        so_col[j * (R / obs) + g] = A / D;
                    }
                if (col_outer) memcpy(col_outer, so_col, sizeof(float) * (size_t)(C * (R / obs)));
            }
            om_c.mode = 2; om_c.s = so_col;
        }
    }
    const int has_outer = (om_r.mode != 0);

    /* step 3 + 4, rowwise */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j)
            vn_r[i * C + j] = has_outer ? normalize(v[i * C + j], outer_at(&om_r, R, C, i, j)) : v[i * C + j];
    if (N) memset(rc_codes, 0, (size_t)(N / 2));
    float* tmax = NULL;
    if (prm->inner_2d) {
        tmax = (float*)malloc(sizeof(float) * (size_t)((R / INNER) * (C / INNER) + 1));
        tile_maxima(vn_r, R, C, tmax);
    }
    quantize_rows(vn_r, u, R, C, sfmt, prm->stochastic, tmax, rc_codes, rc_scales, p_r);

    /* step 5 + 6, rowwise */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            float so = has_outer ? outer_at(&om_r, R, C, i, j) : 1.0f;
            float w = dequant_value(p_r[i * C + j], has_outer, so);
            if (row_y) store_y(row_y, y_f32, i * C + j, w);
            if (residual) residual[i * C + j] = v[i * C + j] - w;
        }

    /* columnwise with 2D inner scaling: the transpose of the rowwise result
     * ([BSWQ] section 6: the scale moves with the tile, so the columnwise
     * codes and scales follow by transposition, with no second decision) */
    if (want_cols && prm->inner_2d) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < C; ++j)
            for (int64_t i = 0; i < R; ++i) {
                const uint8_t rb = rc_codes[i * (C / 2) + j / 2];
                const int code = (j & 1) ? (rb >> 4) : (rb & 0x0F);
                uint8_t* byte = &col_codes[j * (R / 2) + i / 2];
                if ((i & 1) == 0) *byte = (uint8_t)((*byte & 0xF0) | code);
                else *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
                if (i % INNER == 0) col_scales[j * (R / INNER) + i / INNER] = rc_scales[i * (C / INNER) + j / INNER];
                if (col_y) {
                    float so = has_outer ? outer_at(&om_r, R, C, i, j) : 1.0f;
                    store_y(col_y, y_f32, j * R + i, dequant_value(p_r[i * C + j], has_outer, so));
                }
            }
    }

    /* columnwise: quantise the rows of the transpose, [BSWQ] sections 2-4 */
    if (want_cols && !prm->inner_2d) {
        float* vT = (float*)malloc(sizeof(float) * (size_t)(N ? N : 1));
        uint16_t* uT = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N ? N : 1));
        float* pT = (float*)malloc(sizeof(float) * (size_t)(N ? N : 1));
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < C; ++j)
            for (int64_t i = 0; i < R; ++i) {
                float vv = v[i * C + j];
                /* element (j, i) of X^T, whose outer group is looked up in the [C, R] frame */
                vT[j * R + i] = has_outer ? normalize(vv, outer_at(&om_c, C, R, j, i)) : vv;
                uT[j * R + i] = u[i * C + j];
            }
        if (N) memset(col_codes, 0, (size_t)(N / 2));
        quantize_rows(vT, uT, C, R, sfmt, prm->stochastic, NULL, col_codes, col_scales, pT);
        if (col_y) {
#pragma omp parallel for schedule(static)
            for (int64_t j = 0; j < C; ++j)
                for (int64_t i = 0; i < R; ++i) {
                    float so = has_outer ? outer_at(&om_c, C, R, j, i) : 1.0f;
                    store_y(col_y, y_f32, j * R + i, dequant_value(pT[j * R + i], has_outer, so));
                }
        }
        free(vT); free(uT); free(pT);
    }

    free(tmax);
    if (so_row && so_row != &tensor_scale) free(so_row);
    if (so_col) free(so_col);
    if (!row_codes) free(rc_codes);
    if (!row_scales) free(rc_scales);
    free(v); free(u); free(vn_r); free(p_r);
    return 0;
}

int orc_nv_quantize(const orc_nv_params* prm, const uint16_t* X, int64_t R, int64_t C,
                    float* residual,
                    uint8_t* row_codes, uint8_t* row_scales, float* row_outer, uint16_t* row_y,
                    uint8_t* col_codes, uint8_t* col_scales, float* col_outer, uint16_t* col_y)
{
    return nv_quantize_impl(prm, X, 0, R, C, residual, row_codes, row_scales, row_outer, row_y,
                            col_codes, col_scales, col_outer, col_y, 0);
}

/* The same with the source's and the outputs' dtypes chosen: x_f32 = 1 reads
 * X as binary32, y_f32 = 1 writes the dequantised outputs as binary32 (the
 * FP32 value w itself, no bf16 rounding). */
int orc_nv_quantize_ex(const orc_nv_params* prm, const void* X, int x_f32, int64_t R, int64_t C,
                       float* residual,
                       uint8_t* row_codes, uint8_t* row_scales, float* row_outer, void* row_y,
                       uint8_t* col_codes, uint8_t* col_scales, float* col_outer, void* col_y, int y_f32)
{
    return nv_quantize_impl(prm, X, x_f32, R, C, residual, row_codes, row_scales, row_outer, row_y,
                            col_codes, col_scales, col_outer, col_y, y_f32);
}

/* Grouped (per-expert) quantisation ([ALTO] Implementation: grouped MoE GEMM
 * with a per-expert outer scale): G independent calls on stacked buffers; the
 * SR index of group g starts at index_base + (rows before g) * C. */
int orc_nv_quantize_grouped(const orc_nv_params* prm, int32_t G, const int64_t* rows, int64_t C,
                            const uint16_t* X, float* residual,
                            uint8_t* row_codes, uint8_t* row_scales, float* row_outer,
                            uint8_t* col_codes, uint8_t* col_scales, float* col_outer)
{
    int64_t r0 = 0, outer_r_off = 0, outer_c_off = 0;
    for (int32_t g = 0; g < G; ++g) {
        int64_t R = rows[g];
        orc_nv_params p = *prm;
        p.index_base = prm->index_base + (uint64_t)(r0 * C);
        int64_t n_outer_r = 0, n_outer_c = 0;
        if (p.two_level == 1) { n_outer_r = 1; n_outer_c = 1; }
        else if (p.two_level == 2 && p.outer_2d) { n_outer_r = (R / p.obs) * (C / p.obs); n_outer_c = n_outer_r; }
        else if (p.two_level == 2) { n_outer_r = R * (C / p.obs); n_outer_c = C * (R / p.obs); }
        int rc = orc_nv_quantize(&p, X + r0 * C, R, C, residual ? residual + r0 * C : NULL,
                                 row_codes + r0 * C / 2, row_scales + r0 * C / INNER,
                                 row_outer ? row_outer + outer_r_off : NULL, NULL,
                                 col_codes ? col_codes + r0 * C / 2 : NULL,
                                 col_scales ? col_scales + r0 * C / INNER : NULL,
                                 (col_outer && p.two_level == 2 && !p.outer_2d) ? col_outer + outer_c_off : NULL,
                                 NULL);
        if (rc) return rc;
        r0 += R;
        outer_r_off += n_outer_r;
        outer_c_off += n_outer_c;
    }
    return 0;
}

/* Dequantise stored NVFP4 / AMD-FP4 buffers of a logical [R, C] matrix:
 * y = bf16(RN(+-G[m] * dec(s_i) * s_o)) with the inner product exact (with
 * y_f32 the binary32 value itself).
 * outer_kind: 0 none, 1 tensorwise, 2 1D [R, C/obs], 3 2D [R/obs, C/obs],
 * 4 2D stored transposed [C/obs, R/obs] (the shared tile scale read from the
 * columnwise buffer's frame). */
int orc_nv_dequantize_ex(int sfmt, int outer_kind, int64_t obs,
                         const uint8_t* codes, const uint8_t* scales, const float* outer,
                         int64_t R, int64_t C, void* y, int y_f32)
{
    if (C % INNER) return -2;
    outer_map om = {outer_kind, obs, outer};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint8_t byte = codes[i * (C / 2) + j / 2];
            int code = (j & 1) ? (byte >> 4) : (byte & 0xF);
            float d = (float)orc_scale_decode(sfmt, scales[i * (C / INNER) + j / INNER]);
            float p = (float)E2M1_GRID[code & 7] * d;
            float w = (outer_kind != 0) ? p * outer_at(&om, R, C, i, j) : p;
            if (code & 8) w = -w;
            store_y(y, y_f32, i * C + j, w);
        }
    return 0;
}

int orc_nv_dequantize(int sfmt, int outer_kind, int64_t obs,
                      const uint8_t* codes, const uint8_t* scales, const float* outer,
                      int64_t R, int64_t C, uint16_t* y)
{
    return orc_nv_dequantize_ex(sfmt, outer_kind, obs, codes, scales, outer, R, C, y, 0);
}

/* ------------------------------------------------------------------------ */
/* MXFP4: 1x32 blocks, UE8M0 power-of-two scale, E2M1 RNE ([TEQAT] Overview,  */
/* Design, Correctness, Known limitations).                                  */
/* ------------------------------------------------------------------------ */

#define MXB 32

/* Scale exponent of one block.  Reading of "integer-bit amax/exponent
 * derivation" with floor 2^-126 and cap 2^125: k is the smallest integer with
 * 6 * 2^k >= amax (= ceil(log2(amax/6)), so the block maximum lands at or
 * below the E2M1 maximum 6), then clamped to [-126, 125]; amax == 0 gives the
 * floor.  Exact comparisons in double. */
static int mx_exponent(double amax)
{
    if (amax == 0.0) return -126;
    int k = -200;
    while (ldexp(6.0, k) < amax) ++k;
    if (k < -126) k = -126;
    if (k > 125) k = 125;
    return k;
}

/* MXFP4 fake-quant of X [R, C] (bf16 bits, or binary32 with x_f32): codes
 * [R, C/2], scale bytes [R, C/32], y [R, C] as bf16 (or binary32 with y_f32).
 * A block holding any NaN or +-inf is poisoned ([TEQAT] Correctness: inf/NaN
 * block poisoning): scale byte 0xFF (the NaN code), codes 0, every y the quiet
 * NaN (0x7FC0, or 0x7FC00000 as binary32).  Otherwise t = |x| * 2^-k (exact),
 * m = RNE(t) saturating at 6, sign kept (also for zero), y = +-G[m] * 2^k,
 * which bf16 represents exactly ([TEQAT] Design). */
int orc_mx_qdq_ex(const void* X, int x_f32, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales, void* y,
                  int y_f32)
{
    if (C % MXB) return -2;
    const int64_t nb = R * (C / MXB);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; ++b) {
        int poisoned = 0;
        double A = 0.0;
        for (int k = 0; k < MXB; ++k) {
            float f = load_x(X, x_f32, b * MXB + k);
            if (isnan(f) || isinf(f)) poisoned = 1;
            else if (fabs((double)f) > A) A = fabs((double)f);
        }
        uint8_t* cb = codes ? codes + b * (MXB / 2) : NULL;
        if (poisoned) {
            if (scales) scales[b] = 0xFF;
            for (int k = 0; k < MXB; ++k) {
                if (cb && (k & 1) == 0) cb[k / 2] = 0;
                if (y) store_y(y, y_f32, b * MXB + k, f_from_bits(0x7FC00000u));
            }
            continue;
        }
        int e = mx_exponent(A);
        if (scales) scales[b] = (uint8_t)(e + 127);
        for (int k = 0; k < MXB; ++k) {
            float f = load_x(X, x_f32, b * MXB + k);
            double t = fabs((double)f) * ldexp(1.0, -e);
            int m = orc_e2m1_rne(t);
            int s = signbit(f) ? 1 : 0;
            int code = (s << 3) | m;
            if (cb) {
                if ((k & 1) == 0) cb[k / 2] = (uint8_t)code;
                else cb[k / 2] = (uint8_t)(cb[k / 2] | (code << 4));
            }
            if (y) {
                double w = E2M1_GRID[m] * ldexp(1.0, e);
                float wf = (float)(s ? -w : w);
                store_y(y, y_f32, b * MXB + k, wf);
            }
        }
    }
    return 0;
}

int orc_mx_qdq(const uint16_t* X, int64_t R, int64_t C, uint8_t* codes, uint8_t* scales, uint16_t* y)
{
    return orc_mx_qdq_ex(X, 0, R, C, codes, scales, y, 0);
}

/* MXFP4 dequantise from stored codes and UE8M0 scales: y = +-G[m] * 2^(c-127)
 * as bf16 (or binary32 with y_f32); scale byte 0xFF (NaN) gives the quiet NaN. */
int orc_mx_dequantize_ex(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C, void* y, int y_f32)
{
    if (C % MXB) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R; ++i)
        for (int64_t j = 0; j < C; ++j) {
            uint8_t byte = codes[i * (C / 2) + j / 2];
            int code = (j & 1) ? (byte >> 4) : (byte & 0xF);
            int sc = scales[i * (C / MXB) + j / MXB];
            if (sc == 255) { store_y(y, y_f32, i * C + j, f_from_bits(0x7FC00000u)); continue; }
            double w = E2M1_GRID[code & 7] * orc_ue8m0_decode(sc);
            float wf = (float)((code & 8) ? -w : w);
            store_y(y, y_f32, i * C + j, wf);
        }
    return 0;
}

int orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t R, int64_t C, uint16_t* y)
{
    return orc_mx_dequantize_ex(codes, scales, R, C, y, 0);
}

/* ------------------------------------------------------------------------ */
/* FP8 re-encodings of the MXFP4 projection ([TEQAT] Overview, Design,       */
/* Correctness: the projected weight goes to the MXFP8 (1x32 UE8M0 scale,    */
/* E4M3 payload) and Float8 128x128 block-scaling hosts; the rowwise MXFP8   */
/* encoding is bitwise lossless, the 128x128 encoding is lossless within a   */
/* tile's E4M3 headroom, the columnwise 32x1 encoding is a bounded           */
/* re-quantisation).                                                         */
/* ------------------------------------------------------------------------ */

/* E4M3 (OCP E4M3FN) payload byte of v: RNE onto the finite grid with
 * subnormals (orc_scale_encode on |v|), sign bit 0x80 kept also for zero.
 * NaN encodes as 0xFF (an E4M3FN NaN; reading: the pages fix no NaN payload).
 * Above 448 the code saturates to 0x7E (never reached below: every encoding
 * here keeps |v| <= 384). */
static uint8_t e4m3_payload(double v)
{
    if (isnan(v)) return 0xFF;
    const uint8_t s = signbit(v) ? 0x80 : 0x00;
    return (uint8_t)(s | (uint8_t)orc_scale_encode(1, (float)fabs(v)));
}

uint8_t orc_e4m3_payload(double v) { return e4m3_payload(v); }

/* MXFP8 shared exponent of a block (OCP Microscaling formats v1.0: the scale
 * is 2^(floor(log2(amax)) - emax) with emax = 8 for E4M3), clamped to the
 * UE8M0 range [-127, 127]; a block with no nonzero finite element takes -127
 * (code 0).  Reading: amax is over the finite elements. */
static int mx8_exponent(double amax)
{
    if (!(amax > 0.0)) return -127;
    int e;
    (void)frexp(amax, &e);          /* amax = f * 2^e, f in [0.5, 1) */
    int E = (e - 1) - 8;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    return E;
}

/* Power-of-two scale exponent of a 128 x 128 block: the smallest e with
 * amax <= 448 * 2^e (reading of "lossless within each tile's E4M3 headroom":
 * a power-of-two scale keeps the E4M3 payload grid exact down to 2^14 below
 * the tile maximum); amax == 0 (no nonzero finite element) gives e = 0. */
static int blk_exponent(double amax)
{
    if (!(amax > 0.0)) return 0;
    int e = -300;
    while (amax > ldexp(448.0, e)) ++e;
    return e;
}

#define F8BLK 128

/* MXFP4 projection of X [R, C] (bf16 bits) and its FP8 re-encodings, every
 * output optional (NULL skips it):
 *   y        bf16 [R, C]        the projection (orc_mx_qdq)
 *   mx8_row  E4M3 [R, C], mx8_row_sc UE8M0 [R, C/32]: 1 x 32 blocks of y along rows
 *   mx8_col  E4M3 [C, R], mx8_col_sc UE8M0 [C, R/32]: 32 x 1 blocks of y down the
 *            columns, stored as the rowwise layout of y^T
 *   blk      E4M3 [R, C], blk_t E4M3 [C, R] (its transpose), blk_sc FP32
 *            [R/128, C/128]: 128 x 128 blocks with a power-of-two scale
 * Payload = e4m3(y / scale) with the scale of the element's block. */
int orc_mx_project_encode(const uint16_t* X, int64_t R, int64_t C, uint16_t* y_out,
                          uint8_t* mx8_row, uint8_t* mx8_row_sc, uint8_t* mx8_col, uint8_t* mx8_col_sc,
                          uint8_t* blk, uint8_t* blk_t, float* blk_sc)
{
    if (R < 0 || C < 0 || C % MXB) return -2;
    if ((mx8_col || mx8_col_sc) && R % MXB) return -2;
    if ((blk || blk_t || blk_sc) && (R % F8BLK || C % F8BLK)) return -2;
    const int64_t N = R * C;
    uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N ? N : 1));
    orc_mx_qdq(X, R, C, NULL, NULL, y);
    if (y_out) memcpy(y_out, y, sizeof(uint16_t) * (size_t)N);

    /* rowwise MXFP8: the 1 x 32 blocks of y along each row */
    if (mx8_row || mx8_row_sc) {
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < R * (C / MXB); ++b) {
            const uint16_t* yb = y + b * MXB;
            double A = 0.0;
            for (int k = 0; k < MXB; ++k) {
                double v = (double)orc_bf16_to_f32(yb[k]);
                if (!isnan(v) && fabs(v) > A) A = fabs(v);
            }
            const int E = mx8_exponent(A);
            if (mx8_row_sc) mx8_row_sc[b] = (uint8_t)(E + 127);
            if (mx8_row)
                for (int k = 0; k < MXB; ++k)
                    mx8_row[b * MXB + k] = e4m3_payload((double)orc_bf16_to_f32(yb[k]) * ldexp(1.0, -E));
        }
    }

    /* columnwise MXFP8: 32 x 1 blocks down each column, i.e. the rowwise
     * encoding of y^T */
    if (mx8_col || mx8_col_sc) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < C; ++j)
            for (int64_t g = 0; g < R / MXB; ++g) {
                double A = 0.0;
                for (int64_t i = g * MXB; i < (g + 1) * MXB; ++i) {
                    double v = (double)orc_bf16_to_f32(y[i * C + j]);
                    if (!isnan(v) && fabs(v) > A) A = fabs(v);
                }
                const int E = mx8_exponent(A);
                if (mx8_col_sc) mx8_col_sc[j * (R / MXB) + g] = (uint8_t)(E + 127);
                if (mx8_col)
                    for (int64_t i = g * MXB; i < (g + 1) * MXB; ++i)
                        mx8_col[j * R + i] = e4m3_payload((double)orc_bf16_to_f32(y[i * C + j]) * ldexp(1.0, -E));
            }
    }

    /* 128 x 128 blocks with one power-of-two FP32 scale each; blk_t is the
     * same payload transposed (a square block is transpose-consistent) */
    if (blk || blk_t || blk_sc) {
        const int64_t TR = R / F8BLK, TC = C / F8BLK;
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < TR * TC; ++t) {
            const int64_t ti = t / TC, tj = t % TC;
            double A = 0.0;
            for (int64_t i = ti * F8BLK; i < (ti + 1) * F8BLK; ++i)
                for (int64_t j = tj * F8BLK; j < (tj + 1) * F8BLK; ++j) {
                    double v = (double)orc_bf16_to_f32(y[i * C + j]);
                    if (!isnan(v) && fabs(v) > A) A = fabs(v);
                }
            const int e = blk_exponent(A);
            if (blk_sc) blk_sc[t] = (float)ldexp(1.0, e);
            for (int64_t i = ti * F8BLK; i < (ti + 1) * F8BLK; ++i)
                for (int64_t j = tj * F8BLK; j < (tj + 1) * F8BLK; ++j) {
                    const uint8_t p = e4m3_payload((double)orc_bf16_to_f32(y[i * C + j]) * ldexp(1.0, -e));
                    if (blk) blk[i * C + j] = p;
                    if (blk_t) blk_t[j * R + i] = p;
                }
        }
    }
    free(y);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FP4 GEMM consumer: C = A . B^T with MXFP4 operands ("fp4-train" README,   */
/* API: fp4_mm(a, b) is a @ b^T on FP4 operands; Correctness: the FP4 GEMM   */
/* equals the dequantise-then-multiply path).                                */
/* ------------------------------------------------------------------------ */

/* Value of element (i, k) of an MXFP4 operand stored as rowwise codes
 * [rows, K/2] and UE8M0 scale bytes [rows, K/32]: +-G[m] * 2^(s-127), NaN for
 * scale byte 0xFF. */
static double mx_operand(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t i, int64_t k)
{
    const uint8_t byte = codes[i * (K / 2) + k / 2];
    const int code = (k & 1) ? (byte >> 4) : (byte & 0xF);
    const int sc = scales[i * (K / MXB) + k / MXB];
    if (sc == 255) return NAN;
    const double v = E2M1_GRID[code & 7] * orc_ue8m0_decode(sc);
    return (code & 8) ? -v : v;
}

/* c[i, j] = sum_k a(i, k) * b(j, k) and s[i, j] = sum_k |a(i, k) * b(j, k)|,
 * both in binary64, k ascending (each product is exact in binary64).  The
 * absolute sum bounds the rounding error of any binary32 evaluation order. */
int orc_mx_mm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
              int64_t M, int64_t N, int64_t K, double* c, double* s)
{
    if (K % MXB || M < 0 || N < 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = mx_operand(a_codes, a_scales, K, i, k) * mx_operand(b_codes, b_scales, K, j, k);
                acc += p;
                mag += fabs(p);
            }
            c[i * N + j] = acc;
            if (s) s[i * N + j] = mag;
        }
    return 0;
}
