/* CPU check of the two-term reciprocal quotients the quantisation kernels use
 * for the inner (per-16) scale.  Test infrastructure: built and run by
 * tests/test_inner_quotient_identity.py.
 *
 * An inner scale d = D 2^E has D in 8..15, so its reciprocal is taken as
 * Kh + Kl with Kh = RD32(1/D) 2^-E and Kl = RN32(1/D - RD32(1/D)) 2^-E (the
 * kernels' table per scale code).  Two identities are checked for every scale
 * code of E4M3 (bias 7) and UE5M3 (bias 15):
 *   RNE   fma(v, Kh, RN32(v Kl)) == RN32(v / d) as binary32, sign included,
 *         wherever |v / d| >= 2^-100; below that (the low term v Kl is then
 *         subnormal and the last bits may differ) both quotients are far below
 *         0.25, so the E2M1 code is 0 with v's sign either way, which is checked;
 *   SR    ceil(fma(|v|, Kh 2^23, fma(|v|, Kl 2^23, -2^-127))) ==
 *         ceil(RN32(|v| RN64(1/d) 2^23) - 2^-127), also with the clamp to
 *         [0, 6 2^23] (resp. [2^-127, 6 2^23]) of the no-outer-scale case.
 * The reference quotient RN32(v / d) is computed as a binary64 division
 * rounded to binary32; that double rounding is exact here because v / d lies
 * at least 2^-29 (relative) away from every binary32 rounding midpoint.
 *
 * Values: log-uniform |v / d| over 2^-160 .. 2^8 with random significands,
 * every binary32 within 2048 ulps of random points t in [0, 6) times d, every
 * binary32 within 4096 ulps of 2^-150 d, and the first 2e5 binary32 patterns
 * (zero and the subnormals).  argv[1] scales the random counts (default 1).
 * Prints the number of cases and of mismatches; exits 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float decode(int bias, uint32_t c)
{
    uint32_t e = c >> 3, m = c & 7u;
    if (e == 0) return (float)m * ldexpf(1.0f, 1 - bias - 3);
    return ldexpf(1.0f + (float)m / 8.0f, (int)e - bias);
}

/* RD32(1/D) and RN32(1/D - RD32(1/D)) for D = 8..15 */
static const float kh[8] = {0x1p-3f, 0x1.c71c7p-4f, 0x1.999998p-4f, 0x1.745d16p-4f,
                            0x1.555554p-4f, 0x1.3b13bp-4f, 0x1.249248p-4f, 0x1.11111p-4f};
static const float kl[8] = {0.0f, 0x1.c71c72p-28f, 0x1.99999ap-28f, 0x1.45d174p-28f,
                            0x1.555556p-28f, 0x1.3b13b2p-28f, 0x1.24924ap-28f, 0x1.111112p-28f};

static uint64_t state = 88172645463325252ull;
static uint64_t next(void) { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return state; }

static long cases = 0, bad = 0;

static void check(int bias, uint32_t code, float d, float Kh, float Kl, float v)
{
    /* RNE: the binary32 quotient itself */
    const float t_ref = (float)((double)v / (double)d);
    const float t_two = fmaf(v, Kh, v * Kl);
    /* SR: the fixed-point input of the stochastic-rounding convert, plain and clamped */
    const double rd23 = (1.0 / (double)d) * 0x1p23;
    const float T = (float)((double)v * rd23);
    const float av = fabsf(v);
    const float T2 = fmaf(av, Kh * 0x1p23f, fmaf(av, Kl * 0x1p23f, -0x1p-127f));
    const float c_ref = ceilf(fabsf(T) - 0x1p-127f), c_two = ceilf(T2);
    const float cc_ref = ceilf(fminf(fmaxf(fabsf(T), 0x1p-127f), 0x1.8p25f) - 0x1p-127f);
    const float cc_two = ceilf(fminf(fmaxf(T2, 0.0f), 0x1.8p25f));
    cases++;
    const int rne_ok = fabsf(t_ref) >= 0x1p-100f ? f2u(t_ref) == f2u(t_two)
                                                 : fabsf(t_two) < 0.25f && signbit(t_two) == signbit(v);
    if (!rne_ok || !(c_ref == c_two) || !(cc_ref == cc_two)) {
        if (bad < 10)
            printf("bias %d code 0x%02x v %a: t %a / %a, c %a / %a, clamped %a / %a\n", bias, code, v, t_ref, t_two,
                   c_ref, c_two, cc_ref, cc_two);
        bad++;
    }
}

int main(int argc, char** argv)
{
    const double scale = argc > 1 ? atof(argv[1]) : 1.0;
    const int n_random = (int)(400000 * scale), n_points = (int)(60 * scale);
    for (int bias = 7; bias <= 15; bias += 8) {
        const uint32_t max_code = bias == 7 ? 0x7Eu : 0xFEu;
        for (uint32_t code = 1; code <= max_code; ++code) {
            const float d = decode(bias, code);
            const uint32_t bd = f2u(d);
            const int m = (int)((bd >> 20) & 7u), e = (int)(bd >> 23) - 127 - 3;
            const float Kh = ldexpf(kh[m], -e), Kl = ldexpf(kl[m], -e);
            for (int i = 0; i < n_random; ++i) {
                const double lt = -160.0 + (double)(next() % 1000000) * (168.0 / 1000000.0);
                float v = (float)(ldexp(1.0 + (double)(next() % (1u << 30)) / (double)(1u << 30), (int)floor(lt)) * d);
                if (next() & 1) v = -v;
                check(bias, code, d, Kh, Kl, v);
            }
            for (int k = 0; k < n_points; ++k) {
                const uint32_t u0 = f2u((float)((double)(next() % 6000000) / 1e6 * d));
                for (int j = -2048; j <= 2048; ++j) check(bias, code, d, Kh, Kl, u2f(u0 + (uint32_t)j));
            }
            const uint32_t ut = f2u((float)(0x1p-150 * (double)d));
            for (int j = -4096; j <= 4096; ++j)
                if ((int64_t)ut + j >= 0) check(bias, code, d, Kh, Kl, u2f(ut + (uint32_t)j));
            for (uint32_t u = 0; u < 200000; ++u) check(bias, code, d, Kh, Kl, u2f(u));
        }
    }
    printf("cases %ld mismatches %ld\n", cases, bad);
    return bad != 0;
}
