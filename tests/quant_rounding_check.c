/* Exhaustive host check of the divide-free rounding used by the W4A8
 * activation quantiser (QQQ PR "Support W4A8 quantization for vllm", the
 * per-token dynamic quantisation: q = clamp(rint(x / s), -128, 127) with
 * s = amax / 127 in fp16).
 *
 * The kernel replaces the divide by q0 = rint(x * r), r ~ 1/s, then takes the
 * residual d = fma(-q0, s, x) and, on an exact tie |d| == s/2 with q0 odd,
 * moves q0 one step towards d.  For every positive s the quantiser can produce
 * (s = fp16(amax / 127) for a finite fp16 amax) and every finite fp16 x with
 * |x| <= the largest amax giving that s, this program checks that the result
 * equals clamp(rint(x / s)) for each reciprocal r within +-KMAX ulps of the
 * correctly rounded 1/s (the hardware reciprocal is within one ulp).
 *
 * usage: quant_rounding_check SLICE NSLICES KMAX   (exit status 0 = no mismatch)
 * Test infrastructure; it shares nothing with the kernels. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

static float h2f(uint16_t h) {
    const uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0) v = ldexpf((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(m | 1024), (int)e - 25);
    return s ? -v : v;
}

/* fp32 -> fp16 bits, round to nearest even (finite positive inputs only) */
static uint16_t f2h(float f) {
    uint16_t best = 0;
    double bestd = INFINITY;
    /* binary search on the monotone positive fp16 range, then pick the nearest (ties to even) */
    uint32_t lo = 0, hi = 0x7C00;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (h2f((uint16_t)mid) <= f) lo = mid; else hi = mid;
    }
    for (uint32_t c = lo; c <= hi && c < 0x7C00; ++c) {
        const double d = fabs((double)h2f((uint16_t)c) - (double)f);
        if (d < bestd || (d == bestd && (c & 1) == 0)) { bestd = d; best = (uint16_t)c; }
    }
    return best;
}

static float clampq(float r) { return fminf(fmaxf(r, -128.0f), 127.0f); }

int main(int argc, char **argv) {
    if (argc != 4) { fprintf(stderr, "usage: %s SLICE NSLICES KMAX\n", argv[0]); return 2; }
    const int slice = atoi(argv[1]), nslices = atoi(argv[2]), kmax = atoi(argv[3]);
    static float amax_of_s[65536];
    static unsigned char reach[65536];
    for (uint32_t a = 1; a < 0x7C00; ++a) {
        const float af = h2f((uint16_t)a);
        const uint16_t sb = f2h(af / 127.0f);
        if (h2f(sb) == 0.0f) continue;
        reach[sb] = 1;
        if (af > amax_of_s[sb]) amax_of_s[sb] = af;
    }
    long long checked = 0, bad = 0, ties = 0;
    for (uint32_t sb = 1; sb < 0x7C00; ++sb) {
        if (!reach[sb] || (int)(sb % (uint32_t)nslices) != slice) continue;
        const float s = h2f((uint16_t)sb), hs = 0.5f * s, lim = amax_of_s[sb];
        const float r0 = 1.0f / s;
        for (int k = -kmax; k <= kmax; ++k) {
            float r = r0;
            for (int t = 0; t < abs(k); ++t) r = nextafterf(r, k < 0 ? 0.0f : INFINITY);
            for (uint32_t xb = 0; xb < 0x10000; ++xb) {
                if ((xb & 0x7FFF) >= 0x7C00) continue;
                const float x = h2f((uint16_t)xb);
                if (fabsf(x) > lim) continue;
                const float ref = clampq(rintf(x / s));
                float q0 = rintf(x * r);
                const float d = fmaf(-q0, s, x);
                if (fabsf(d) == hs) {
                    ties += (k == 0);
                    if (fmodf(q0, 2.0f) != 0.0f) q0 += d > 0 ? 1.0f : -1.0f;
                }
                const float got = clampq(q0);
                ++checked;
                if (got != ref) {
                    if (bad < 5) printf("mismatch s=%a x=%a r=%a ref=%g got=%g\n", s, x, r, ref, got);
                    ++bad;
                }
            }
        }
    }
    printf("slice %d/%d: %lld pairs, %lld ties, %lld mismatches\n", slice, nslices, checked, ties, bad);
    return bad != 0;
}
