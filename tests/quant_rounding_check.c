/* Exhaustive host check of the divide-free rounding used by the W4A8
 * activation quantiser (QQQ PR "Support W4A8 quantization for vllm", the
 * per-token dynamic quantisation: q = clamp(rint(x / s), -128, 127) with
 * s = amax / 127 in fp16).
 *
 * The kernel replaces the divide by one of two divide-free forms, r ~ 1/s:
 *  mode 0 (residual): q0 = rint(x * r), d = fma(-q0, s, x), and on an exact
 *    tie |d| == s/2 with q0 odd, q0 moves one step towards d;
 *  mode 1 (snap): t = fma(x, r, 1536) - 1536, which rounds x * r to a multiple
 *    of 2^-13 (the fp32 spacing in [1024, 2048)), then q0 = rint(t).  An exact
 *    quotient of two fp16 values is a half-integer or at least 2^-12 from one,
 *    and |x * r - x / s| stays far below 2^-14, so ties land exactly on the
 *    half-integer and everything else stays on its side of it;
 *  mode 2 (snap, as the kernel computes it): t = fma(x, r, 1536) clamped to
 *    [1536 - 128, 1536 + 127], then the low byte of the bits of
 *    t + (1.5 * 2^23 - 1536), whose rounding to an integer is round half to
 *    even of the snapped quotient, read as an int8;
 *  mode 3: mode 2 for bf16 x and s = bf16(fp32(amax) / 127) (bf16 has 8
 *    significant bits, so a non-tie quotient is at least 2^-9 from a
 *    half-integer), over every such s of at least 2^-126 (smaller scales take
 *    the divide).
 * For every positive s the quantiser can produce
 * (s = fp16(amax / 127) for a finite fp16 amax) and every finite fp16 x with
 * |x| <= the largest amax giving that s, this program checks that the result
 * equals clamp(rint(x / s)) for each reciprocal r within +-KMAX ulps of the
 * correctly rounded 1/s (the hardware reciprocal is within one ulp).
 *
 * usage: quant_rounding_check SLICE NSLICES KMAX [MODE]   (exit status 0 = no mismatch)
 * Test infrastructure; it shares nothing with the kernels. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

static float b2f(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t f2b(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static float clampq(float r) { return fminf(fmaxf(r, -128.0f), 127.0f); }

int main(int argc, char **argv) {
    if (argc != 4 && argc != 5) { fprintf(stderr, "usage: %s SLICE NSLICES KMAX [MODE]\n", argv[0]); return 2; }
    const int slice = atoi(argv[1]), nslices = atoi(argv[2]), kmax = atoi(argv[3]);
    const int mode = argc == 5 ? atoi(argv[4]) : 0;
    static float amax_of_s[65536];
    static unsigned char reach[65536];
    const int bf = mode == 3;
    const uint32_t finite_end = bf ? 0x7F80u : 0x7C00u;
    for (uint32_t a = 1; a < finite_end; ++a) {
        const float af = bf ? b2f((uint16_t)a) : h2f((uint16_t)a);
        const uint16_t sb = bf ? f2b(af / 127.0f) : f2h(af / 127.0f);
        const float sf = bf ? b2f(sb) : h2f(sb);
        if (sf == 0.0f || (bf && sf < 0x1p-126f)) continue;
        reach[sb] = 1;
        if (af > amax_of_s[sb]) amax_of_s[sb] = af;
    }
    long long checked = 0, bad = 0, ties = 0;
    for (uint32_t sb = 1; sb < finite_end; ++sb) {
        if (!reach[sb] || (int)(sb % (uint32_t)nslices) != slice) continue;
        const float s = bf ? b2f((uint16_t)sb) : h2f((uint16_t)sb), hs = 0.5f * s, lim = amax_of_s[sb];
        const float r0 = 1.0f / s;
        for (int k = -kmax; k <= kmax; ++k) {
            float r = r0;
            for (int t = 0; t < abs(k); ++t) r = nextafterf(r, k < 0 ? 0.0f : INFINITY);
            for (uint32_t xb = 0; xb < 0x10000; ++xb) {
                if ((xb & 0x7FFF) >= finite_end) continue;
                const float x = bf ? b2f((uint16_t)xb) : h2f((uint16_t)xb);
                if (fabsf(x) > lim) continue;
                const float ref = clampq(rintf(x / s));
                float q0;
                if (mode == 2 || mode == 3) {
                    const float t = fminf(fmaxf(fmaf(x, r, 1536.0f), 1408.0f), 1663.0f);
                    const float y = t + (12582912.0f - 1536.0f);
                    uint32_t bits;
                    memcpy(&bits, &y, 4);
                    q0 = (float)(int8_t)(uint8_t)(bits & 0xFFu);
                    ties += (k == 0 && fabsf(fmaf(-q0, s, x)) == hs);
                } else if (mode == 1) {
                    q0 = rintf(fmaf(x, r, 1536.0f) - 1536.0f);
                    ties += (k == 0 && fabsf(fmaf(-q0, s, x)) == hs);
                } else {
                    q0 = rintf(x * r);
                    const float d = fmaf(-q0, s, x);
                    if (fabsf(d) == hs) {
                        ties += (k == 0);
                        if (fmodf(q0, 2.0f) != 0.0f) q0 += d > 0 ? 1.0f : -1.0f;
                    }
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
