/* Exhaustive host check of the divide-free quotient used by the INT4-FP8
 * activation quantiser (the reading of the QQQ PR "Support W4A8 quantization
 * for vllm" for E4M3 codes: code = e4m3(clamp(x / s, +-448)) with the fp32
 * quotient correctly rounded and s = act(fp32(amax) / 448)).
 *
 * The kernel divides once per row, r = RN(1 / s'), and per value computes
 *   q0 = RN(x' * r),  e = RN(x' - q0 * s') (exact, one FMA),  q1 = RN(q0 + e * r)
 * (Markstein's correction step; with r the correctly rounded reciprocal, q1
 * is the correctly rounded quotient when nothing underflows), where x' and s'
 * are x and s times 2^64 on rows with s < 2^-60 (exact, and the same
 * quotient): then every x whose quotient can reach the smallest E4M3 subnormal
 * is at least 2^-72, far above the range where the residual e would round.
 * Without the scaling, bf16 rows with s near 2^-120 and subnormal x give
 * wrong codes.  The kernel gives the result x's sign (the correction turns
 * -0 into +0), so negative x are the mirror image and x = 0 gives code 0 of
 * its sign.  For every
 * positive s the quantiser can produce from a finite fp16 (MODE 0) or bf16
 * (MODE 1) amax -- bf16 scales of at least 2^-126; smaller ones keep the
 * divide -- and every finite positive x of that type with x <= the largest
 * amax giving that s (and x = 0), this program checks that the E4M3 code of clamp(q1)
 * equals that of clamp(x / s), and counts the pairs where q1 itself differs
 * from x / s (quotients far below the smallest E4M3 subnormal, code 0).
 *
 * usage: fp8_quotient_check SLICE NSLICES MODE   (exit status 0 = no code mismatch)
 * Test infrastructure; it shares nothing with the kernels. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float h2f(uint16_t h) {
    const uint32_t e = (h >> 10) & 31, m = h & 1023;
    if (e == 0) return ldexpf((float)m, -24);
    return ldexpf((float)(m | 1024), (int)e - 25);
}

/* fp32 -> fp16 bits, round to nearest even (finite positive inputs) */
static uint16_t f2h(float f) {
    uint32_t lo = 0, hi = 0x7C00;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (h2f((uint16_t)mid) <= f) lo = mid; else hi = mid;
    }
    const double dl = fabs((double)h2f((uint16_t)lo) - f);
    const double dh = hi < 0x7C00 ? fabs((double)h2f((uint16_t)hi) - f) : INFINITY;
    if (dl < dh || (dl == dh && (lo & 1) == 0)) return (uint16_t)lo;
    return (uint16_t)hi;
}

static float b2f(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f2b(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* E4M3 code of a non-negative fp32 value <= 448, round to nearest even */
static uint32_t e4m3(float q) {
    uint32_t a;
    memcpy(&a, &q, 4);
    if (a < 0x3C800000u) return (uint32_t)rintf(q * 512.0f);
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    return r - ((127u - 7u) << 3);
}

int main(int argc, char **argv) {
    if (argc != 4) { fprintf(stderr, "usage: %s SLICE NSLICES MODE\n", argv[0]); return 2; }
    const int slice = atoi(argv[1]), nslices = atoi(argv[2]), bf = atoi(argv[3]) == 1;
    static float amax_of_s[65536];
    static unsigned char reach[65536];
    const uint32_t finite_end = bf ? 0x7F80u : 0x7C00u;
    for (uint32_t a = 1; a < finite_end; ++a) {
        const float af = bf ? b2f((uint16_t)a) : h2f((uint16_t)a);
        const uint16_t sb = bf ? f2b(af / 448.0f) : f2h(af / 448.0f);
        const float sf = bf ? b2f(sb) : h2f(sb);
        if (sf == 0.0f || (bf && sf < 0x1p-126f)) continue;
        reach[sb] = 1;
        if (af > amax_of_s[sb]) amax_of_s[sb] = af;
    }
    long long checked = 0, bad = 0, qdiff = 0;
    for (uint32_t sb = 1; sb < finite_end; ++sb) {
        if (!reach[sb] || (int)(sb % (uint32_t)nslices) != slice) continue;
        const float s = bf ? b2f((uint16_t)sb) : h2f((uint16_t)sb), lim = amax_of_s[sb];
        const float sc = s < 0x1p-60f ? 0x1p64f : 1.0f, ss = s * sc;
        const float r = 1.0f / ss;
        for (uint32_t xb = 0; xb < finite_end; ++xb) {
            const float x = bf ? b2f((uint16_t)xb) : h2f((uint16_t)xb);
            if (x > lim) continue;
            const float ref = fminf(x / s, 448.0f);
            const float xs = x * sc;
            const float q0 = xs * r;
            const float e = fmaf(-q0, ss, xs);
            const float q1 = fminf(copysignf(fmaf(e, r, q0), x), 448.0f);
            ++checked;
            qdiff += q1 != ref;
            if (e4m3(q1) != e4m3(ref)) {
                if (bad < 5) printf("mismatch s=%a x=%a q1=%a ref=%a\n", s, x, q1, ref);
                ++bad;
            }
        }
    }
    printf("slice %d/%d: %lld pairs, %lld quotient differences, %lld code mismatches\n", slice, nslices, checked,
           qdiff, bad);
    return bad != 0;
}
