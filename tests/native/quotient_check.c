/*
 * quotient_check.c -- CPU check of the quantizers' division sequence (test
 * only).  The quantizer forms fl32(x / s) without a divide instruction:
 *     r = RN(1/s),  y = RN(x * r),  e = RN(y * s - x) (one FMA),
 *     q = RN(y - e * r)             (one FMA),
 * the correction step of Markstein (IBM J. Res. Dev. 34(1), 1990; see also
 * the chapter on division with an FMA in Muller et al., Handbook of
 * Floating-Point Arithmetic).  This program evaluates the same sequence with
 * IEEE fp32 operations (fmaf is correctly rounded) and compares q with the
 * correctly rounded quotient x / s bit for bit, for
 *   - scales s = RN(amax / 448) over many amax (random, powers of two, and
 *     values next to the fast-path threshold 2^-64 and to the top of the range),
 *   - x next to every point where the E4M3 code of the quotient changes
 *     (the 126 midpoints between consecutive magnitudes and the saturation
 *     boundary 448), +-8 fp32 ulps around RN(mid * s), both signs,
 *   - random x in [-amax, amax], and +-0.
 * Usage: quotient_check <n_scales> <seed>; prints counts; exit status 1 on a
 * mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float quotient(float x, float s, float r) {
    float y = x * r;
    float e = fmaf(y, s, -x);
    return fmaf(-e, r, y);
}

static uint64_t rng_state;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static double mids[128];
static int n_mids;

static void build_mids(void) {
    double mag[127];
    for (int c = 0; c < 127; ++c) {
        int e = c >> 3, m = c & 7;
        mag[c] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    }
    n_mids = 0;
    for (int c = 0; c < 126; ++c) mids[n_mids++] = 0.5 * (mag[c] + mag[c + 1]);
    mids[n_mids++] = 448.0;
}

static long long n_checked, n_bad;

static void check(float x, float s, float r) {
    float q = quotient(x, s, r);
    float d = x / s;
    ++n_checked;
    if (bits(q) != bits(d)) {
        if (++n_bad <= 10)
            printf("mismatch: x=%a s=%a fast=%a ieee=%a\n", (double)x, (double)s, (double)q, (double)d);
    }
}

static void check_scale(float amax) {
    float s = amax / 448.0f;
    if (!(s >= 0x1p-64f) || !isfinite(s)) return; /* the quantizer divides exactly below 2^-64 */
    float r = 1.0f / s;
    for (int i = 0; i < n_mids; ++i) {
        float x0 = (float)(mids[i] * (double)s);
        if (!isfinite(x0)) continue;
        for (int k = -8; k <= 8; ++k) {
            uint32_t b = bits(x0);
            if (k < 0 && b < (uint32_t)(-k)) continue;
            float x = fbits(b + (uint32_t)k);
            if (!isfinite(x) || fabsf(x) > amax) continue;
            check(x, s, r);
            check(-x, s, r);
        }
    }
    for (int i = 0; i < 64; ++i) {
        float u = (float)((next_u64() >> 40) * 0x1p-24); /* [0, 1) */
        float x = u * amax;
        check((next_u64() & 1) ? x : -x, s, r);
    }
    check(0.0f, s, r);
    check(-0.0f, s, r);
    check(amax, s, r);
    check(-amax, s, r);
}

int main(int argc, char** argv) {
    long n = argc > 1 ? atol(argv[1]) : 20000;
    rng_state = argc > 2 ? strtoull(argv[2], 0, 10) : 1;
    build_mids();
    /* random amax: uniform exponent over [2^-57, 2^127), random mantissa */
    for (long i = 0; i < n; ++i) {
        uint32_t e = 70 + (uint32_t)(next_u64() % 184); /* biased exponents 70 .. 253 */
        uint32_t m = (uint32_t)(next_u64() & 0x7fffff);
        check_scale(fbits((e << 23) | m));
    }
    /* powers of two, the threshold neighbourhood and the top of the range */
    for (int e = -60; e <= 127; ++e) check_scale(ldexpf(1.0f, e));
    for (uint32_t k = 0; k < 4096; ++k) {
        check_scale(fbits(bits(448.0f * 0x1p-64f) + k));
        check_scale(fbits(bits(448.0f * 0x1p-64f) - k));
        check_scale(fbits(0x7f7fffffu - k));
        check_scale(fbits(bits(448.0f) + k));
        check_scale(fbits(bits(1.0f) + k));
    }
    printf("checked %lld quotients, %lld differ from IEEE division\n", n_checked, n_bad);
    return n_bad ? 1 : 0;
}
