/*
 * quotient_check.c -- CPU check of the division-free grid level the GPU
 * kernels use (test code; it emulates the kernels' formula with the C
 * library's correctly rounded fmaf and compares it with IEEE division).
 *
 * The kernels decide a code as clamp(rint(x / s + zoff), qlo, qhi) where the
 * binary32 quotient x / s (page "LLM 量化方法原理与实现详解", §2.2: the
 * printed quantizers round x / scale (+ zero_point) in the tensor's own
 * precision) is formed without a division per element:
 *     s = s' 2^-k with s' in [1, 2)   (frexp, once per group)
 *     r = RN(1 / s')                  (one IEEE division per group)
 *     x' = clamp(x 2^k, -2^21, 2^21)
 *     q0 = RN(x' r);  q = RN(q0 + RN(x' - q0 s') r)   (two fused multiply-adds)
 * Markstein's theorem (IBM J. Res. Dev. 34(1), 1990) makes q = RN(x' / s').
 *
 * Checks, each counting disagreements with RN(x / s) and with the code the
 * division gives:
 *   exhaustive  every s' = 1 + m 2^-23 in [1, 2); for each, quotients next to
 *               the half-integers n + 1/2 (the ties of rint) and the integers,
 *               x' = RN((n + 1/2) s') and its neighbours +-1, 2 ulp, for
 *               n = 0, 1, 2, 7, 15, 127, 255, 1000, 2^20 - 1, and random x'
 *   random      (x, s) over the whole binary32 range: subnormal and huge
 *               scales, subnormal and huge weights, both signs, through the
 *               kernels' full path (frexp of s, ldexp of x, the clamp)
 *
 * The quotient is compared where x' is at least 2^-100 (below, the remainder
 * can underflow, and |x / s| is then far below 1/2, where every code is the
 * zero point either way); codes are compared everywhere.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off quotient_check.c -lm
 * Usage: quotient_check [m_stride] [n_random]; prints "<bad_q> <bad_code> <checked>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* The kernels' grid scaling of one group: s' = 2 m, k = 1 - e for s = m 2^e. */
static void grid_scale(float s, float *ss, float *rs, int *k)
{
    int e;
    float m = frexpf(s, &e);
    *ss = 2.0f * m;
    *k = 1 - e;
    *rs = 1.0f / *ss;
}

static float med3(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

/* The kernels' quotient of x by the group scale. */
static float kernel_quotient(float x, float ss, float rs, int k)
{
    float xs = med3(ldexpf(x, k), -2097152.0f, 2097152.0f);
    float q0 = xs * rs;
    return fmaf(fmaf(-q0, ss, xs), rs, q0);
}

/* splitmix64 step on a per-iteration state, so threads draw independent streams */
static uint64_t next(uint64_t *state)
{
    uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

typedef struct { long bad_q, bad_code, checked; } tally;

/* One (x', s') pair with s' in [1, 2): quotient and 4-bit asymmetric / symmetric codes. */
static void check_scaled(tally *t, float xs, float ss, float rs)
{
    float q = kernel_quotient(xs, ss, rs, 0);
    float ref = xs / ss;
    t->checked++;
    if (fabsf(xs) >= 0x1p-100f && to_bits(q) != to_bits(ref)) t->bad_q++;
    for (int zoff = 0; zoff < 2; ++zoff) {
        float a = med3(rintf(q + (float)zoff), 0.0f, 15.0f);
        float b = med3(rintf(ref + (float)zoff), 0.0f, 15.0f);
        if (a != b) t->bad_code++;
    }
}

/* One (x, s) pair through the whole path, against the division on the unscaled values. */
static void check_full(tally *t, float x, float s, int bits, int sym, float zoff)
{
    float ss, rs;
    int k;
    grid_scale(s, &ss, &rs, &k);
    float q = kernel_quotient(x, ss, rs, k);
    float ref = x / s;
    float qlo = sym ? -(float)((1 << (bits - 1)) - 1) : 0.0f;
    float qhi = sym ? (float)((1 << (bits - 1)) - 1) : (float)((1 << bits) - 1);
    float a = med3(rintf(q + zoff), qlo, qhi);
    float b = med3(rintf(ref + zoff), qlo, qhi);
    t->checked++;
    if (a != b) t->bad_code++;
    /* where nothing was clamped the quotient itself must be the division's */
    if (fabsf(ref) < 1048576.0f && fabsf(ref) > 1e-30f && to_bits(q) != to_bits(ref)) t->bad_q++;
}

int main(int argc, char **argv)
{
    long stride = argc > 1 ? atol(argv[1]) : 1;
    long n_random = argc > 2 ? atol(argv[2]) : 1000000;
    static const float ns[] = {0.0f, 1.0f, 2.0f, 7.0f, 15.0f, 127.0f, 255.0f, 1000.0f, 1048575.0f};
    long bad_q = 0, bad_code = 0, checked = 0;
#pragma omp parallel for schedule(static, 4096) reduction(+ : bad_q, bad_code, checked)
    for (long m = 0; m < (1l << 23); m += stride) {
        tally t = {0, 0, 0};
        uint64_t st = 0x243F6A8885A308D3ull ^ ((uint64_t)m << 20);
        float ss = from_bits(0x3F800000u | (uint32_t)m); /* 1 + m 2^-23 */
        float rs = 1.0f / ss;
        for (unsigned i = 0; i < sizeof ns / sizeof ns[0]; ++i) {
            for (int half = 0; half < 2; ++half) {
                float tq = half ? (float)((double)ns[i] + 0.5) : ns[i];
                float x0 = (float)((double)tq * (double)ss);
                for (int d = -2; d <= 2; ++d) {
                    float x = from_bits(to_bits(x0) + (uint32_t)d);
                    if (!(x > 0.0f) || x > 2097152.0f) continue;
                    check_scaled(&t, x, ss, rs);
                    check_scaled(&t, -x, ss, rs);
                }
            }
        }
        /* a random x' in [2^-30, 2^21) */
        float xr = ldexpf(1.0f + (float)(next(&st) >> 41) * 0x1p-23f, (int)(next(&st) % 51) - 30);
        check_scaled(&t, xr, ss, rs);
        bad_q += t.bad_q;
        bad_code += t.bad_code;
        checked += t.checked;
    }
#pragma omp parallel for schedule(static, 4096) reduction(+ : bad_q, bad_code, checked)
    for (long i = 0; i < n_random; ++i) {
        tally t = {0, 0, 0};
        uint64_t st = 0x13198A2E03707344ull ^ ((uint64_t)i << 16);
        /* any finite positive scale (subnormal included) and any finite weight */
        uint32_t su = (uint32_t)(next(&st) % 0x7F7FFFFFu) + 1u;
        uint32_t xu = (uint32_t)(next(&st) % 0x7F800000u) | ((uint32_t)(next(&st) & 1) << 31);
        float s = from_bits(su), x = from_bits(xu);
        int bits = 2 + (int)(next(&st) % 7);
        int sym = (int)(next(&st) & 1);
        float zoff = sym ? 0.0f : (float)(next(&st) % (1u << bits));
        check_full(&t, x, s, bits, sym, zoff);
        /* a weight within a few grid steps of the scale (the usual case): x = (n + f) s */
        float tq = (float)(next(&st) % 300) - 150.0f + (float)(next(&st) % 8) * 0.125f;
        check_full(&t, tq * s, s, bits, sym, zoff);
        check_full(&t, from_bits(to_bits(tq * s) + 1u), s, bits, sym, zoff);
        bad_q += t.bad_q;
        bad_code += t.bad_code;
        checked += t.checked;
    }
    printf("%ld %ld %ld\n", bad_q, bad_code, checked);
    return 0;
}
