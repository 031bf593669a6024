/*
 * division_check.c -- CPU proof of the quotient arithmetic of the GPU fast
 * paths (test infrastructure; neither the library nor the oracle uses it).
 *
 * The method computes v = x / s as one correctly rounded binary32 division
 * (post "浅谈低精度浮点数", section "FP8": x^ = s * round(x / s)).  The GPU
 * kernels reach that quotient without a division instruction:
 *   - a constant divisor Q (scales alpha / 127, / 448, / 57344; block
 *     maxima A / 6 and A / 7) by one correction step from RN(1/Q):
 *       q0 = a * r;  e = fma(-Q, q0, a);  q = fma(e, r, q0)
 *   - a unit's scale s by the correction step from y = RN(1/s):
 *       q0 = x * y;  r = fma(s, q0, -x);  v = fma(-r, y, q0)
 *     where, for the INT4 FP16 scales, y comes from a 1024-entry table of
 *     RN(1 / (1 + f/1024)) scaled by 2^-e.
 * This program restates that arithmetic in C (binary32, explicit fmaf, no
 * contraction) and compares it bit for bit with the correctly rounded C
 * division over the domains the kernels use it on.  A quotient below 2^-20
 * may differ (every code grid rounds it to a signed zero): there the check
 * is that the corrected value stays below 2^-19 with the same sign.
 *
 * Usage: division_check <check>   with <check> one of
 *   divconst     every finite binary32 a >= 0 (the kernels divide absolute
 *                maxima only) against a / Q, Q in {6, 7, 15, 127, 448, 57344}:
 *                any difference where the quotient is normal counts, and
 *                for Q = 7, 15 and 127 any difference at all
 *   row_bf16     per-row INT8 / E4M3 / E5M2: every BF16 absmax alpha in
 *                [2^-40, 2^60], s = alpha / Q, every BF16 x with |x| <= alpha
 *   int4_fp16    every normal FP16 scale sf: the table reciprocal equals
 *                RN(1/sf), and every BF16 x with |x| <= 7.5 sf
 *   nvfp4        64 seeded global maxima G, s_g = G / 2688, every E4M3 block
 *                code c: s = s_g * value(c), every BF16 x with |x| <= 6.5 s;
 *                and the block-scale quotient (A/6) / s_g for every BF16
 *                A <= G
 *   random_f32   10^8 seeded binary32 pairs per Q with |x| <= alpha
 *   int4zp       asymmetric INT4: 32768 seeded BF16 group ranges, the scale
 *                span / 15, the shift quotient and every BF16 x in range
 *   a7_double_rounding  the INT4 FP16 scale: rounding A / 7 to binary32
 *                first gives the same binary16 as one rounding, for every
 *                finite binary32 A up to the binary16 range
 * It prints "<check> <pairs checked> <mismatches>" per line; exit status 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static inline float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* The empty asm statements keep gcc from folding a negation into an fma
 * (-fma(a, b, c) -> fma(-a, b, -c)), which changes the sign of exact zeros;
 * the GPU code is compiled as written. */
#define KEEP(v) __asm__("" : "+x"(v))

static inline float corrected_quotient(float x, float s, float y) {
    float q0 = x * y;
    KEEP(q0);
    float r = fmaf(s, q0, -x);
    KEEP(r);
    return fmaf(-r, y, q0);
}

/* Called on a >= 0 only, where no zero changes sign: no barriers, so the
 * exhaustive loop vectorizes. */
static inline float const_quotient(float a, float Q, float r) {
    const float q0 = a * r;
    const float e = fmaf(-Q, q0, a);
    return fmaf(e, r, q0);
}

/* 1 if the corrected quotient vm is acceptable for the true quotient v. */
static inline int quotient_ok(float vm, float v) {
    if (bf(vm) == bf(v)) return 1;
    return fabsf(v) < 0x1p-20f && fabsf(vm) < 0x1p-19f && signbit(vm) == signbit(v);
}

static float e4m3_value(uint32_t c) {   /* positive E4M3 codes 1 .. 0x7E */
    const uint32_t e = c >> 3, m = c & 7u;
    return e ? ldexpf((float)(8 + m), (int)e - 7 - 3) : ldexpf((float)m, -9);
}

static void divconst(void) {
    const float Qs[6] = {6.f, 7.f, 15.f, 127.f, 448.f, 57344.f};
    for (int qi = 0; qi < 6; ++qi) {
        const float Q = Qs[qi], r = 1.0f / Q;
        const int strict = Q == 7.f || Q == 15.f || Q == 127.f;
        uint64_t bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
        for (int64_t hi = 0; hi < 32768; ++hi) {   /* a >= 0: every caller passes an absolute maximum */
            if ((((uint32_t)hi << 16) & 0x7F800000u) == 0x7F800000u) continue;   /* Inf, NaN */
            uint32_t b = 0;
            for (uint32_t lo = 0; lo < 65536; ++lo) {
                const float a = fb(((uint32_t)hi << 16) | lo);
                const float q = a / Q, qc = const_quotient(a, Q, r);
                b += (bf(q) != bf(qc)) & (strict | (fabsf(q) >= 0x1p-126f));
            }
            bad += b;
            n += 65536;
        }
        printf("divconst_%g %llu %llu\n", (double)Q, (unsigned long long)n, (unsigned long long)bad);
    }
}

/* every BF16 x with |x| <= lim (both signs) against scale s, reciprocal y */
static void sweep_bf16(float s, float y, float lim, uint64_t* n, uint64_t* bad) {
    for (uint32_t b = 0; b < 0x7F80u; ++b) {
        const float xa = fb(b << 16);
        if (xa > lim) break;
        for (int sg = 0; sg < 2; ++sg) {
            const float x = sg ? -xa : xa;
            ++*n;
            if (!quotient_ok(corrected_quotient(x, s, y), x / s)) ++*bad;
        }
    }
}

static void row_bf16(void) {
    const float Qs[3] = {127.f, 448.f, 57344.f};
    const uint32_t lo = bf(0x1p-40f) >> 16, hi = bf(0x1p60f) >> 16;
    for (int qi = 0; qi < 3; ++qi) {
        const float Q = Qs[qi];
        uint64_t bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(dynamic, 16)
        for (int64_t a = lo; a <= (int64_t)hi; ++a) {
            const float alpha = fb((uint32_t)a << 16);
            const float s = alpha / Q, y = 1.0f / s;
            uint64_t nn = 0, bb = 0;
            sweep_bf16(s, y, alpha, &nn, &bb);
            n += nn;
            bad += bb;
        }
        printf("row_bf16_%g %llu %llu\n", (double)Q, (unsigned long long)n, (unsigned long long)bad);
    }
}

static void int4_fp16(void) {
    float rtab[1024];
    for (int f = 0; f < 1024; ++f) rtab[f] = 1.0f / (1.0f + (float)f * 0x1p-10f);
    uint64_t bad = 0, n = 0, bad_tab = 0;
#pragma omp parallel for reduction(+ : bad, n, bad_tab) schedule(dynamic, 64)
    for (int64_t h = 0x0400; h <= 0x7BFF; ++h) {
        const int ex = (int)((h >> 10) & 0x1F) - 15;
        const float sf = ldexpf(1.0f + (float)(h & 0x3FF) * 0x1p-10f, ex);
        const float y = ldexpf(rtab[h & 0x3FF], -ex);
        if (bf(y) != bf(1.0f / sf)) ++bad_tab;
        uint64_t nn = 0, bb = 0;
        sweep_bf16(sf, y, 7.5f * sf, &nn, &bb);
        n += nn;
        bad += bb;
    }
    printf("int4_fp16_table 30720 %llu\n", (unsigned long long)bad_tab);
    printf("int4_fp16 %llu %llu\n", (unsigned long long)n, (unsigned long long)bad);
}

static uint64_t splitmix(uint64_t* s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void nvfp4(void) {
    uint64_t seed = 0x6E7646700001ull;
    float G[64];
    for (int i = 0; i < 64; ++i) {          /* positive normal BF16 maxima over the whole range */
        const uint32_t b = 0x0080u + (uint32_t)(splitmix(&seed) % (0x7F7Fu - 0x0080u));
        G[i] = fb(b << 16);
    }
    uint64_t bad = 0, n = 0, bad_t = 0, n_t = 0;
#pragma omp parallel for reduction(+ : bad, n, bad_t, n_t) schedule(dynamic, 1) collapse(2)
    for (int gi = 0; gi < 64; ++gi) {
        for (int c = 1; c <= 0x7E; ++c) {
            const float s_g = G[gi] / 2688.0f;
            const float s = s_g * e4m3_value((uint32_t)c);
            if (s < 0x1p-64f || !(s > 0.f)) continue;        /* tiny scales: the division path */
            const float y = 1.0f / s;
            uint64_t nn = 0, bb = 0;
            sweep_bf16(s, y, 6.5f * s, &nn, &bb);
            n += nn;
            bad += bb;
            if (c == 1) {                               /* block-scale quotient (A/6)/s_g, A <= G */
                const float y_g = 1.0f / s_g;
                for (uint32_t b = 1; b < 0x7F80u; ++b) {
                    const float A = fb(b << 16);
                    if (A > G[gi]) break;
                    const float t1 = A / 6.0f, t = t1 / s_g;
                    if (!(t1 >= 0x1p-100f && t >= 0x1p-100f && t <= 0x1p120f)) continue;
                    ++n_t;
                    if (bf(corrected_quotient(t1, s_g, y_g)) != bf(t)) ++bad_t;
                }
            }
        }
    }
    printf("nvfp4_block_scale %llu %llu\n", (unsigned long long)n_t, (unsigned long long)bad_t);
    printf("nvfp4 %llu %llu\n", (unsigned long long)n, (unsigned long long)bad);
}

/* Asymmetric INT4 groups: span = hi + nlo (hi = max(0, max x), nlo =
 * -min(0, min x), BF16 magnitudes), sc = span / 15 by the constant-divisor
 * correction, y = RN(1 / sc).  Seeded pairs (hi, nlo), one within 24
 * binades of the other, max(hi, nlo) in the fast range [2^-40, 2^60] and
 * sc >= 2^-64, one in four one-sided:
 * sc against the division, the shift RNE(nlo / sc) clamped to [0, 15]
 * from the corrected quotient against the division's, and the corrected
 * quotient of every BF16 x in [-nlo, hi]. */
static void int4zp(void) {
    uint64_t bad = 0, n = 0, bad_sc = 0, bad_sh = 0, groups = 0;
    const float lo_lim = 0x1p-40f, hi_lim = 0x1p60f;
    const uint32_t blo = bf(lo_lim) >> 16, bhi = bf(hi_lim) >> 16;
#pragma omp parallel for reduction(+ : bad, n, bad_sc, bad_sh, groups) schedule(dynamic, 4)
    for (int64_t pi = 0; pi < 32768; ++pi) {
        uint64_t seed = 0x7A70000000ull + (uint64_t)pi * 0x10001ull;
        const uint64_t r = splitmix(&seed);
        /* hi anywhere in the fast range, nlo within 24 binades of it */
        uint32_t hb = blo + (uint32_t)(r % (bhi - blo + 1));
        int32_t nbs = (int32_t)hb + (int32_t)((r >> 24) % (48u * 128u)) - 24 * 128;
        uint32_t nb = nbs < 0x0080 ? 0x0080u : nbs > 0x7F7F ? 0x7F7Fu : (uint32_t)nbs;
        if ((r >> 61) == 0) hb = 0;          /* one-sided groups */
        else if ((r >> 61) == 1) nb = 0;
        if ((r >> 56) & 1) { const uint32_t t = hb; hb = nb; nb = t; }
        const float hi = fb(hb << 16), nlo = fb(nb << 16), m = hi > nlo ? hi : nlo;
        if (!(m >= lo_lim && m <= hi_lim)) continue;
        const float span = hi + nlo;
        const float sc = span / 15.0f;
        if (bf(const_quotient(span, 15.0f, 1.0f / 15.0f)) != bf(sc)) ++bad_sc;
        if (!(sc >= 0x1p-64f)) continue;
        ++groups;
        const float y = 1.0f / sc;
        const float shd = fminf(fmaxf(rintf(nlo / sc), 0.f), 15.f);
        const float shm = fminf(fmaxf(rintf(corrected_quotient(nlo, sc, y)), 0.f), 15.f);
        if (bf(shd) != bf(shm)) ++bad_sh;
        uint64_t nn = 0, bb = 0;
        for (uint32_t b = 0; b < 0x7F80u; ++b) {
            const float xa = fb(b << 16);
            if (xa > hi && xa > nlo) break;
            if (xa <= hi) { ++nn; if (!quotient_ok(corrected_quotient(xa, sc, y), xa / sc)) ++bb; }
            if (xa <= nlo) { ++nn; if (!quotient_ok(corrected_quotient(-xa, sc, y), -xa / sc)) ++bb; }
        }
        n += nn;
        bad += bb;
    }
    printf("int4zp_scale %llu %llu\n", (unsigned long long)groups, (unsigned long long)bad_sc);
    printf("int4zp_shift %llu %llu\n", (unsigned long long)groups, (unsigned long long)bad_sh);
    printf("int4zp %llu %llu\n", (unsigned long long)n, (unsigned long long)bad);
}

/* The INT4 scale rounds A / 7 to binary32 first, then to binary16 (RNE).
 * Every finite binary32 A whose quotient is within the binary16 range:
 * fp16(fl32(A / 7)) against the single rounding fp16(A / 7), taken from
 * the binary64 quotient (53 bits: its own rounding cannot reach a binary16
 * midpoint).  f16 rounds a non-negative double to binary16, exactly. */
static double f16_of(double v) {
    if (v == 0) return 0;
    int e;
    frexp(v, &e);
    e -= 1;
    if (e < -14) e = -14;
    const double ulp = ldexp(1.0, e - 10);
    return nearbyint(v / ulp) * ulp;
}

static void a7_double_rounding(void) {
    uint64_t bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
    for (int64_t hi = 0; hi < 0x7F80; ++hi) {
        for (uint32_t lo = 0; lo < 65536; ++lo) {
            float A = fb(((uint32_t)hi << 16) | lo);
            KEEP(A);
            float q32 = A / 7.0f;
            KEEP(q32);
            const double q64 = (double)A / 7.0;
            if (q64 > 65520.0) continue;   /* beyond it the scale saturates at 65504 */
            ++n;
            if (f16_of((double)q32) != f16_of(q64)) ++bad;
        }
    }
    printf("a7_double_rounding %llu %llu\n", (unsigned long long)n, (unsigned long long)bad);
}

static void random_f32(void) {
    const float Qs[5] = {127.f, 448.f, 57344.f, 6.f, 7.f};
    for (int qi = 0; qi < 5; ++qi) {
        const float Q = Qs[qi];
        uint64_t bad = 0, n = 0;
#pragma omp parallel for reduction(+ : bad, n) schedule(static)
        for (int64_t blk = 0; blk < 1000; ++blk) {
            uint64_t seed = 0x5EED0000ull * (uint64_t)(qi + 1) + (uint64_t)blk;
            for (int i = 0; i < 100000; ++i) {
                const uint64_t r = splitmix(&seed);
                /* alpha: exponent in [-40, 60], random significand */
                const int ea = -40 + (int)(r % 101);
                const float alpha = ldexpf(1.0f + (float)((r >> 8) & 0x7FFFFF) * 0x1p-23f, ea);
                const float s = alpha / Q, y = 1.0f / s;
                /* x: |x| <= alpha, magnitude spread over 60 binades below alpha */
                const uint64_t r2 = splitmix(&seed);
                float x = ldexpf(1.0f + (float)(r2 & 0x7FFFFF) * 0x1p-23f, ea - (int)((r2 >> 32) % 61));
                if (x > alpha) x = alpha;
                if (r2 >> 63) x = -x;
                ++n;
                if (!quotient_ok(corrected_quotient(x, s, y), x / s)) ++bad;
            }
        }
        printf("random_f32_%g %llu %llu\n", (double)Q, (unsigned long long)n, (unsigned long long)bad);
    }
}

int main(int argc, char** argv) {
    if (argc != 2) return 2;
    if (!strcmp(argv[1], "divconst")) divconst();
    else if (!strcmp(argv[1], "row_bf16")) row_bf16();
    else if (!strcmp(argv[1], "int4_fp16")) int4_fp16();
    else if (!strcmp(argv[1], "nvfp4")) nvfp4();
    else if (!strcmp(argv[1], "random_f32")) random_f32();
    else if (!strcmp(argv[1], "int4zp")) int4zp();
    else if (!strcmp(argv[1], "a7_double_rounding")) a7_double_rounding();
    else return 2;
    return 0;
}
