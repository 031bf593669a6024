/*
 * iq_oracle.c -- plain, slow, CPU oracle for block-scaled quantization.
 *
 * TEST INFRASTRUCTURE ONLY: called by tests, the smoke check and the
 * bench's CPU baseline, never by the GPU library.
 *
 * Sources, cited by page and section:
 *   [LP]  Lorn blog, post "浅谈低精度浮点数" (a brief talk on low-precision
 *         floats): section "IEEE 754 标准浮点数" (FP32 fields, the 25.125
 *         example, FP16/BF16 splits); section "FP8" (the symmetric quantizer
 *         x^ = s*round(x/s), s = alpha/127, |x - x^| <= s/2, FP error model
 *         2^-(M+1)); section "FP4 / MXFP4 / NVFP4" (E2M1 value set, MXFP4
 *         E8M0 block scale per 32, NVFP4 s_global = amax/(6*448) and
 *         s_block = (block_amax/6)/s_global, INT4 s = A/7).
 *   [TR]  Lorn blog, post "Triton", Puzzle 12 "Quantized Matrix Mult": the
 *         extract() helper puts element i of a packed word in bits [4i, 4i+4).
 *
 * Readings where the pages are silent or loose (each also listed in the
 * design notes):
 *   round()            round to nearest, ties to even, on integer and float grids;
 *   overflow           saturate to the largest finite code (127, 7, 448, 57344, 6);
 *   FP8 scale          s = alpha/448 (E4M3) or alpha/57344 (E5M2), by analogy with alpha/127;
 *   x/s                one correctly rounded binary32 division;
 *   scale precision    every scale is computed in binary32; the INT4 scale is then
 *                      rounded to FP16 and that rounded value is the one applied;
 *   MXFP4 exponent     E = clamp(floor(log2 A) - 2 + 127, 0, 254) by default;
 *   NVFP4 block scale  smallest E4M3 value >= (A_b/6)/s_g, capped at 448 (the
 *                      bound analysis of [LP] assumes rounding up);
 *   zero scale         a zero scale (all-zero unit) gives +0 codes and x^ = 0;
 *   absmax             over finite elements only; +-Inf saturates, NaN -> NaN code
 *                      (FP8: 0x7F) or +0 (E2M1, INT);
 *   nibble order       element 2t in bits 3:0 of byte t, element 2t+1 in bits 7:4;
 *   asymmetric INT4    [TR] Puzzle 12 fixes the decoder x^ = sc*(w - sh) with
 *                      unsigned 4-bit w and sh and a float sc per group; the
 *                      encoder is the min-max one: range [lo, hi] widened to
 *                      hold 0, sc = (hi - lo)/15 (binary32; an overflowing
 *                      range is clamped to the largest float), sh = RNE(-lo/sc)
 *                      in [0, 15], w = clamp(RNE(x/sc) + sh, 0, 15); groups of
 *                      128, shifts two per byte;
 *   FP4 GEMM           a product of two MXFP4 operands multiplies their
 *                      dequantized values; the oracle forms that sum exactly.
 */
#include "iq_oracle.h"

#include <fenv.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ---- [LP] "IEEE 754": BF16 is the top half of an FP32 (E8M7) ------------ */
float iqo_bf16_to_f32(uint16_t b) { return f_from_bits((uint32_t)b << 16); }

/* FP32 -> BF16, round to nearest even on the dropped 16 bits; NaN stays NaN. */
uint16_t iqo_f32_to_bf16(float f) {
    uint32_t u = bits_from_f(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xFFFFu, upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* ---- minifloat formats (sign / exponent / mantissa with bias) ----------- */
/* E4M3 and E5M2 are the two FP8 layouts of [LP] "FP8"; E2M1 is the OCP FP4
 * of [LP] "FP4"; FP16 (E5M10) holds the INT4 group scale.  max_mag is the
 * magnitude code of the largest finite value. */
typedef struct {
    int mbits, bias;
    uint32_t max_mag, sign_bit, nan_code;
} minifloat;

static const minifloat MF[4] = {
    /* E4M3: bias 7, no Inf, S.1111.111 is NaN, max 1.75*2^8 = 448 (0x7E) */
    {3, 7, 0x7Eu, 0x80u, 0x7Fu},
    /* E5M2: bias 15, exponent 31 is Inf/NaN, max 1.75*2^15 = 57344 (0x7B) */
    {2, 15, 0x7Bu, 0x80u, 0x7Fu},
    /* E2M1: bias 1, every code finite, max 1.5*2^2 = 6 (0x7) */
    {1, 1, 0x7u, 0x8u, 0x0u},
    /* FP16: bias 15, max 65504 (0x7BFF) */
    {10, 15, 0x7BFFu, 0x8000u, 0x7E00u},
};

/* Value of a code: (1 + m/2^M) * 2^(e - bias) for e > 0, (m/2^M) * 2^(1 - bias)
 * for e = 0.  Computed in double (exact), then narrowed (exact). */
float iqo_fp_decode(int kind, uint32_t code) {
    const minifloat* f = &MF[kind];
    uint32_t mag = code & (f->sign_bit - 1u);
    int neg = (code & f->sign_bit) != 0;
    uint32_t efield = mag >> f->mbits;
    uint32_t m = mag & ((1u << f->mbits) - 1u);
    if (kind == IQO_K_E4M3 && mag == 0x7Fu) return NAN;
    if ((kind == IQO_K_E5M2 || kind == IQO_K_F16) && efield == 31u) {
        if (m) return NAN;
        return neg ? -INFINITY : INFINITY;
    }
    double val;
    if (efield == 0)
        val = ldexp((double)m, 1 - f->bias - f->mbits);
    else
        val = ldexp((double)((1u << f->mbits) + m), (int)efield - f->bias - f->mbits);
    return (float)(neg ? -val : val);
}

/* Round v to the nearest representable value of the format, ties to the even
 * mantissa, keep the sign (also on zero), and saturate magnitudes beyond the
 * largest finite value ([LP] "FP8": 2^M evenly spaced samples per binade
 * [2^e, 2^(e+1)), spacing 2^(e-M); below the smallest normal binade the
 * spacing stays at 2^(emin-M)).  NaN maps to the format's NaN code (0 for
 * E2M1, which has none). */
uint32_t iqo_fp_encode(int kind, float v) {
    const minifloat* f = &MF[kind];
    if (isnan(v)) return f->nan_code;
    uint32_t sign = signbit(v) ? f->sign_bit : 0u;
    double a = fabs((double)v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | f->max_mag;
    int e;
    (void)frexp(a, &e);
    e -= 1;                              /* a in [2^e, 2^(e+1)) */
    int emin = 1 - f->bias;              /* exponent of the smallest normal */
    int eb = e < emin ? emin : e;        /* binade whose spacing applies */
    double n = nearbyint(ldexp(a, f->mbits - eb)); /* a / 2^(eb-M), ties to even */
    /* code magnitude = (binade index) * 2^M + integer significand; a carry
     * n == 2^(M+1) lands exactly on the next binade's first code. */
    double mag = (double)(eb - emin) * (double)(1u << f->mbits) + n;
    if (mag > (double)f->max_mag) mag = (double)f->max_mag;
    return sign | (uint32_t)mag;
}

/* ---- [LP] "FP8": symmetric integer grid, q in [-qmax, qmax] ------------- */
int iqo_int_encode(float v, int qmax) {
    if (isnan(v)) return 0;
    float r = nearbyintf(v); /* current rounding mode: to nearest, ties to even */
    if (r > (float)qmax) return qmax;
    if (r < -(float)qmax) return -qmax;
    return (int)r;
}

/* ---- [LP] "FP4 / MXFP4": E8M0 shared exponent per 32 elements ----------- */
/* Default rule: E = floor(log2 A) - 2 (so the block maximum lands in [4, 8)
 * in the scaled domain).  Flag variants: the page's round(log2(A/6)) and its
 * round-up form.  Biased by 127 and clamped to the finite codes [0, 254];
 * A == 0 gives code 0. */
uint8_t iqo_e8m0_code(float A, uint32_t flags) {
    if (!(A > 0.0f)) return 0;
    int e;
    if (flags & IQO_FLAG_MX_ROUND_NEAREST) {
        e = (int)nearbyint(log2((double)A / 6.0));
    } else if (flags & IQO_FLAG_MX_ROUND_UP) {
        e = (int)ceil(log2((double)A / 6.0));
    } else {
        e = ilogbf(A) - 2;                /* ilogb = floor(log2 |A|), exact */
    }
    int E = e + 127;
    if (E < 0) E = 0;
    if (E > 254) E = 254;
    return (uint8_t)E;
}

float iqo_e8m0_value(uint8_t code) {
    if (code == 255) return NAN;
    return ldexpf(1.0f, (int)code - 127); /* 2^-127 is an FP32 subnormal, exact */
}

/* Smallest E4M3 value >= t (t >= 0), capped at the largest finite 448. */
uint8_t iqo_e4m3_ceil(float t) {
    for (uint32_t c = 0; c <= 0x7Eu; ++c)
        if ((double)iqo_fp_decode(IQO_K_E4M3, c) >= (double)t) return (uint8_t)c;
    return 0x7E;
}

void iqo_fp_encode_n(int kind, const float* v, uint32_t* code, int64_t n) {
    for (int64_t i = 0; i < n; ++i) code[i] = iqo_fp_encode(kind, v[i]);
}
void iqo_fp_decode_n(int kind, const uint32_t* code, float* v, int64_t n) {
    for (int64_t i = 0; i < n; ++i) v[i] = iqo_fp_decode(kind, code[i]);
}
void iqo_int_encode_n(const float* v, int32_t* q, int64_t n, int qmax) {
    for (int64_t i = 0; i < n; ++i) q[i] = iqo_int_encode(v[i], qmax);
}

/* ---- descriptors --------------------------------------------------------- */
int64_t iqo_block_size(int fmt, int gran) {
    switch (fmt) {
    case IQO_INT8: case IQO_E4M3: case IQO_E5M2:
        return (gran == IQO_PER_TENSOR || gran == IQO_PER_ROW) ? 0 : -1; /* 0: whole row/tensor */
    case IQO_MXFP4: return gran == IQO_PER_BLOCK ? 32 : -1;
    case IQO_NVFP4: return gran == IQO_PER_BLOCK ? 16 : -1;
    case IQO_INT4:  return gran == IQO_PER_BLOCK ? 128 : -1;
    case IQO_INT4ZP: return gran == IQO_PER_BLOCK ? 128 : -1;
    default: return -1;
    }
}

int iqo_check(const iqo_desc* d) {
    if (!d) return -1;
    if (d->in_dtype != IQO_F32 && d->in_dtype != IQO_BF16) return -1;
    int64_t b = iqo_block_size(d->fmt, d->gran);
    if (b < 0) return -1;
    if (d->rows < 0 || d->cols < 0 || d->ld < d->cols) return -1;
    if (b > 0 && d->cols % b) return -1;
    if (d->fmt == IQO_INT4ZP && d->cols % 256) return -1; /* whole shift bytes per row */
    return 0;
}

static float load_x(const iqo_desc* d, const void* x, int64_t r, int64_t c) {
    int64_t i = r * d->ld + c;
    if (d->in_dtype == IQO_F32) return ((const float*)x)[i];
    return iqo_bf16_to_f32(((const uint16_t*)x)[i]);
}

/* max |x| over the finite elements of row r, columns [c0, c1). */
static float amax_span(const iqo_desc* d, const void* x, int64_t r, int64_t c0, int64_t c1) {
    float m = 0.0f;
    for (int64_t c = c0; c < c1; ++c) {
        float v = load_x(d, x, r, c);
        if (isfinite(v) && fabsf(v) > m) m = fabsf(v);
    }
    return m;
}

float iqo_amax(const iqo_desc* d, const void* x) {
    float m = 0.0f;
    for (int64_t r = 0; r < d->rows; ++r) {
        float a = amax_span(d, x, r, 0, d->cols);
        if (a > m) m = a;
    }
    return m;
}

/* ---- error statistics ([LP] error analysis: e = x - x^) ----------------- */
typedef struct {
    uint64_t n, n_zero_flush, n_saturated, n_nonfinite;
    double sum_x2, sum_err2, sum_abs_err;
    float max_abs_err;
} acc_t;

/* v is the scaled value x/s (0 when the scale is zero); qmax the largest
 * code magnitude of the grid, for the saturation count. */
static void acc_elem_sat(acc_t* a, float x, int saturated, float xh) {
    a->n++;
    if (saturated) a->n_saturated++;
    if (!isfinite(x)) { a->n_nonfinite++; return; }
    float d = x - xh; /* exact: x and x^ are within a factor 2 (Sterbenz) or x^ = 0 */
    a->sum_x2 += (double)x * (double)x;
    a->sum_err2 += (double)d * (double)d;
    a->sum_abs_err += fabs((double)d);
    if (fabsf(d) > a->max_abs_err) a->max_abs_err = fabsf(d);
    if (x != 0.0f && xh == 0.0f) a->n_zero_flush++;
}

static void acc_elem(acc_t* a, float x, float v, float xh, float qmax) {
    acc_elem_sat(a, x, fabsf(v) > qmax, xh);
}

static void acc_add(acc_t* t, const acc_t* a) {
    t->n += a->n; t->n_zero_flush += a->n_zero_flush; t->n_saturated += a->n_saturated;
    t->n_nonfinite += a->n_nonfinite;
    t->sum_x2 += a->sum_x2; t->sum_err2 += a->sum_err2; t->sum_abs_err += a->sum_abs_err;
    if (a->max_abs_err > t->max_abs_err) t->max_abs_err = a->max_abs_err;
}

static void put_nibble(uint8_t* row_codes, int64_t c, uint32_t nib) {
    uint8_t* p = &row_codes[c >> 1];
    if (c & 1) *p = (uint8_t)((*p & 0x0Fu) | ((nib & 0xFu) << 4));
    else       *p = (uint8_t)((*p & 0xF0u) | (nib & 0xFu));
}

/* ---- one row of each format --------------------------------------------- */

/* [LP] "FP8": INT8 x^ = s*round(x/s), s = alpha/127, q in [-127, 127];
 * FP8 with s = alpha/FMAX and the FP8 cast in place of round(). */
static void row_int8_fp8(const iqo_desc* d, const void* x, int64_t r, float alpha, uint8_t* codes,
                         float* scales, float* xhat, acc_t* a) {
    int is_int = d->fmt == IQO_INT8;
    int kind = d->fmt == IQO_E4M3 ? IQO_K_E4M3 : IQO_K_E5M2;
    float qmax = is_int ? 127.0f : (d->fmt == IQO_E4M3 ? 448.0f : 57344.0f);
    float s = alpha / qmax;
    if (d->gran == IQO_PER_ROW) scales[r] = s;
    uint8_t* rc = codes + r * d->cols;
    for (int64_t c = 0; c < d->cols; ++c) {
        float xv = load_x(d, x, r, c);
        float v = 0.0f, xh;
        if (s == 0.0f) {
            rc[c] = 0;
            xh = 0.0f;
        } else if (is_int) {
            v = xv / s;
            int q = iqo_int_encode(v, 127);
            rc[c] = (uint8_t)(int8_t)q;
            xh = s * (float)q;
        } else {
            v = xv / s;
            uint32_t code = iqo_fp_encode(kind, v);
            rc[c] = (uint8_t)code;
            xh = s * iqo_fp_decode(kind, code);
        }
        if (xhat) xhat[r * d->cols + c] = xh;
        acc_elem(a, xv, v, xh, qmax);
    }
}

/* [LP] "MXFP4": x^ = s_mx * Q_E2M1(x / s_mx), s_mx = 2^(E-127) per 32. */
static void row_mxfp4(const iqo_desc* d, const void* x, int64_t r, uint8_t* codes, uint8_t* scales,
                      float* xhat, acc_t* a) {
    int64_t nb = d->cols / 32;
    uint8_t* rc = codes + r * (d->cols / 2);
    for (int64_t b = 0; b < nb; ++b) {
        float A = amax_span(d, x, r, b * 32, b * 32 + 32);
        uint8_t E = iqo_e8m0_code(A, d->flags);
        scales[r * nb + b] = E;
        float s = iqo_e8m0_value(E);
        for (int64_t c = b * 32; c < b * 32 + 32; ++c) {
            float xv = load_x(d, x, r, c);
            float v = xv / s;
            uint32_t q = iqo_fp_encode(IQO_K_E2M1, v);
            put_nibble(rc, c, q);
            float xh = s * iqo_fp_decode(IQO_K_E2M1, q);
            if (xhat) xhat[r * d->cols + c] = xh;
            acc_elem(a, xv, v, xh, 6.0f);
        }
    }
}

/* NVFP4 block-scale code for t = (A_b/6)/s_g. */
static uint8_t nv_block_code(float t, uint32_t flags) {
    if (flags & IQO_FLAG_NV_SCALE_RNE) return (uint8_t)iqo_fp_encode(IQO_K_E4M3, t);
    return iqo_e4m3_ceil(t);
}

/* [LP] "NVFP4": s_global = gamax/(6*448); s_block = (bamax/6)/s_global cast to
 * E4M3; x^ = s_global*s_block*Q_E2M1(x/(s_global*s_block)), blocks of 16. */
static void row_nvfp4(const iqo_desc* d, const void* x, int64_t r, float s_g, uint8_t* codes,
                      uint8_t* scales, float* xhat, acc_t* a) {
    int64_t nb = d->cols / 16;
    uint8_t* rc = codes + r * (d->cols / 2);
    for (int64_t b = 0; b < nb; ++b) {
        uint8_t sb = 0;
        float s_nv = 0.0f;
        if (s_g != 0.0f) {
            float A = amax_span(d, x, r, b * 16, b * 16 + 16);
            float t = (A / 6.0f) / s_g;
            sb = nv_block_code(t, d->flags);
            s_nv = s_g * iqo_fp_decode(IQO_K_E4M3, sb);
        }
        scales[r * nb + b] = sb;
        for (int64_t c = b * 16; c < b * 16 + 16; ++c) {
            float xv = load_x(d, x, r, c);
            float v = 0.0f;
            uint32_t q = 0;
            if (s_nv != 0.0f) {
                v = xv / s_nv;
                q = iqo_fp_encode(IQO_K_E2M1, v);
            }
            put_nibble(rc, c, q);
            float xh = s_nv * iqo_fp_decode(IQO_K_E2M1, q);
            if (xhat) xhat[r * d->cols + c] = xh;
            acc_elem(a, xv, v, xh, 6.0f);
        }
    }
}

/* [LP] "INT4": symmetric q in [-7, 7], s = A/7, per group of 128; the scale
 * is stored as FP16 and the stored value is the one applied.  Codes are
 * two's-complement nibbles packed as [TR] Puzzle 12 extract() reads them. */
static void row_int4(const iqo_desc* d, const void* x, int64_t r, uint8_t* codes, uint16_t* scales,
                     float* xhat, acc_t* a) {
    int64_t ng = d->cols / 128;
    uint8_t* rc = codes + r * (d->cols / 2);
    for (int64_t g = 0; g < ng; ++g) {
        float A = amax_span(d, x, r, g * 128, g * 128 + 128);
        uint16_t s16 = (uint16_t)iqo_fp_encode(IQO_K_F16, A / 7.0f);
        scales[r * ng + g] = s16;
        float sf = iqo_fp_decode(IQO_K_F16, s16);
        for (int64_t c = g * 128; c < g * 128 + 128; ++c) {
            float xv = load_x(d, x, r, c);
            float v = 0.0f;
            int q = 0;
            if (sf != 0.0f) {
                v = xv / sf;
                q = iqo_int_encode(v, 7);
            }
            put_nibble(rc, c, (uint32_t)q & 0xFu);
            float xh = sf * (float)q;
            if (xhat) xhat[r * d->cols + c] = xh;
            acc_elem(a, xv, v, xh, 7.0f);
        }
    }
}

static void stats_out(iqo_stats* st, const acc_t* t) {
    st->n = t->n; st->n_zero_flush = t->n_zero_flush; st->n_saturated = t->n_saturated;
    st->n_nonfinite = t->n_nonfinite; st->sum_x2 = t->sum_x2; st->sum_err2 = t->sum_err2;
    st->sum_abs_err = t->sum_abs_err; st->max_abs_err = t->max_abs_err; st->reserved = 0;
}

/* [TR] Puzzle 12: asymmetric 4-bit codes.  The page gives the decoder
 * x^ = sc * (w - sh) (w, sh unsigned 4-bit, sc a float per group); the
 * encoder below is the min-max reading.  Over the group's finite elements,
 * lo = min(0, min x) and hi = max(0, max x), so 0 is on the grid;
 * sc = (hi - lo) / 15 in binary32 (clamped to the largest float if the
 * range overflows); sh = RNE(-lo / sc) clamped to [0, 15]; each element
 * takes q = RNE(x / sc) as the symmetric INT formats do and stores
 * w = clamp(q + sh, 0, 15).  sc == 0 gives w = sh = 0 and x^ = 0.  NaN
 * maps to w = sh (x^ = 0), +-Inf to 15 or 0.  Saturated: x/sc beyond the
 * grid's ends, above 15 - sh or below -sh. */
static uint8_t zp_code(float v, int sh) {
    if (isnan(v)) return (uint8_t)sh;
    double w = nearbyint((double)v) + (double)sh; /* v is finite or +-Inf */
    if (w < 0.0) w = 0.0;
    if (w > 15.0) w = 15.0;
    return (uint8_t)w;
}

static void row_int4zp(const iqo_desc* d, const void* x, int64_t r, uint8_t* codes, float* scales,
                       uint8_t* shifts, float* xhat, acc_t* a) {
    int64_t ng = d->cols / 128;
    uint8_t* rc = codes + r * (d->cols / 2);
    uint8_t* rs = shifts + r * (ng / 2);
    for (int64_t g = 0; g < ng; ++g) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t c = g * 128; c < g * 128 + 128; ++c) {
            float v = load_x(d, x, r, c);
            if (!isfinite(v)) continue;
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        float sc = (hi - lo) / 15.0f;
        if (isinf(sc)) sc = 3.40282347e38f; /* largest binary32 */
        int sh = 0;
        if (sc != 0.0f) {
            float z = nearbyintf(-lo / sc);
            sh = z < 0.0f ? 0 : (z > 15.0f ? 15 : (int)z);
        }
        scales[r * ng + g] = sc;
        put_nibble(rs, g, (uint32_t)sh);
        for (int64_t c = g * 128; c < g * 128 + 128; ++c) {
            float xv = load_x(d, x, r, c);
            float v = 0.0f;
            uint8_t w = (uint8_t)sh;
            if (sc != 0.0f) {
                v = xv / sc;
                w = zp_code(v, sh);
            }
            put_nibble(rc, c, w);
            float xh = sc * (float)((int)w - sh);
            if (xhat) xhat[r * d->cols + c] = xh;
            acc_elem_sat(a, xv, v > (float)(15 - sh) || v < (float)(-sh), xh);
        }
    }
}

int iqo_quantize_zp_rows(const iqo_desc* d, const void* x, int64_t r0, int64_t r1, uint8_t* codes,
                         float* scales, uint8_t* shifts, float* xhat, iqo_stats* st) {
    if (iqo_check(d) || d->fmt != IQO_INT4ZP || r0 < 0 || r1 > d->rows || r0 > r1) return -1;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    acc_t total;
    memset(&total, 0, sizeof total);
    for (int64_t r = r0; r < r1; ++r) {
        acc_t a;
        memset(&a, 0, sizeof a);
        row_int4zp(d, x, r, codes, scales, shifts, xhat, &a);
        acc_add(&total, &a);
    }
    if (st) stats_out(st, &total);
    return 0;
}

int iqo_dequantize_zp(const iqo_desc* d, const uint8_t* codes, const float* scales, const uint8_t* shifts,
                      void* xhat, int xhat_dtype) {
    if (iqo_check(d) || d->fmt != IQO_INT4ZP) return -1;
    if (xhat_dtype != IQO_F32 && xhat_dtype != IQO_BF16) return -1;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    int64_t ng = d->cols / 128;
    for (int64_t r = 0; r < d->rows; ++r) {
        for (int64_t c = 0; c < d->cols; ++c) {
            uint8_t byte = codes[r * (d->cols / 2) + c / 2];
            int w = (int)((c & 1) ? (byte >> 4) : (byte & 0xFu));
            int64_t g = c / 128;
            uint8_t sb = shifts[r * (ng / 2) + g / 2];
            int sh = (int)((g & 1) ? (sb >> 4) : (sb & 0xFu));
            float xh = scales[r * ng + g] * (float)(w - sh);
            if (xhat_dtype == IQO_F32) ((float*)xhat)[r * d->cols + c] = xh;
            else ((uint16_t*)xhat)[r * d->cols + c] = iqo_f32_to_bf16(xh);
        }
    }
    return 0;
}

int iqo_quantize_rows(const iqo_desc* d, const void* x, int64_t r0, int64_t r1, float tensor_amax,
                      uint8_t* codes, void* scales, float* global_scale, float* xhat, iqo_stats* st) {
    if (iqo_check(d) || d->fmt == IQO_INT4ZP || r0 < 0 || r1 > d->rows || r0 > r1) return -1;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    acc_t total;
    memset(&total, 0, sizeof total);
    float s_g = 0.0f;
    if (d->fmt == IQO_NVFP4) {
        s_g = tensor_amax / 2688.0f; /* 2688 = 6 * 448 */
        if (r0 == 0 && global_scale) *global_scale = s_g;
    }
    if (d->gran == IQO_PER_TENSOR && r0 == 0) {
        float qmax = d->fmt == IQO_INT8 ? 127.0f : (d->fmt == IQO_E4M3 ? 448.0f : 57344.0f);
        ((float*)scales)[0] = tensor_amax / qmax;
    }
    for (int64_t r = r0; r < r1; ++r) {
        acc_t a;
        memset(&a, 0, sizeof a);
        switch (d->fmt) {
        case IQO_INT8: case IQO_E4M3: case IQO_E5M2: {
            float alpha = d->gran == IQO_PER_TENSOR ? tensor_amax : amax_span(d, x, r, 0, d->cols);
            row_int8_fp8(d, x, r, alpha, codes, (float*)scales, xhat, &a);
            break;
        }
        case IQO_MXFP4: row_mxfp4(d, x, r, codes, (uint8_t*)scales, xhat, &a); break;
        case IQO_NVFP4: row_nvfp4(d, x, r, s_g, codes, (uint8_t*)scales, xhat, &a); break;
        case IQO_INT4:  row_int4(d, x, r, codes, (uint16_t*)scales, xhat, &a); break;
        }
        acc_add(&total, &a); /* rows summed in row order */
    }
    if (st) stats_out(st, &total);
    return 0;
}

int iqo_quantize(const iqo_desc* d, const void* x, uint8_t* codes, void* scales,
                 float* global_scale, float* xhat, iqo_stats* st) {
    if (iqo_check(d)) return -1;
    float amax = 0.0f;
    if (d->gran == IQO_PER_TENSOR || d->fmt == IQO_NVFP4) amax = iqo_amax(d, x);
    return iqo_quantize_rows(d, x, 0, d->rows, amax, codes, scales, global_scale, xhat, st);
}

/* ---- static scaling: the absmax of "FP8" / "NVFP4" supplied by the caller -- */
float iqo_static_amax(float amax_in) {
    if (!(amax_in >= 0.0f) || isinf(amax_in)) return 0.0f;
    return fabsf(amax_in);
}

int iqo_quantize_static(const iqo_desc* d, const void* x, float amax_in, uint8_t* codes, void* scales,
                        float* global_scale, float* xhat, iqo_stats* st) {
    if (iqo_check(d)) return -1;
    if (!(d->gran == IQO_PER_TENSOR || d->fmt == IQO_NVFP4)) return -1;
    return iqo_quantize_rows(d, x, 0, d->rows, iqo_static_amax(amax_in), codes, scales, global_scale, xhat, st);
}

/* ---- [TR] Puzzle 12: the dequantize-then-dot consumer -------------------- */
/* z[j, k] = sum_l sc * (w - sh) * y[l, k], written out: sc * (w - sh) has at
 * most 24 + 5 significant bits and y at most 24, so each product is exact in
 * binary64; the sum over l runs in order. */
int iqo_zp_gemm(const iqo_desc* d, const uint8_t* codes, const float* scales, const uint8_t* shifts,
                const void* x, int x_dtype, int64_t n1, double* z, double* zabs) {
    if (iqo_check(d) || d->fmt != IQO_INT4ZP || n1 < 0) return -1;
    if (x_dtype != IQO_F32 && x_dtype != IQO_BF16) return -1;
    const int64_t K = d->cols, ng = K / 128;
    for (int64_t j = 0; j < d->rows; ++j) {
        for (int64_t k = 0; k < n1; ++k) {
            double acc = 0.0, mag = 0.0;
            for (int64_t l = 0; l < K; ++l) {
                uint8_t byte = codes[j * (K / 2) + l / 2];
                int w = (int)((l & 1) ? (byte >> 4) : (byte & 0xFu));
                int64_t g = l / 128;
                uint8_t sb = shifts[j * (ng / 2) + g / 2];
                int sh = (int)((g & 1) ? (sb >> 4) : (sb & 0xFu));
                double y = x_dtype == IQO_F32 ? (double)((const float*)x)[k * K + l]
                                              : (double)iqo_bf16_to_f32(((const uint16_t*)x)[k * K + l]);
                double t = (double)scales[j * ng + g] * (double)(w - sh) * y;
                acc += t;
                mag += fabs(t);
            }
            z[j * n1 + k] = acc;
            if (zabs) zabs[j * n1 + k] = mag;
        }
    }
    return 0;
}

/* ---- FP4 GEMM over MXFP4 operands ---------------------------------------
 * [LP] "FP4 / MXFP4 / NVFP4": an MXFP4 value is its E2M1 code times the
 * block's power-of-two scale 2^(E - 127); a GEMM over two such operands
 * multiplies those values.  Written out as the definition: one binary64
 * product per k (exact: at most 2 significant bits each, exponents far
 * inside the binary64 range) and a binary64 sum in k order. */
static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t K, int64_t r, int64_t k) {
    uint8_t byte = codes[r * (K / 2) + k / 2];
    uint32_t q = (k & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 0xFu);
    return (double)iqo_e8m0_value(scales[r * (K / 32) + k / 32]) * (double)iqo_fp_decode(IQO_K_E2M1, q);
}

int iqo_mx_gemm(const iqo_desc* d, const uint8_t* codes_w, const uint8_t* scales_w, const uint8_t* codes_a,
                const uint8_t* scales_a, int64_t n1, double* z, double* zabs) {
    if (iqo_check(d) || d->fmt != IQO_MXFP4 || d->gran != IQO_PER_BLOCK || n1 < 0) return -1;
    const int64_t K = d->cols;
    for (int64_t j = 0; j < d->rows; ++j) {
        for (int64_t t = 0; t < n1; ++t) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double term = mx_value(codes_w, scales_w, K, j, k) * mx_value(codes_a, scales_a, K, t, k);
                acc += term;
                mag += fabs(term);
            }
            z[j * n1 + t] = acc;
            if (zabs) zabs[j * n1 + t] = mag;
        }
    }
    return 0;
}

/* The same weights against unquantized activations: one binary64 product
 * per k (the MXFP4 value has at most 2 significant bits, a BF16 or FP32
 * activation at most 24) and a binary64 sum in k order. */
int iqo_mxw_gemm(const iqo_desc* d, const uint8_t* codes_w, const uint8_t* scales_w, const void* x, int x_dtype,
                 int64_t n1, double* z, double* zabs) {
    if (iqo_check(d) || d->fmt != IQO_MXFP4 || d->gran != IQO_PER_BLOCK || n1 < 0) return -1;
    if (x_dtype != IQO_F32 && x_dtype != IQO_BF16) return -1;
    const int64_t K = d->cols;
    for (int64_t j = 0; j < d->rows; ++j) {
        for (int64_t t = 0; t < n1; ++t) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double y = x_dtype == IQO_F32 ? (double)((const float*)x)[t * K + k]
                                              : (double)iqo_bf16_to_f32(((const uint16_t*)x)[t * K + k]);
                double term = mx_value(codes_w, scales_w, K, j, k) * y;
                acc += term;
                mag += fabs(term);
            }
            z[j * n1 + t] = acc;
            if (zabs) zabs[j * n1 + t] = mag;
        }
    }
    return 0;
}

/* ---- dequantization: x^ = s * decode(q), the same products as above ----- */
int iqo_dequantize(const iqo_desc* d, const uint8_t* codes, const void* scales,
                   const float* global_scale, void* xhat, int xhat_dtype) {
    if (iqo_check(d) || d->fmt == IQO_INT4ZP) return -1;
    if (xhat_dtype != IQO_F32 && xhat_dtype != IQO_BF16) return -1;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    for (int64_t r = 0; r < d->rows; ++r) {
        for (int64_t c = 0; c < d->cols; ++c) {
            float xh = 0.0f;
            switch (d->fmt) {
            case IQO_INT8: case IQO_E4M3: case IQO_E5M2: {
                float s = ((const float*)scales)[d->gran == IQO_PER_TENSOR ? 0 : r];
                uint8_t q = codes[r * d->cols + c];
                if (s == 0.0f) xh = 0.0f;
                else if (d->fmt == IQO_INT8) xh = s * (float)(int8_t)q;
                else xh = s * iqo_fp_decode(d->fmt == IQO_E4M3 ? IQO_K_E4M3 : IQO_K_E5M2, q);
                break;
            }
            case IQO_MXFP4: case IQO_NVFP4: case IQO_INT4: {
                uint8_t byte = codes[r * (d->cols / 2) + c / 2];
                uint32_t nib = (c & 1) ? (byte >> 4) : (byte & 0xFu);
                if (d->fmt == IQO_MXFP4) {
                    float s = iqo_e8m0_value(((const uint8_t*)scales)[r * (d->cols / 32) + c / 32]);
                    xh = s * iqo_fp_decode(IQO_K_E2M1, nib);
                } else if (d->fmt == IQO_NVFP4) {
                    uint8_t sb = ((const uint8_t*)scales)[r * (d->cols / 16) + c / 16];
                    float s_nv = global_scale[0] * iqo_fp_decode(IQO_K_E4M3, sb);
                    xh = s_nv * iqo_fp_decode(IQO_K_E2M1, nib);
                } else {
                    float sf = iqo_fp_decode(IQO_K_F16, ((const uint16_t*)scales)[r * (d->cols / 128) + c / 128]);
                    int q = (int)(nib & 7u) - (int)(nib & 8u); /* two's-complement nibble */
                    xh = sf * (float)q;
                }
                break;
            }
            }
            if (xhat_dtype == IQO_F32) ((float*)xhat)[r * d->cols + c] = xh;
            else ((uint16_t*)xhat)[r * d->cols + c] = iqo_f32_to_bf16(xh);
        }
    }
    return 0;
}
