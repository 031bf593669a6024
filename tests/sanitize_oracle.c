/*
 * Drives every entry point of the CPU oracle (oracle/iq_oracle.c) over small
 * tensors whose buffers are allocated to their exact sizes, with finite,
 * special (NaN, +-Inf, subnormal, +-0, huge) and all-zero rows, every legal
 * format / granularity / flag combination and both input types.  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (float-cast-overflow
 * included): any read or write outside a buffer, any use of uninitialized
 * heap through a sanitizer-visible path, any signed overflow, bad shift or
 * out-of-range float-to-int conversion aborts the run.
 *
 * Test infrastructure: this file is compiled only by the CPU test suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/iq_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {   /* xorshift64* (Vigna 2016) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* One value of the mixture: row kind 0 finite spread over exponents,
 * 1 with specials sprinkled in, 2 all zeros, 3 tiny (subnormal) values,
 * 4 huge values near FLT_MAX. */
static float draw(int kind) {
    const uint64_t r = next_u64();
    const float sign = (r & 1) ? -1.f : 1.f;
    const float mag = ldexpf((float)((r >> 8) & 0xFFFFFF) / 16777216.f + 0.5f, (int)((r >> 40) % 24) - 12);
    switch (kind) {
    case 0: return sign * mag;
    case 1: {
        const uint32_t pick = (uint32_t)((r >> 32) % 16);
        if (pick == 0) return NAN;
        if (pick == 1) return sign * INFINITY;
        if (pick == 2) return sign * 0.f;
        if (pick == 3) return f_from_bits((uint32_t)(r >> 41) | (r & 1 ? 0x80000000u : 0u));   /* subnormal */
        return sign * mag;
    }
    case 2: return (r & 1) ? -0.f : 0.f;
    case 3: return f_from_bits((uint32_t)(r >> 42) + 1u) * sign;
    default: return sign * ldexpf(1.f + (float)((r >> 20) & 0xFFFF) / 65536.f, 126 - (int)((r >> 50) % 3));
    }
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* x with rows of the given kinds, stored row-major with stride ld, in
 * exactly (rows - 1) * ld + cols elements. */
static void* make_x(int dtype, int64_t rows, int64_t cols, int64_t ld, int salt) {
    const int64_t n = rows ? (rows - 1) * ld + cols : 0;
    const size_t es = dtype == IQO_F32 ? 4 : 2;
    uint8_t* x = (uint8_t*)xmalloc((size_t)n * es);
    memset(x, 0x7F, (size_t)n * es);   /* the gaps between rows hold NaN patterns */
    for (int64_t r = 0; r < rows; ++r) {
        const int kind = (int)((r + salt) % 5);
        for (int64_t c = 0; c < cols; ++c) {
            const float v = draw(kind);
            if (dtype == IQO_F32) memcpy(x + (size_t)(r * ld + c) * 4, &v, 4);
            else {
                const uint16_t b = iqo_f32_to_bf16(v);
                memcpy(x + (size_t)(r * ld + c) * 2, &b, 2);
            }
        }
    }
    return x;
}

static size_t scales_bytes(const iqo_desc* d) {
    switch (d->fmt) {
    case IQO_INT8: case IQO_E4M3: case IQO_E5M2:
        return d->gran == IQO_PER_TENSOR ? 4 : (size_t)d->rows * 4;
    case IQO_MXFP4: return (size_t)(d->rows * (d->cols / 32));
    case IQO_NVFP4: return (size_t)(d->rows * (d->cols / 16));
    case IQO_INT4ZP: return (size_t)(d->rows * (d->cols / 128)) * 4;
    default: return (size_t)(d->rows * (d->cols / 128)) * 2;
    }
}

static int four_bit(int fmt) { return fmt == IQO_MXFP4 || fmt == IQO_NVFP4 || fmt == IQO_INT4 || fmt == IQO_INT4ZP; }

static long n_calls = 0;
static void expect_ok(int rc, const char* what, const iqo_desc* d) {
    ++n_calls;
    if (rc != 0) {
        fprintf(stderr, "%s failed (fmt %d gran %d dtype %d rows %lld cols %lld)\n", what, d->fmt, d->gran,
                d->in_dtype, (long long)d->rows, (long long)d->cols);
        exit(1);
    }
}

static void run_case(int fmt, int gran, int dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags, int salt) {
    iqo_desc d = {fmt, gran, dtype, rows, cols, ld, flags};
    if (iqo_check(&d) != 0) { fprintf(stderr, "illegal descriptor in the case list\n"); exit(1); }
    void* x = make_x(dtype, rows, cols, ld, salt);
    const size_t ncodes = (size_t)(rows * (four_bit(fmt) ? cols / 2 : cols));
    uint8_t* codes = (uint8_t*)xmalloc(ncodes);
    void* scales = xmalloc(scales_bytes(&d));
    float* gs = (float*)xmalloc(4);
    float* xhat = (float*)xmalloc((size_t)(rows * cols) * 4);
    uint16_t* xhat16 = (uint16_t*)xmalloc((size_t)(rows * cols) * 2);
    iqo_stats st;
    if (fmt == IQO_INT4ZP) {
        uint8_t* shifts = (uint8_t*)xmalloc((size_t)(rows * (cols / 256)));
        expect_ok(iqo_quantize_zp_rows(&d, x, 0, rows, codes, (float*)scales, shifts, xhat, &st), "zp quantize", &d);
        expect_ok(iqo_quantize_zp_rows(&d, x, 0, rows, codes, (float*)scales, shifts, NULL, NULL), "zp quantize", &d);
        expect_ok(iqo_dequantize_zp(&d, codes, (const float*)scales, shifts, xhat, IQO_F32), "zp dequantize", &d);
        expect_ok(iqo_dequantize_zp(&d, codes, (const float*)scales, shifts, xhat16, IQO_BF16), "zp dequantize", &d);
        /* Puzzle 12's consumer over these weights, 3 tokens */
        const int64_t n1 = 3;
        void* y = make_x(dtype, n1, cols, cols, salt + 1);
        double* z = (double*)xmalloc((size_t)(rows * n1) * 8);
        double* za = (double*)xmalloc((size_t)(rows * n1) * 8);
        expect_ok(iqo_zp_gemm(&d, codes, (const float*)scales, shifts, y, dtype, n1, z, za), "zp gemm", &d);
        free(y); free(z); free(za); free(shifts);
    } else {
        expect_ok(iqo_quantize(&d, x, codes, scales, gs, xhat, &st), "quantize", &d);
        expect_ok(iqo_quantize(&d, x, codes, scales, gs, NULL, NULL), "quantize", &d);
        expect_ok(iqo_dequantize(&d, codes, scales, gs, xhat, IQO_F32), "dequantize", &d);
        expect_ok(iqo_dequantize(&d, codes, scales, gs, xhat16, IQO_BF16), "dequantize", &d);
        if (rows > 1)   /* a row range that starts past row 0 */
            expect_ok(iqo_quantize_rows(&d, x, 1, rows, iqo_amax(&d, x), codes, scales, gs, xhat, &st), "rows", &d);
        if (gran == IQO_PER_TENSOR || fmt == IQO_NVFP4) {
            const float amaxes[] = {NAN, -1.f, INFINITY, -0.f, 0.f, 1e-30f, 3.0f, 3e38f};
            for (size_t k = 0; k < sizeof(amaxes) / sizeof(amaxes[0]); ++k)
                expect_ok(iqo_quantize_static(&d, x, amaxes[k], codes, scales, gs, xhat, &st), "static", &d);
        }
        if (fmt == IQO_MXFP4) {   /* FP4 GEMMs over these codes as weights and as activations */
            const int64_t n1 = rows;
            double* z = (double*)xmalloc((size_t)(rows * n1) * 8);
            double* za = (double*)xmalloc((size_t)(rows * n1) * 8);
            expect_ok(iqo_mx_gemm(&d, codes, (const uint8_t*)scales, codes, (const uint8_t*)scales, n1, z, za),
                      "mx gemm", &d);
            void* y = make_x(dtype, n1, cols, cols, salt + 2);
            expect_ok(iqo_mxw_gemm(&d, codes, (const uint8_t*)scales, y, dtype, n1, z, za), "mxw gemm", &d);
            free(y); free(z); free(za);
        }
    }
    free(x); free(codes); free(scales); free(gs); free(xhat); free(xhat16);
}

static void codecs(void) {
    /* every binary32 pattern with a stride, through every scalar codec */
    const int kinds[] = {IQO_K_E4M3, IQO_K_E5M2, IQO_K_E2M1, IQO_K_F16};
    for (uint64_t u = 0; u <= 0xFFFFFFFFull; u += 4099) {
        const float v = f_from_bits((uint32_t)u);
        for (int k = 0; k < 4; ++k) (void)iqo_fp_decode(kinds[k], iqo_fp_encode(kinds[k], v));
        (void)iqo_int_encode(v, 127);
        (void)iqo_int_encode(v, 7);
        (void)iqo_e8m0_code(v, 0);
        (void)iqo_e8m0_code(v, IQO_FLAG_MX_ROUND_NEAREST);
        (void)iqo_e8m0_code(v, IQO_FLAG_MX_ROUND_UP);
        (void)iqo_e4m3_ceil(v);
        (void)iqo_static_amax(v);
        (void)iqo_bf16_to_f32(iqo_f32_to_bf16(v));
    }
    for (int c = 0; c < 256; ++c) {
        (void)iqo_e8m0_value((uint8_t)c);
        for (int k = 0; k < 4; ++k) (void)iqo_fp_decode(kinds[k], (uint32_t)c);
    }
    for (uint32_t c = 0; c < 65536; ++c) (void)iqo_fp_decode(IQO_K_F16, c);
    /* array forms with exact-size buffers */
    const int64_t n = 1000;
    float* v = (float*)xmalloc(n * 4);
    uint32_t* code = (uint32_t*)xmalloc(n * 4);
    int32_t* q = (int32_t*)xmalloc(n * 4);
    for (int64_t i = 0; i < n; ++i) v[i] = draw((int)(i % 5));
    for (int k = 0; k < 4; ++k) {
        iqo_fp_encode_n(kinds[k], v, code, n);
        iqo_fp_decode_n(kinds[k], code, v, n);
    }
    iqo_int_encode_n(v, q, n, 127);
    free(v); free(code); free(q);
}

int main(void) {
    codecs();
    const int dtypes[] = {IQO_F32, IQO_BF16};
    for (int t = 0; t < 2; ++t) {
        const int dt = dtypes[t];
        int salt = 0;
        for (int fmt = IQO_INT8; fmt <= IQO_E5M2; ++fmt)
            for (int gran = IQO_PER_TENSOR; gran <= IQO_PER_ROW; ++gran) {
                run_case(fmt, gran, dt, 7, 40, 40, 0, salt++);
                run_case(fmt, gran, dt, 5, 24, 40, 0, salt++);    /* row stride beyond cols */
                run_case(fmt, gran, dt, 1, 8, 8, 0, salt++);
                run_case(fmt, gran, dt, 0, 16, 16, 0, salt++);    /* empty */
            }
        const uint32_t mx_flags[] = {0, IQO_FLAG_MX_ROUND_NEAREST, IQO_FLAG_MX_ROUND_UP};
        for (int k = 0; k < 3; ++k) {
            run_case(IQO_MXFP4, IQO_PER_BLOCK, dt, 6, 128, 128, mx_flags[k], salt++);
            run_case(IQO_MXFP4, IQO_PER_BLOCK, dt, 5, 96, 104, mx_flags[k], salt++);
        }
        const uint32_t nv_flags[] = {0, IQO_FLAG_NV_SCALE_RNE};
        for (int k = 0; k < 2; ++k) {
            run_case(IQO_NVFP4, IQO_PER_BLOCK, dt, 6, 64, 64, nv_flags[k], salt++);
            run_case(IQO_NVFP4, IQO_PER_BLOCK, dt, 5, 48, 56, nv_flags[k], salt++);
            run_case(IQO_NVFP4, IQO_PER_BLOCK, dt, 0, 32, 32, nv_flags[k], salt++);
        }
        run_case(IQO_INT4, IQO_PER_BLOCK, dt, 6, 256, 256, 0, salt++);
        run_case(IQO_INT4, IQO_PER_BLOCK, dt, 5, 384, 392, 0, salt++);
        run_case(IQO_INT4ZP, IQO_PER_BLOCK, dt, 6, 256, 256, 0, salt++);
        run_case(IQO_INT4ZP, IQO_PER_BLOCK, dt, 5, 512, 520, 0, salt++);
    }
    printf("ok %ld calls\n", n_calls);
    return 0;
}
