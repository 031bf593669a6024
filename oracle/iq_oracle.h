/*
 * iq_oracle.h -- CPU oracle for block-scaled low-precision quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's
 * cpu_baseline leg may load or call this code.  It shares no source, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Every floating-point operation is one IEEE-754 binary32 (or binary64 where
 * stated) operation, round-to-nearest-even, no contraction into FMA, no
 * fast-math.  Built with gcc -O2 -ffp-contract=off on x86-64 (SSE arithmetic).
 *
 * Parity unpinned (no value on the pages fixes them; the oracle's own reading
 * is the only reference):
 *   - the code chosen for NaN inputs (0x7F for FP8, +0 for E2M1 and INT);
 *   - the sign kept on codes that round to zero (-0 -> 0x80 / 0x8);
 *   - statistics over non-finite inputs (excluded from sums and maxima).
 */
#ifndef IQ_ORACLE_H
#define IQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantized formats. */
enum { IQO_INT8 = 0, IQO_E4M3 = 1, IQO_E5M2 = 2, IQO_MXFP4 = 3, IQO_NVFP4 = 4, IQO_INT4 = 5,
       IQO_INT4ZP = 6 /* unsigned 4-bit codes, per-group scale and 4-bit shift (Puzzle 12) */ };
/* Scale granularity. */
enum { IQO_PER_TENSOR = 0, IQO_PER_ROW = 1, IQO_PER_BLOCK = 2 };
/* Element types of inputs and dequantized outputs. */
enum { IQO_F32 = 0, IQO_BF16 = 1 };
/* Minifloat kinds understood by iqo_fp_encode / iqo_fp_decode. */
enum { IQO_K_E4M3 = 0, IQO_K_E5M2 = 1, IQO_K_E2M1 = 2, IQO_K_F16 = 3 };

/* Optional rule variants (flags); 0 selects the default readings. */
#define IQO_FLAG_MX_ROUND_NEAREST 0x1u /* E8M0 = 2^round(log2(A/6)) */
#define IQO_FLAG_MX_ROUND_UP      0x2u /* E8M0 = 2^ceil(log2(A/6))  */
#define IQO_FLAG_NV_SCALE_RNE     0x4u /* NVFP4 block scale by RNE instead of ceil */

typedef struct {
    int fmt, gran, in_dtype;
    int64_t rows, cols, ld; /* ld = row stride of x in elements */
    uint32_t flags;
} iqo_desc;

/* n counts every element; the sums, the maximum and n_zero_flush cover the
 * finite inputs only.  MSE = sum_err2 / (n - n_nonfinite). */
typedef struct {
    uint64_t n, n_zero_flush, n_saturated, n_nonfinite;
    double sum_x2, sum_err2, sum_abs_err;
    float max_abs_err;
    uint32_t reserved;
} iqo_stats;

/* --- scalar codecs ------------------------------------------------------ */
float    iqo_bf16_to_f32(uint16_t b);
uint16_t iqo_f32_to_bf16(float f);
uint32_t iqo_fp_encode(int kind, float v);   /* saturating round-to-nearest-even */
float    iqo_fp_decode(int kind, uint32_t code);
int      iqo_int_encode(float v, int qmax);  /* clamp(round-half-even(v), -qmax, qmax); NaN -> 0 */
uint8_t  iqo_e8m0_code(float A, uint32_t flags);
float    iqo_e8m0_value(uint8_t code);
uint8_t  iqo_e4m3_ceil(float t);             /* smallest E4M3 value >= t, capped at 448 */
/* Array forms of the codecs above (element-wise, for exhaustive tests). */
void     iqo_fp_encode_n(int kind, const float* v, uint32_t* code, int64_t n);
void     iqo_fp_decode_n(int kind, const uint32_t* code, float* v, int64_t n);
void     iqo_int_encode_n(const float* v, int32_t* q, int64_t n, int qmax);

/* --- tensor-level ------------------------------------------------------- */
int64_t iqo_block_size(int fmt, int gran);   /* elements per scale along a row, -1 if invalid */
int     iqo_check(const iqo_desc* d);        /* 0 if the descriptor is a legal combination */
float   iqo_amax(const iqo_desc* d, const void* x); /* max |x| over finite elements */

/* Quantize rows [r0, r1).  x, codes, scales, xhat address the full tensors.
 * tensor_amax is used by per-tensor formats and NVFP4 (the global absmax).
 * Per-tensor scales and the NVFP4 global scale are written only when r0 == 0.
 * xhat (FP32, [rows, cols]) and st may be NULL. */
int iqo_quantize_rows(const iqo_desc* d, const void* x, int64_t r0, int64_t r1, float tensor_amax,
                      uint8_t* codes, void* scales, float* global_scale, float* xhat, iqo_stats* st);
/* Whole tensor: absmax pre-pass when needed, then every row in order. */
int iqo_quantize(const iqo_desc* d, const void* x, uint8_t* codes, void* scales,
                 float* global_scale, float* xhat, iqo_stats* st);
/* Static (calibrated) scaling: the per-tensor absmax is the caller's value,
 * taken as 0 when it is NaN, negative or infinite (and -0 as +0). */
float iqo_static_amax(float amax_in);
/* Whole tensor with a caller-supplied absmax (per-tensor formats, NVFP4). */
int iqo_quantize_static(const iqo_desc* d, const void* x, float amax_in, uint8_t* codes, void* scales,
                        float* global_scale, float* xhat, iqo_stats* st);
/* Asymmetric INT4 (IQO_INT4ZP, per block of 128; cols a multiple of 256):
 * codes [rows, cols/2] unsigned nibbles, scales float [rows, cols/128],
 * shifts [rows, cols/256] bytes, group 2t in bits 3:0.  Rows [r0, r1). */
int iqo_quantize_zp_rows(const iqo_desc* d, const void* x, int64_t r0, int64_t r1, uint8_t* codes,
                         float* scales, uint8_t* shifts, float* xhat, iqo_stats* st);
int iqo_dequantize_zp(const iqo_desc* d, const uint8_t* codes, const float* scales, const uint8_t* shifts,
                      void* xhat, int xhat_dtype);
/* [TR] Puzzle 12: z[j, k] = sum_l sc[j, l/128] * (w[j, l] - sh[j, l/128]) * y[l, k]
 * for the asymmetric INT4 weights of d (rows N0 = d->rows, K = d->cols) and
 * activations given token-major, y[l, k] = x[k * K + l] (x: n1 rows of K,
 * FP32 or BF16 by x_dtype).  Every product is exact in binary64 and the sum
 * runs in l order in binary64; z and zabs (the sum of |terms|, the scale of
 * any rounding bound) are [N0, n1] row-major. */
int iqo_zp_gemm(const iqo_desc* d, const uint8_t* codes, const float* scales, const uint8_t* shifts,
                const void* x, int x_dtype, int64_t n1, double* z, double* zabs);
/* [LP] FP4 GEMM over two MXFP4 operands: z[j, t] = sum_k xw[j, k] * xa[t, k]
 * with x = 2^(E - 127) * e2m1(code) the dequantized values of the weights
 * (rows N0 = d->rows, K = d->cols, codes [N0, K/2], E8M0 scales [N0, K/32])
 * and of the activations (codes [n1, K/2], scales [n1, K/32]).  Every
 * product is exact in binary64 and the sum runs in k order in binary64; z
 * and zabs (the sum of |terms|) are [N0, n1] row-major. */
int iqo_mx_gemm(const iqo_desc* d, const uint8_t* codes_w, const uint8_t* scales_w, const uint8_t* codes_a,
                const uint8_t* scales_a, int64_t n1, double* z, double* zabs);
/* [LP] MXFP4 weights against activations kept in BF16 or FP32:
 * z[j, t] = sum_k xw[j, k] * y[t, k] with xw the dequantized weights of d
 * (as for iqo_mx_gemm) and y token-major [n1, K] (x_dtype IQO_F32 or
 * IQO_BF16).  Exact binary64 products, binary64 sum in k order; z and zabs
 * [N0, n1] row-major. */
int iqo_mxw_gemm(const iqo_desc* d, const uint8_t* codes_w, const uint8_t* scales_w, const void* x, int x_dtype,
                 int64_t n1, double* z, double* zabs);
/* Reconstruct xhat ([rows, cols], FP32 or BF16) from codes and scales. */
int iqo_dequantize(const iqo_desc* d, const uint8_t* codes, const void* scales,
                   const float* global_scale, void* xhat, int xhat_dtype);

#ifdef __cplusplus
}
#endif
#endif
