/*
 * iq.h -- C ABI of libiq, block-scaled low-precision quantization on MI355X.
 *
 * The method (Lorn blog, post "浅谈低精度浮点数", sections "FP8" and
 * "FP4 / MXFP4 / NVFP4"): a tensor x is represented as x^ = s * Q(x / s),
 * where s is a scale derived from an absolute maximum (per tensor, per row,
 * or per block along the contiguous dimension) and Q rounds onto a small
 * code grid.  One call reads x once and, in the same pass, derives the
 * scales, casts with saturating round-to-nearest-even, packs codes and
 * scales, dequantizes in registers and reduces error statistics.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, codes, scales, global_scale, stats, xhat, workspace,
 *   amax_in and amax_out are DEVICE pointers (HIP device memory of the current
 *   device).  The descriptor is a HOST pointer.  The caller allocates and
 *   owns every buffer; the library allocates nothing and never
 *   synchronizes.  Between calls it keeps only a cache of occupancy queries
 *   per kernel and device (host memory, guarded by a mutex), and the
 *   workspace tickets it leaves at zero.
 * - All work is enqueued on `stream` (0 = the null stream).  Functions
 *   return before the GPU finishes; outputs are valid after the caller
 *   synchronizes with the stream.
 * - Arguments are validated on the host before anything is enqueued.  On
 *   any error nothing is enqueued and no output is touched.
 * - x is row-major [rows, cols] with a row stride of ld_in >= cols elements.
 *   The base address must be 16-byte aligned and ld_in * sizeof(element) a
 *   multiple of 16.  codes, scales and xhat are dense row-major and 16-byte
 *   aligned; workspace is 256-byte aligned.
 * - rows == 0 or cols == 0 is legal: no codes or scales are written and the
 *   statistics (if requested) are written as zeros.
 *
 * Code and scale layouts (element (r, c); K = cols):
 *   INT8        codes  int8  [rows, K]   (two's complement, q in [-127, 127])
 *   FP8 E4M3/E5M2 codes uint8 [rows, K]  (OCP E4M3: max 448, NaN 0x7F;
 *                                         OCP E5M2: max 57344)
 *   MXFP4       codes  uint8 [rows, K/2]  E2M1 nibbles; scales uint8 E8M0 [rows, K/32]
 *   NVFP4       codes  uint8 [rows, K/2]  E2M1 nibbles; scales uint8 E4M3 [rows, K/16];
 *               global_scale float32 [1]
 *   INT4        codes  uint8 [rows, K/2]  two's-complement nibbles, q in [-7, 7];
 *               scales float16 bits [rows, K/128]
 *   INT4_ZP     codes  uint8 [rows, K/2]  unsigned nibbles w in [0, 15];
 *               scales float32 [rows, K/128]; shifts uint8 [rows, K/256]
 *               (4-bit sh, group 2t in bits 3:0); K a multiple of 256
 *   INT8 / FP8 scales: float32 [1] per tensor, float32 [rows] per row.
 *   4-bit codes: element 2t in bits 3:0 of byte t, element 2t+1 in bits 7:4
 *   (the order of the packed-word extract() of the Triton post, Puzzle 12).
 */
#ifndef IQ_H
#define IQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IQ_ABI_VERSION 2

typedef enum {
    IQ_OK = 0,
    IQ_EINVAL = 1,       /* NULL required pointer, bad enum, bad shape, cols not a multiple of the block */
    IQ_EALIGN = 2,       /* a pointer or the row stride breaks the alignment rules above */
    IQ_EUNSUPPORTED = 3, /* legal but not supported: unknown flags, sizes beyond 2^31 chunks */
    IQ_EHIP = 4          /* the HIP runtime reported an error when launching */
} iq_status;

typedef enum {
    IQ_INT8 = 0,     /* symmetric, s = alpha / 127 ("FP8" section, INT8 quantizer) */
    IQ_FP8_E4M3 = 1, /* s = alpha / 448 */
    IQ_FP8_E5M2 = 2, /* s = alpha / 57344 */
    IQ_MXFP4 = 3,    /* E2M1 codes, one E8M0 scale per 32 elements ("MXFP4") */
    IQ_NVFP4 = 4,    /* E2M1 codes, one E4M3 scale per 16 + FP32 global scale ("NVFP4") */
    IQ_INT4 = 5,     /* symmetric, s = A / 7 per group of 128, FP16 scale ("INT4") */
    IQ_INT4_ZP = 6   /* asymmetric: unsigned codes, FP32 scale + 4-bit shift per group of 128
                        (Triton post, Puzzle 12); only through iq_quantize_zp / iq_dequantize_zp */
} iq_format;

typedef enum { IQ_F32 = 0, IQ_BF16 = 1 } iq_dtype;

typedef enum {
    IQ_PER_TENSOR = 0, /* INT8 / FP8 */
    IQ_PER_ROW = 1,    /* INT8 / FP8 */
    IQ_PER_BLOCK = 2   /* MXFP4 (32), NVFP4 (16), INT4 and INT4_ZP (128): the only legal choice for those */
} iq_gran;

/* Rule variants (iq_desc.flags); 0 selects the default readings. */
#define IQ_FLAG_MX_ROUND_NEAREST 0x1u /* MXFP4: E8M0 = 2^round(log2(A/6)) instead of 2^(floor(log2 A)-2) */
#define IQ_FLAG_MX_ROUND_UP 0x2u      /* MXFP4: E8M0 = 2^ceil(log2(A/6)) */
#define IQ_FLAG_NV_SCALE_RNE 0x4u     /* NVFP4: block scale to E4M3 by RNE instead of rounding up */

typedef struct {
    int32_t fmt;      /* iq_format */
    int32_t gran;     /* iq_gran */
    int32_t in_dtype; /* iq_dtype of x */
    int32_t reserved0;
    int64_t rows, cols;
    int64_t ld_in;    /* row stride of x, in elements */
    uint32_t flags;
    uint32_t reserved1;
} iq_desc;

/* Error statistics of one iq_quantize call, written to device memory.
 * n counts every element; sums, max_abs_err and n_zero_flush cover the
 * finite inputs.  d = x - x^ (exact in FP32).  MSE = sum_err2 / (n - n_nonfinite).
 *   n_saturated   elements with |x/s| above the grid's largest value
 *   n_zero_flush  finite x != 0 whose x^ is 0 */
typedef struct {
    uint64_t n, n_zero_flush, n_saturated, n_nonfinite;
    double sum_x2, sum_err2, sum_abs_err;
    float max_abs_err;
    uint32_t reserved;
} iq_stats;

/* Bytes of the codes / scales arrays for a descriptor (0 on an invalid one). */
size_t iq_codes_bytes(const iq_desc* d);
size_t iq_scales_bytes(const iq_desc* d);
/* Bytes of device workspace iq_quantize / iq_amax need (>= 256). */
size_t iq_workspace_bytes(const iq_desc* d);

/*
 * Quantize x (the whole hot path).  Sections "FP8" (x^ = s * round(x / s),
 * s = alpha / 127; FP8 with its own grid) and "FP4 / MXFP4 / NVFP4"
 * (MXFP4 x^ = s_mx * Q(x / s_mx); NVFP4 s_global = amax / (6 * 448),
 * s_block = (block_amax / 6) / s_global; INT4 s = A / 7).
 *   codes, scales    outputs, layouts above (required)
 *   global_scale     NVFP4 output s_global (required for NVFP4, else ignored)
 *   stats            optional output (NULL skips the statistics)
 *   xhat             optional dequantized output [rows, cols] of xhat_dtype
 *   workspace        iq_workspace_bytes(d) bytes of device scratch, zero-filled
 *                    before its first use (e.g. hipMemset once, or torch.zeros);
 *                    every call leaves it ready for the next one.  The
 *                    workgroups of a call count themselves on it to decide
 *                    which one folds the partial statistics, and the absmax
 *                    pre-pass leaves its per-workgroup maxima there for the
 *                    cast, so concurrent calls need separate workspaces
 */
iq_status iq_quantize(const iq_desc* d, const void* x, void* codes, void* scales,
                      float* global_scale, iq_stats* stats, void* xhat, int32_t xhat_dtype,
                      void* workspace, hipStream_t stream);

/*
 * iq_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments and results, with the library's own
 * workspace in place of the caller's.
 *   The workspace is one device array per GPU of 128 KiB (IQ_NOALLOC_SCRATCH_BYTES),
 *   zero-filled when the library loads and held until the process ends; the
 *   call rejects a descriptor whose workspace would not fit it
 *   (IQ_EUNSUPPORTED; every descriptor iq_quantize accepts fits).
 *   No hipMalloc, hipFree or other allocating call is made.  The first call
 *   on a device resolves the array's address on that device (make one call
 *   before capturing a graph); a failure to resolve it returns IQ_EHIP.
 *   Every call on a GPU shares that GPU's array, and each call leaves it
 *   ready for the next: calls that may overlap on one GPU (other streams,
 *   other host threads) race and must be serialized by the caller.
 */
#define IQ_NOALLOC_SCRATCH_BYTES (128u * 1024u)
iq_status iq_quantize_noalloc(const iq_desc* d, const void* x, void* codes, void* scales,
                              float* global_scale, iq_stats* stats, void* xhat, int32_t xhat_dtype,
                              hipStream_t stream);

/*
 * Dequantize: x^ = s * decode(q), bit-identical to the x^ of iq_quantize.
 * Sections "FP8" (x^ = s * round(x / s): the code's value times the scale)
 * and "FP4 / MXFP4 / NVFP4" (MXFP4: E2M1 value times 2^(E - 127); NVFP4:
 * E2M1 value times s_global times the E4M3 block scale; INT4: q times the
 * FP16 group scale).
 * d->in_dtype and d->ld_in are ignored; xhat is dense [rows, cols] of
 * xhat_dtype (BF16 output is the FP32 x^ rounded to nearest even).
 * No workspace.  Errors as for iq_quantize.
 */
iq_status iq_dequantize(const iq_desc* d, const void* codes, const void* scales,
                        const float* global_scale, void* xhat, int32_t xhat_dtype,
                        hipStream_t stream);

/*
 * Per-tensor absmax over the finite elements of x (the per-tensor "alpha"
 * of section "FP8", the global amax of NVFP4), written to amax_out (device
 * float32 [1]).  Only d->in_dtype, rows, cols and ld_in are used.  The
 * workspace rules are those of iq_quantize (zero-filled before first use).
 */
iq_status iq_amax(const iq_desc* d, const void* x, float* amax_out, void* workspace,
                  hipStream_t stream);

/*
 * Static (calibrated) scaling: iq_quantize with the per-tensor absmax taken
 * from *amax_in (device float32 [1], e.g. written by iq_amax over
 * calibration data) instead of measured, so x is read once.  The scale is
 * derived from it exactly as iq_quantize derives it from the measured one
 * (section "FP8": s = alpha / FMAX; "NVFP4": s_global = amax / (6 * 448)).
 *   Legal for INT8 / E4M3 / E5M2 per tensor and for NVFP4 (the global
 *   scale; block scales still come from each block).  Any other
 *   descriptor returns IQ_EINVAL.
 *   Elements beyond alpha saturate and are counted in n_saturated; NaN and
 *   +-Inf inputs are handled as in iq_quantize.
 *   A NaN, negative or infinite *amax_in is taken as 0 (every code +0,
 *   scale 0); -0 is taken as +0.
 *   The other arguments, layouts, workspace rules and errors are those of
 *   iq_quantize; amax_in must be 4-byte aligned (IQ_EALIGN otherwise).
 */
iq_status iq_quantize_static(const iq_desc* d, const void* x, const float* amax_in, void* codes,
                             void* scales, float* global_scale, iq_stats* stats, void* xhat,
                             int32_t xhat_dtype, void* workspace, hipStream_t stream);

/*
 * Asymmetric INT4, the format of the Triton post's Puzzle 12 ("Quantized
 * Matrix Mult"): unsigned 4-bit codes w, and per group of 128 along the row
 * an FP32 scale sc and a 4-bit shift sh, with x^ = sc * (w - sh).  The page
 * prints this decoder only; the encoder is the min-max one:
 *   lo = min(0, min x), hi = max(0, max x) over the group's finite elements;
 *   sc = (hi - lo) / 15 in FP32 (the largest float if that overflows);
 *   sh = round-half-even(-lo / sc), clamped to [0, 15];
 *   w  = clamp(round-half-even(x / sc) + sh, 0, 15).
 * sc == 0 gives w = sh = 0; NaN gives w = sh (x^ = 0), +-Inf the ends 15 / 0.
 * n_saturated counts x / sc above 15 - sh or below -sh.
 *   d->fmt must be IQ_INT4_ZP with IQ_PER_BLOCK and cols a multiple of 256
 *   (IQ_EINVAL otherwise); d->flags must be 0.
 *   codes   uint8 [rows, cols/2]: element 2t in bits 3:0 of byte t, i.e.
 *           eight per little-endian 32-bit word, element i in bits
 *           [4i, 4i+4) (the page's extract() order)
 *   scales  float32 [rows, cols/128], 4-byte aligned
 *   shifts  uint8 [rows, cols/256], group 2t in bits 3:0 of byte t (whole
 *           32-bit words of eight shifts per row when cols % 1024 == 0)
 * The other arguments, layouts, workspace rules and errors are those of
 * iq_quantize.  iq_quantize and iq_dequantize reject IQ_INT4_ZP.
 */
iq_status iq_quantize_zp(const iq_desc* d, const void* x, void* codes, float* scales, uint8_t* shifts,
                         iq_stats* stats, void* xhat, int32_t xhat_dtype, void* workspace,
                         hipStream_t stream);
/* x^ = sc * (w - sh) from codes, scales and shifts laid out as above;
 * otherwise as iq_dequantize. */
iq_status iq_dequantize_zp(const iq_desc* d, const void* codes, const float* scales,
                           const uint8_t* shifts, void* xhat, int32_t xhat_dtype, hipStream_t stream);
/* Bytes of the shifts array for an IQ_INT4_ZP descriptor (0 otherwise). */
size_t iq_shifts_bytes(const iq_desc* d);

/*
 * The consumer of Puzzle 12 (Triton post, "Quantized Matrix Mult"):
 *   z[j, k] = sum_l sc[j, l/128] * (w[j, l] - sh[j, l/128]) * y[l, k]
 * with the IQ_INT4_ZP weights of d (N0 = d->rows, K = d->cols; codes,
 * scales and shifts laid out as for iq_quantize_zp) and activations given
 * token-major: x is [n1, K] row-major BF16 with x[k, l] = y[l, k].
 *   z       output float32 [N0, n1] row-major, 4-byte aligned
 *   x_dtype must be IQ_BF16 (IQ_EUNSUPPORTED otherwise): the products
 *           (w - sh) * x are formed exactly on the BF16 matrix cores and
 *           summed in FP32; each group's sum is scaled by sc with one fma.
 * Accuracy: |z - exact| <= (K + 2) * 2^-24 * sum_l |sc (w - sh) y|.
 * d->in_dtype and d->ld_in are ignored; codes and x 16-byte aligned.
 * N0, n1 and K must fit 31 bits, and (N0/128)(n1/128) output tiles must
 * stay below 2^31 (IQ_EUNSUPPORTED).  n1 == 0 or N0 == 0 is
 * legal and writes nothing.  No workspace.
 * Grids too small to fill the GPU (from 33 tokens, below about one tile
 * per CU) split K in two halves: the call zeroes z with a kernel of its own,
 * then each half adds its FP32 sum atomically.  Two addends on a +0 start
 * give a + b rounded once in either order, so every call returns the same
 * bits; z must not be touched by other work until the call completes.
 */
iq_status iq_zp_gemm(const iq_desc* d, const void* codes, const float* scales, const uint8_t* shifts,
                     const void* x, int32_t x_dtype, int64_t n1, float* z, hipStream_t stream);

/*
 * FP4 GEMM over two MXFP4 operands (low-precision post, section "FP4 /
 * MXFP4 / NVFP4": an MXFP4 value is its E2M1 code times the block scale
 * 2^(E - 127), one E8M0 byte per 32 elements):
 *   z[j, t] = sum_k xw[j, k] * xa[t, k]
 * with the weights described by d (IQ_MXFP4, IQ_PER_BLOCK; N0 = d->rows,
 * K = d->cols) and n1 activation rows of the same K, both laid out as
 * iq_quantize writes MXFP4 (codes [rows, K/2], element 2t in the low
 * nibble; scales [rows, K/32] E8M0 bytes).
 *   z       output float32 [N0, n1] row-major, 4-byte aligned
 * The matrix cores form every product exactly (with its two block scales)
 * and sum in FP32: |z - exact| <= (K + 2) * 2^-24 * sum_k |xw xa|.  A scale
 * byte of 255 (E8M0 NaN; iq_quantize never writes it) makes every output of
 * its row or token NaN.
 * K must be a multiple of 128 (IQ_EINVAL); codes 16-byte aligned, scales
 * 4-byte aligned (IQ_EALIGN).  N0, n1 and K must fit 31 bits, and
 * (N0/128)(n1/128) output tiles must stay below 2^31 (IQ_EUNSUPPORTED).  n1 == 0 or N0 == 0 is legal and writes nothing.
 * d->in_dtype and d->ld_in are ignored.  No workspace; inputs are not
 * modified.
 */
iq_status iq_mx_gemm(const iq_desc* d, const void* codes_w, const void* scales_w, const void* codes_a,
                     const void* scales_a, int64_t n1, float* z, hipStream_t stream);

/*
 * MXFP4 weights against BF16 activations (low-precision post, section
 * "FP4 / MXFP4 / NVFP4": the weight values are E2M1 codes times the block
 * scale 2^(E - 127)):
 *   z[j, t] = sum_k xw[j, k] * x[t, k]
 * with the weights described by d (IQ_MXFP4, IQ_PER_BLOCK; N0 = d->rows,
 * K = d->cols; laid out as iq_quantize writes MXFP4) and x token-major
 * [n1, K] row-major.
 *   z       output float32 [N0, n1] row-major, 4-byte aligned
 *   x_dtype must be IQ_BF16 (IQ_EUNSUPPORTED otherwise).  Each weight is
 *           exact in BF16, so the BF16 matrix cores form exact products,
 *           summed in FP32: |z - exact| <= (K + 2) * 2^-24 * sum_k |xw x|.
 *           A scale byte of 255 (E8M0 NaN) makes its row's outputs NaN.
 * K must be a multiple of 128 (IQ_EINVAL); codes and x 16-byte aligned,
 * scales 4-byte aligned (IQ_EALIGN).  N0, n1 and K must fit 31 bits, and
 * (N0/128)(n1/128) output tiles must stay below 2^31 (IQ_EUNSUPPORTED).
 * n1 == 0 or N0 == 0 is legal and writes nothing.  d->in_dtype and d->ld_in
 * are ignored.  No workspace.  Grids too small to fill the GPU use 64-row
 * tiles; K is never split and z is written directly, once.
 */
iq_status iq_mxw_gemm(const iq_desc* d, const void* codes, const void* scales, const void* x, int32_t x_dtype,
                      int64_t n1, float* z, hipStream_t stream);

const char* iq_status_str(iq_status s);
int iq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
