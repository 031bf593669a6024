/*
 * Seeded synthetic inputs for the quantization path: Gaussian tensors with
 * outlier rows or columns, written as FP32 or BF16 row-major with a row
 * stride.  This module holds only input synthesis; it contains none of the
 * quantization arithmetic, and both the GPU path's tests/bench and the CPU
 * oracle consume the bytes it writes.
 *
 * The outlier model stands in for the workload described in the low-precision
 * float post (Blog on Lorn, "浅谈低精度浮点数", section FP8, the W4AFP8
 * discussion): weights carry outliers tens of times the typical magnitude,
 * activations up to hundreds of times.
 *
 * Random numbers: a counter-based splitmix64 (Steele, Lea, Flood 2014
 * finaliser applied to seed + (i+1)*golden-gamma), so element i of a tensor
 * is a pure function of (seed, i) and any thread split gives the same bytes.
 * Normal variates come from the Box-Muller transform in double precision.
 *
 * Value pipeline per element (row r, column c):
 *   z      = Box-Muller normal for the flat index r*cols + c
 *   val    = sigma * z * (outlier factor if r or c is an outlier index)
 *   f32    = (float)val                       (round to nearest even)
 *   bf16   = top half of f32, rounded to nearest even (BF16 outputs only)
 * Padding between cols and ld is filled with a large finite sentinel so that
 * any kernel read outside [0, cols) changes the absmax and is caught.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ull

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* i-th output of the splitmix64 stream started at `seed`. */
uint64_t synth_u64(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1) * GOLDEN_GAMMA); }

/* Uniform in (0, 1] with 53 random bits (never 0, so log() is finite). */
static double u01_open0(uint64_t bits) { return ((double)(bits >> 11) + 1.0) * 0x1p-53; }
/* Uniform in [0, 1). */
static double u01(uint64_t bits) { return (double)(bits >> 11) * 0x1p-53; }

/* Standard normal for flat index i: pair p = i/2 uses draws 2p and 2p+1 of
 * the stream; even i takes the cosine branch, odd i the sine branch. */
double synth_normal(uint64_t seed, uint64_t i) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t p = i >> 1;
    double u1 = u01_open0(synth_u64(seed, 2 * p));
    double u2 = u01(synth_u64(seed, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1));
    return (i & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
}

/* Outlier index set: the first k entries of a Fisher-Yates shuffle of
 * [0, dim) driven by the stream seeded with seed ^ 0x0D1E5EEDull.
 * mask[j] = 1 marks an outlier index.  k = floor(frac*dim + 0.5). */
int synth_outlier_mask(uint64_t seed, int64_t dim, double frac, uint8_t* mask) {
    if (dim <= 0) return 0;
    int64_t k = (int64_t)floor(frac * (double)dim + 0.5);
    if (k > dim) k = dim;
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)dim);
    if (!perm) return -1;
    for (int64_t j = 0; j < dim; ++j) perm[j] = j;
    uint64_t s = seed ^ 0x0D1E5EEDull;
    for (int64_t j = dim - 1; j > 0; --j) {
        uint64_t pick = synth_u64(s, (uint64_t)j) % (uint64_t)(j + 1);
        int64_t t = perm[j]; perm[j] = perm[pick]; perm[pick] = t;
    }
    memset(mask, 0, (size_t)dim);
    for (int64_t j = 0; j < k; ++j) mask[perm[j]] = 1;
    free(perm);
    return (int)k;
}

static uint16_t f32_to_bf16_bits(float f) {
    uint32_t u; memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef struct {
    void* out; int dtype; /* 0 = f32, 1 = bf16 */
    int64_t row_base, cols, ld, r0, r1; /* rows [r0, r1) of the output = tensor rows row_base + r */
    double sigma, factor; uint64_t seed;
    const uint8_t* row_mask; const uint8_t* col_mask;
} gen_job;

static void* gen_rows(void* arg) {
    gen_job* j = (gen_job*)arg;
    for (int64_t r = j->r0; r < j->r1; ++r) {
        int64_t tr = j->row_base + r; /* row index within the full tensor */
        for (int64_t c = 0; c < j->ld; ++c) {
            float f;
            if (c < j->cols) {
                double v = j->sigma * synth_normal(j->seed, (uint64_t)(tr * j->cols + c));
                if ((j->row_mask && j->row_mask[tr]) || (j->col_mask && j->col_mask[c])) v *= j->factor;
                f = (float)v;
            } else {
                f = 1.0e30f; /* padding sentinel */
            }
            size_t idx = (size_t)r * (size_t)j->ld + (size_t)c;
            if (j->dtype == 0) ((float*)j->out)[idx] = f;
            else ((uint16_t*)j->out)[idx] = f32_to_bf16_bits(f);
        }
    }
    return NULL;
}

/*
 * Fill out[nrows, ld] (FP32 if dtype == 0, BF16 bits if dtype == 1) with rows
 * [row0, row0 + nrows) of a tensor of rows_total x cols.  Every value depends
 * only on (seed, flat index) and the outlier sets only on the full dimension,
 * so any row range reproduces the same bytes as the full tensor.
 * outlier_axis: 0 none, 1 rows, 2 columns.  threads <= 0 means 1.
 * Returns the number of outlier indices, or -1 on bad arguments/allocation.
 */
int synth_fill(void* out, int dtype, int64_t rows_total, int64_t row0, int64_t nrows, int64_t cols,
               int64_t ld, double sigma, int outlier_axis, double outlier_frac,
               double outlier_factor, uint64_t seed, int threads) {
    if (nrows <= 0 || cols <= 0) return 0;
    if (row0 < 0 || row0 + nrows > rows_total || ld < cols) return -1;
    int64_t rows = nrows;
    uint8_t* rmask = NULL; uint8_t* cmask = NULL; int k = 0;
    if (outlier_axis == 1) { rmask = (uint8_t*)malloc((size_t)rows_total); if (!rmask) return -1; k = synth_outlier_mask(seed, rows_total, outlier_frac, rmask); }
    if (outlier_axis == 2) { cmask = (uint8_t*)malloc((size_t)cols); if (!cmask) return -1; k = synth_outlier_mask(seed, cols, outlier_frac, cmask); }
    if (threads <= 0) threads = 1;
    if (threads > 64) threads = 64;
    if (threads > rows) threads = (int)rows;
    pthread_t tid[64]; gen_job jobs[64];
    for (int t = 0; t < threads; ++t) {
        jobs[t] = (gen_job){out, dtype, row0, cols, ld, rows * t / threads, rows * (t + 1) / threads,
                            sigma, outlier_factor, seed, rmask, cmask};
    }
    for (int t = 1; t < threads; ++t) pthread_create(&tid[t], NULL, gen_rows, &jobs[t]);
    gen_rows(&jobs[0]);
    for (int t = 1; t < threads; ++t) pthread_join(tid[t], NULL);
    free(rmask); free(cmask);
    return k;
}
