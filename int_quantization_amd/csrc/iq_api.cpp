// C ABI of libiq: host-side validation, size queries, dispatch to the
// kernel launchers.  Validation happens before any HIP call, so argument
// errors are reported without touching the device.
#include <stddef.h>
#include <stdint.h>

#include "../../include/iq.h"
#include "iq_launch.h"

namespace {

bool is_bf16_or_f32(int32_t t) { return t == IQ_F32 || t == IQ_BF16; }
size_t elem_size(int32_t t) { return t == IQ_F32 ? 4 : 2; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool four_bit(int32_t f) { return f == IQ_MXFP4 || f == IQ_NVFP4 || f == IQ_INT4 || f == IQ_INT4_ZP; }

// Elements per scale along a row (0 = whole row or tensor); -1 if the
// format / granularity pair is illegal.
int64_t block_of(int32_t fmt, int32_t gran) {
    switch (fmt) {
    case IQ_INT8: case IQ_FP8_E4M3: case IQ_FP8_E5M2:
        return (gran == IQ_PER_TENSOR || gran == IQ_PER_ROW) ? 0 : -1;
    case IQ_MXFP4: return gran == IQ_PER_BLOCK ? 32 : -1;
    case IQ_NVFP4: return gran == IQ_PER_BLOCK ? 16 : -1;
    case IQ_INT4: case IQ_INT4_ZP: return gran == IQ_PER_BLOCK ? 128 : -1;
    default: return -1;
    }
}

// A rule variant applies to its own format only, and the two MXFP4
// exponent rules exclude each other.
bool flags_valid(const iq_desc* d) {
    const uint32_t f = d->flags;
    switch (d->fmt) {
    case IQ_MXFP4:
        return (f & ~(IQ_FLAG_MX_ROUND_NEAREST | IQ_FLAG_MX_ROUND_UP)) == 0 &&
               f != (IQ_FLAG_MX_ROUND_NEAREST | IQ_FLAG_MX_ROUND_UP);
    case IQ_NVFP4: return (f & ~IQ_FLAG_NV_SCALE_RNE) == 0;
    default: return f == 0;
    }
}

static_assert(iqk::kScratchBytes == IQ_NOALLOC_SCRATCH_BYTES, "the held workspace is the size the header states");

static_assert(iqk::R_MX_NEAREST == IQ_FLAG_MX_ROUND_NEAREST && iqk::R_MX_UP == IQ_FLAG_MX_ROUND_UP &&
                  iqk::R_NV_RNE == IQ_FLAG_NV_SCALE_RNE,
              "rule bits are the public flag values");

// Whether rows x cols fits the 31-bit chunk indices of the kernels.
bool chunks_fit(int64_t rows, int64_t cols) {
    if (rows > ((int64_t)1 << 31) - 1 || cols / iqk::kChunk > ((int64_t)1 << 31)) return false;
    return rows == 0 || cols == 0 || rows * (cols / iqk::kChunk) < ((int64_t)1 << 31);
}

// Shape rules shared by every entry point.  cols must be a multiple of the
// 8-element chunk (16 for the 4-bit formats' blocks anyway) and of the
// block; the chunk count must fit 31 bits.
iq_status check_shape(const iq_desc* d, bool need_in_dtype) {
    if (!d) return IQ_EINVAL;
    if (need_in_dtype && !is_bf16_or_f32(d->in_dtype)) return IQ_EINVAL;
    int64_t b = block_of(d->fmt, d->gran);
    if (b < 0) return IQ_EINVAL;
    if (d->rows < 0 || d->cols < 0) return IQ_EINVAL;
    if (d->cols % iqk::kChunk) return IQ_EINVAL;
    if (b > 0 && d->cols % b) return IQ_EINVAL;
    if (d->fmt == IQ_INT4_ZP && d->cols % 256) return IQ_EINVAL;   // whole shift bytes per row
    if (!chunks_fit(d->rows, d->cols)) return IQ_EUNSUPPORTED;
    if (!flags_valid(d)) return IQ_EUNSUPPORTED;
    return IQ_OK;
}

// The kernels index chunks with 32 bits and element offsets row * ld_in
// with 64 bits: the chunk count must stay below 2^31 (chunks_fit) and
// rows * ld_in at most 2^59 elements, so byte offsets stay far inside 64
// bits.  Each factor is bounded before any product is formed.
iq_status check_input(const iq_desc* d, const void* x) {
    if (d->ld_in < d->cols) return IQ_EINVAL;
    if (d->ld_in > ((int64_t)1 << 40)) return IQ_EUNSUPPORTED;
    int64_t span = 0;
    if (__builtin_mul_overflow(d->rows, d->ld_in, &span) || span > ((int64_t)1 << 59)) return IQ_EUNSUPPORTED;
    if (d->rows > 0 && d->cols > 0) {
        if (!x) return IQ_EINVAL;
        if (!aligned(x, 16)) return IQ_EALIGN;
        if ((d->ld_in * (int64_t)elem_size(d->in_dtype)) % 16) return IQ_EALIGN;
    }
    return IQ_OK;
}

size_t codes_bytes(const iq_desc* d) {
    return (size_t)(d->rows * (four_bit(d->fmt) ? d->cols / 2 : d->cols));
}

size_t scales_bytes(const iq_desc* d) {
    switch (d->fmt) {
    case IQ_INT8: case IQ_FP8_E4M3: case IQ_FP8_E5M2:
        return d->gran == IQ_PER_TENSOR ? 4 : (size_t)d->rows * 4;
    case IQ_MXFP4: return (size_t)(d->rows * (d->cols / 32));
    case IQ_NVFP4: return (size_t)(d->rows * (d->cols / 16));
    case IQ_INT4_ZP: return (size_t)(d->rows * (d->cols / 128)) * 4;
    default: return (size_t)(d->rows * (d->cols / 128)) * 2;
    }
}

iq_status from_hip(hipError_t e) { return e == hipSuccess ? IQ_OK : IQ_EHIP; }

}  // namespace

extern "C" {

int iq_abi_version(void) { return IQ_ABI_VERSION; }

const char* iq_status_str(iq_status s) {
    switch (s) {
    case IQ_OK: return "ok";
    case IQ_EINVAL: return "invalid argument";
    case IQ_EALIGN: return "misaligned pointer or row stride";
    case IQ_EUNSUPPORTED: return "unsupported size or flags";
    case IQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

size_t iq_codes_bytes(const iq_desc* d) {
    if (check_shape(d, false) != IQ_OK) return 0;
    return codes_bytes(d);
}

size_t iq_scales_bytes(const iq_desc* d) {
    if (check_shape(d, false) != IQ_OK) return 0;
    return scales_bytes(d);
}

size_t iq_workspace_bytes(const iq_desc* d) {
    (void)d;
    return iqk::Workspace::kBytes;
}

size_t iq_shifts_bytes(const iq_desc* d) {
    if (check_shape(d, false) != IQ_OK || d->fmt != IQ_INT4_ZP) return 0;
    return (size_t)(d->rows * (d->cols / 256));
}

}  // extern "C"

namespace {

// Every check of a quantize call except the workspace's.
iq_status check_quantize(const iq_desc* d, const void* x, void* codes, void* scales, float* global_scale,
                         uint8_t* shifts, iq_stats* stats, void* xhat, int32_t xhat_dtype) {
    iq_status st = check_shape(d, true);
    if (st != IQ_OK) return st;
    if ((st = check_input(d, x)) != IQ_OK) return st;
    const bool empty = d->rows == 0 || d->cols == 0;
    const bool needs_scale_slot = d->gran == IQ_PER_TENSOR || !empty;
    if (!empty && !codes) return IQ_EINVAL;
    if (needs_scale_slot && !scales) return IQ_EINVAL;
    if (d->fmt == IQ_NVFP4 && !global_scale) return IQ_EINVAL;
    if (d->fmt == IQ_INT4_ZP && !empty && !shifts) return IQ_EINVAL;
    if (xhat && !is_bf16_or_f32(xhat_dtype)) return IQ_EINVAL;
    if (codes && !aligned(codes, 16)) return IQ_EALIGN;
    if (scales && !aligned(scales, 4)) return IQ_EALIGN;
    if (global_scale && !aligned(global_scale, 4)) return IQ_EALIGN;
    if (stats && !aligned(stats, 8)) return IQ_EALIGN;
    if (xhat && !aligned(xhat, 16)) return IQ_EALIGN;
    return IQ_OK;
}

iq_status quantize_impl(const iq_desc* d, const void* x, const float* static_amax, void* codes, void* scales,
                        float* global_scale, uint8_t* shifts, iq_stats* stats, void* xhat, int32_t xhat_dtype,
                        void* workspace, hipStream_t stream) {
    iq_status st = check_quantize(d, x, codes, scales, global_scale, shifts, stats, xhat, xhat_dtype);
    if (st != IQ_OK) return st;
    if (!workspace) return IQ_EINVAL;
    if (!aligned(workspace, 256)) return IQ_EALIGN;
    const bool empty = d->rows == 0 || d->cols == 0;

    iqk::QuantArgs a;
    a.fmt = d->fmt; a.gran = d->gran; a.in_dtype = d->in_dtype;
    a.rows = d->rows; a.cols = d->cols; a.ld = d->ld_in;
    a.x = x; a.codes = codes; a.scales = scales; a.global_scale = global_scale; a.shifts = shifts;
    a.stats = stats; a.xhat = xhat; a.xhat_dtype = xhat_dtype; a.workspace = workspace;
    a.rule = d->flags;
    a.static_amax = static_amax;
    if (empty) { a.rows = 0; a.cols = 0; }
    return from_hip(iqk::launch_quantize(a, stream));
}

iq_status dequantize_impl(const iq_desc* d, const void* codes, const void* scales, const float* global_scale,
                          const uint8_t* shifts, void* xhat, int32_t xhat_dtype, hipStream_t stream) {
    iq_status st = check_shape(d, false);
    if (st != IQ_OK) return st;
    if (!is_bf16_or_f32(xhat_dtype)) return IQ_EINVAL;
    if (d->rows == 0 || d->cols == 0) return IQ_OK;
    if (!codes || !scales || !xhat) return IQ_EINVAL;
    if (d->fmt == IQ_NVFP4 && !global_scale) return IQ_EINVAL;
    if (d->fmt == IQ_INT4_ZP && !shifts) return IQ_EINVAL;
    if (!aligned(codes, 16) || !aligned(xhat, 16) || !aligned(scales, 4)) return IQ_EALIGN;
    if (global_scale && !aligned(global_scale, 4)) return IQ_EALIGN;
    iqk::DequantArgs a;
    a.fmt = d->fmt; a.gran = d->gran; a.rows = d->rows; a.cols = d->cols;
    a.codes = codes; a.scales = scales; a.global_scale = global_scale; a.shifts = shifts;
    a.xhat = xhat; a.xhat_dtype = xhat_dtype;
    return from_hip(iqk::launch_dequantize(a, stream));
}

}  // namespace

extern "C" {

iq_status iq_quantize(const iq_desc* d, const void* x, void* codes, void* scales, float* global_scale,
                      iq_stats* stats, void* xhat, int32_t xhat_dtype, void* workspace, hipStream_t stream) {
    if (d && d->fmt == IQ_INT4_ZP) return IQ_EINVAL;   // shifts have no slot here: iq_quantize_zp
    return quantize_impl(d, x, nullptr, codes, scales, global_scale, nullptr, stats, xhat, xhat_dtype, workspace,
                         stream);
}

iq_status iq_quantize_noalloc(const iq_desc* d, const void* x, void* codes, void* scales, float* global_scale,
                              iq_stats* stats, void* xhat, int32_t xhat_dtype, hipStream_t stream) {
    if (d && d->fmt == IQ_INT4_ZP) return IQ_EINVAL;
    // every argument is checked before the first HIP call
    iq_status st = check_quantize(d, x, codes, scales, global_scale, nullptr, stats, xhat, xhat_dtype);
    if (st != IQ_OK) return st;
    if (iq_workspace_bytes(d) > iqk::kScratchBytes) return IQ_EUNSUPPORTED;   // beyond the held workspace
    void* ws = nullptr;
    if (iqk::scratch_workspace(&ws) != hipSuccess) return IQ_EHIP;
    return quantize_impl(d, x, nullptr, codes, scales, global_scale, nullptr, stats, xhat, xhat_dtype, ws, stream);
}

iq_status iq_quantize_zp(const iq_desc* d, const void* x, void* codes, float* scales, uint8_t* shifts,
                         iq_stats* stats, void* xhat, int32_t xhat_dtype, void* workspace, hipStream_t stream) {
    if (!d || d->fmt != IQ_INT4_ZP) return IQ_EINVAL;
    return quantize_impl(d, x, nullptr, codes, scales, nullptr, shifts, stats, xhat, xhat_dtype, workspace, stream);
}

iq_status iq_quantize_static(const iq_desc* d, const void* x, const float* amax_in, void* codes, void* scales,
                             float* global_scale, iq_stats* stats, void* xhat, int32_t xhat_dtype,
                             void* workspace, hipStream_t stream) {
    if (!d) return IQ_EINVAL;
    if (!(d->gran == IQ_PER_TENSOR || d->fmt == IQ_NVFP4)) return IQ_EINVAL;   // no per-tensor scale to take
    if (!amax_in) return IQ_EINVAL;
    iq_status st = check_shape(d, true);
    if (st != IQ_OK) return st;
    if (!aligned(amax_in, 4)) return IQ_EALIGN;
    return quantize_impl(d, x, amax_in, codes, scales, global_scale, nullptr, stats, xhat, xhat_dtype, workspace,
                         stream);
}

iq_status iq_dequantize(const iq_desc* d, const void* codes, const void* scales, const float* global_scale,
                        void* xhat, int32_t xhat_dtype, hipStream_t stream) {
    if (d && d->fmt == IQ_INT4_ZP) return IQ_EINVAL;   // iq_dequantize_zp
    return dequantize_impl(d, codes, scales, global_scale, nullptr, xhat, xhat_dtype, stream);
}

iq_status iq_dequantize_zp(const iq_desc* d, const void* codes, const float* scales, const uint8_t* shifts,
                           void* xhat, int32_t xhat_dtype, hipStream_t stream) {
    if (!d || d->fmt != IQ_INT4_ZP) return IQ_EINVAL;
    return dequantize_impl(d, codes, scales, nullptr, shifts, xhat, xhat_dtype, stream);
}

iq_status iq_zp_gemm(const iq_desc* d, const void* codes, const float* scales, const uint8_t* shifts,
                     const void* x, int32_t x_dtype, int64_t n1, float* z, hipStream_t stream) {
    iq_status st = check_shape(d, false);
    if (st != IQ_OK) return st;
    if (d->fmt != IQ_INT4_ZP) return IQ_EINVAL;
    if (!is_bf16_or_f32(x_dtype) || n1 < 0) return IQ_EINVAL;
    if (x_dtype != IQ_BF16) return IQ_EUNSUPPORTED;
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if (d->rows > lim || d->cols > lim || n1 > lim) return IQ_EUNSUPPORTED;
    if (((d->rows + 127) / 128) * ((n1 + 127) / 128) > lim - 64) return IQ_EUNSUPPORTED;   // one launch's grid
    if (d->rows == 0 || d->cols == 0 || n1 == 0) return IQ_OK;
    if (!codes || !scales || !shifts || !x || !z) return IQ_EINVAL;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(scales, 4) || !aligned(z, 4)) return IQ_EALIGN;
    iqk::ZpGemmLaunch g;
    g.codes = codes; g.scales = scales; g.shifts = shifts; g.x = x; g.z = z;
    g.n0 = d->rows; g.n1 = n1; g.K = d->cols;
    return from_hip(iqk::launch_zp_gemm(g, stream));
}

iq_status iq_mx_gemm(const iq_desc* d, const void* codes_w, const void* scales_w, const void* codes_a,
                     const void* scales_a, int64_t n1, float* z, hipStream_t stream) {
    iq_status st = check_shape(d, false);
    if (st != IQ_OK) return st;
    if (d->fmt != IQ_MXFP4 || d->gran != IQ_PER_BLOCK || n1 < 0) return IQ_EINVAL;
    if (d->cols % 128) return IQ_EINVAL;
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if (d->rows > lim || d->cols > lim || n1 > lim) return IQ_EUNSUPPORTED;
    if (((d->rows + 127) / 128) * ((n1 + 127) / 128) > lim - 64) return IQ_EUNSUPPORTED;   // one launch's grid
    if (d->rows == 0 || d->cols == 0 || n1 == 0) return IQ_OK;
    if (!codes_w || !scales_w || !codes_a || !scales_a || !z) return IQ_EINVAL;
    if (!aligned(codes_w, 16) || !aligned(codes_a, 16) || !aligned(scales_w, 4) || !aligned(scales_a, 4) ||
        !aligned(z, 4))
        return IQ_EALIGN;
    iqk::MxGemmLaunch g;
    g.codes_w = codes_w; g.scales_w = scales_w; g.codes_a = codes_a; g.scales_a = scales_a; g.z = z;
    g.n0 = d->rows; g.n1 = n1; g.K = d->cols;
    return from_hip(iqk::launch_mx_gemm(g, stream));
}

iq_status iq_mxw_gemm(const iq_desc* d, const void* codes, const void* scales, const void* x, int32_t x_dtype,
                      int64_t n1, float* z, hipStream_t stream) {
    iq_status st = check_shape(d, false);
    if (st != IQ_OK) return st;
    if (d->fmt != IQ_MXFP4 || d->gran != IQ_PER_BLOCK || n1 < 0) return IQ_EINVAL;
    if (d->cols % 128) return IQ_EINVAL;
    if (!is_bf16_or_f32(x_dtype)) return IQ_EINVAL;
    if (x_dtype != IQ_BF16) return IQ_EUNSUPPORTED;
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if (d->rows > lim || d->cols > lim || n1 > lim) return IQ_EUNSUPPORTED;
    if (((d->rows + 127) / 128) * ((n1 + 127) / 128) > lim - 64) return IQ_EUNSUPPORTED;   // one launch's grid
    if (d->rows == 0 || d->cols == 0 || n1 == 0) return IQ_OK;
    if (!codes || !scales || !x || !z) return IQ_EINVAL;
    if (!aligned(codes, 16) || !aligned(x, 16) || !aligned(scales, 4) || !aligned(z, 4)) return IQ_EALIGN;
    iqk::MxwGemmLaunch g;
    g.codes = codes; g.scales = scales; g.x = x; g.z = z;
    g.n0 = d->rows; g.n1 = n1; g.K = d->cols;
    return from_hip(iqk::launch_mxw_gemm(g, stream));
}

iq_status iq_amax(const iq_desc* d, const void* x, float* amax_out, void* workspace, hipStream_t stream) {
    if (!d) return IQ_EINVAL;
    if (!is_bf16_or_f32(d->in_dtype)) return IQ_EINVAL;
    if (d->rows < 0 || d->cols < 0 || d->cols % iqk::kChunk) return IQ_EINVAL;
    if (!chunks_fit(d->rows, d->cols)) return IQ_EUNSUPPORTED;
    iq_status st = check_input(d, x);
    if (st != IQ_OK) return st;
    if (!amax_out || !workspace) return IQ_EINVAL;
    if (!aligned(workspace, 256)) return IQ_EALIGN;
    if (!aligned(amax_out, 4)) return IQ_EALIGN;
    const bool empty = d->rows == 0 || d->cols == 0;
    return from_hip(iqk::launch_amax(d->in_dtype, empty ? 0 : d->rows, empty ? 0 : d->cols, d->ld_in, x,
                                     amax_out, workspace, stream));
}

}  // extern "C"
