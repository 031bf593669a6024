// Host-side checks of the C ABI's argument validation (iq_api.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer and linked against
// stand-ins for the kernel launchers that only record what they were
// given.  Every entry point is called with legal arguments (exactly one
// launch, with the descriptor's sizes passed through) and with each kind of
// illegal argument: NULL or misaligned pointers, bad enums, shapes that are
// negative, ragged against the block or large enough to overflow 64-bit
// products, strides below the row length or beyond the 2^40 limit, unknown
// flags.  An illegal call must return its documented status and launch
// nothing; any signed overflow or out-of-range conversion on the way aborts
// the run.  No GPU and no HIP runtime are involved.
//
// Test infrastructure: compiled only by the CPU test suite.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "iq.h"
#include "../int_quantization_amd/csrc/iq_launch.h"

namespace iqk {
int launches = 0;
QuantArgs last_q;
DequantArgs last_d;
int64_t last_amax_rows = -1, last_amax_cols = -1;
hipError_t launch_quantize(const QuantArgs& a, hipStream_t) { ++launches; last_q = a; return hipSuccess; }
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t) { ++launches; last_d = a; return hipSuccess; }
hipError_t launch_zp_gemm(const ZpGemmLaunch&, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_mx_gemm(const MxGemmLaunch&, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_mxw_gemm(const MxwGemmLaunch&, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_amax(int, int64_t rows, int64_t cols, int64_t, const void*, float*, void*, hipStream_t) {
    ++launches; last_amax_rows = rows; last_amax_cols = cols; return hipSuccess;
}
hipError_t scratch_workspace(void** p) { *p = reinterpret_cast<void*>(uintptr_t(1) << 40); return hipSuccess; }
}  // namespace iqk

static int failures = 0;
static long checks = 0;
#define EXPECT(cond, ...)                                                  \
    do {                                                                   \
        ++checks;                                                          \
        if (!(cond)) {                                                     \
            ++failures;                                                    \
            std::fprintf(stderr, "line %d: ", __LINE__);                   \
            std::fprintf(stderr, __VA_ARGS__);                             \
            std::fprintf(stderr, "\n");                                    \
        }                                                                  \
    } while (0)

// Device addresses are never dereferenced by the host code: any aligned
// integer stands in for one.
static void* dev(uintptr_t k, uintptr_t misalign = 0) { return reinterpret_cast<void*>((k << 20) + misalign); }

static iq_desc desc(int fmt, int gran, int dt, int64_t rows, int64_t cols, int64_t ld = -1, uint32_t flags = 0) {
    iq_desc d{};
    d.fmt = fmt; d.gran = gran; d.in_dtype = dt; d.rows = rows; d.cols = cols; d.ld_in = ld < 0 ? cols : ld;
    d.flags = flags;
    return d;
}

static iq_status quantize(const iq_desc& d, uintptr_t x_mis = 0, bool gs = true, void* ws = dev(9)) {
    return iq_quantize(&d, dev(1, x_mis), dev(2), dev(3), gs ? static_cast<float*>(dev(4)) : nullptr,
                       static_cast<iq_stats*>(dev(5)), dev(6), IQ_F32, ws, nullptr);
}

// A call that must fail with `want` and launch nothing.
#define EXPECT_REJECT(call, want)                                                            \
    do {                                                                                     \
        const int before = iqk::launches;                                                    \
        const iq_status got = (call);                                                        \
        EXPECT(got == (want), "%s: status %d, expected %d", #call, (int)got, (int)(want));    \
        EXPECT(iqk::launches == before, "%s launched on an error", #call);                   \
    } while (0)

// A call that must succeed with exactly one launch.
#define EXPECT_ONE_LAUNCH(call)                                                              \
    do {                                                                                     \
        const int before = iqk::launches;                                                    \
        const iq_status got = (call);                                                        \
        EXPECT(got == IQ_OK, "%s: status %d", #call, (int)got);                              \
        EXPECT(iqk::launches == before + 1, "%s: %d launches", #call, iqk::launches - before); \
    } while (0)

int main() {
    const int64_t big = std::numeric_limits<int64_t>::max();
    struct Legal { int fmt, gran; int64_t cols; };
    const Legal legal[] = {{IQ_INT8, IQ_PER_TENSOR, 64},   {IQ_INT8, IQ_PER_ROW, 8},       {IQ_FP8_E4M3, IQ_PER_ROW, 8192},
                           {IQ_FP8_E5M2, IQ_PER_TENSOR, 24}, {IQ_MXFP4, IQ_PER_BLOCK, 32}, {IQ_NVFP4, IQ_PER_BLOCK, 16},
                           {IQ_INT4, IQ_PER_BLOCK, 128}};
    for (const Legal& l : legal)
        for (int dt : {IQ_F32, IQ_BF16}) {
            const iq_desc d = desc(l.fmt, l.gran, dt, 37, l.cols);
            EXPECT_ONE_LAUNCH(quantize(d));
            EXPECT(iqk::last_q.rows == 37 && iqk::last_q.cols == l.cols && iqk::last_q.ld == l.cols,
                   "sizes not passed through (fmt %d)", l.fmt);
            EXPECT_ONE_LAUNCH(iq_quantize_noalloc(&d, dev(1), dev(2), dev(3), static_cast<float*>(dev(4)), nullptr,
                                                  nullptr, IQ_F32, nullptr));
            EXPECT(iqk::last_q.workspace == dev(1u << 20), "held workspace not used");
            EXPECT_ONE_LAUNCH(iq_dequantize(&d, dev(2), dev(3), static_cast<const float*>(dev(4)), dev(6), IQ_BF16,
                                            nullptr));
            EXPECT(iqk::last_d.rows == 37 && iqk::last_d.cols == l.cols, "dequantize sizes (fmt %d)", l.fmt);
            EXPECT(iq_codes_bytes(&d) == (size_t)(37 * (l.fmt >= IQ_MXFP4 ? l.cols / 2 : l.cols)), "codes bytes");
            EXPECT(iq_workspace_bytes(&d) >= 256 && iq_workspace_bytes(&d) <= IQ_NOALLOC_SCRATCH_BYTES, "workspace");
            // empty tensors are legal
            EXPECT(quantize(desc(l.fmt, l.gran, dt, 0, l.cols)) == IQ_OK, "empty rows");
            EXPECT(quantize(desc(l.fmt, l.gran, dt, 5, 0)) == IQ_OK, "empty cols");
            // row stride
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, l.cols, l.cols - 8)), IQ_EINVAL);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, l.cols, (int64_t)1 << 41)), IQ_EUNSUPPORTED);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, l.cols, big)), IQ_EUNSUPPORTED);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, (int64_t)1 << 30, l.cols, (int64_t)1 << 40)),
                          IQ_EUNSUPPORTED);
            // shapes that would overflow products of rows and cols
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, big, l.cols)), IQ_EUNSUPPORTED);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 2, big - big % 256)), IQ_EUNSUPPORTED);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, (int64_t)1 << 31, 8192)), IQ_EUNSUPPORTED);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, -1, l.cols)), IQ_EINVAL);
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, -l.cols)), IQ_EINVAL);
            EXPECT(iq_codes_bytes(&d) != 0 && iq_codes_bytes(&(const iq_desc&)desc(l.fmt, l.gran, dt, big, 64)) == 0,
                   "codes bytes of an oversized descriptor");
            // ragged against the chunk or the block
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, l.cols + 4)), IQ_EINVAL);
            // pointers
            EXPECT_REJECT(quantize(d, 4), IQ_EALIGN);
            EXPECT_REJECT(iq_quantize(&d, nullptr, dev(2), dev(3), static_cast<float*>(dev(4)), nullptr, nullptr,
                                      IQ_F32, dev(9), nullptr),
                          IQ_EINVAL);
            EXPECT_REJECT(iq_quantize(&d, dev(1), nullptr, dev(3), static_cast<float*>(dev(4)), nullptr, nullptr,
                                      IQ_F32, dev(9), nullptr),
                          IQ_EINVAL);
            EXPECT_REJECT(iq_quantize(&d, dev(1), dev(2), nullptr, static_cast<float*>(dev(4)), nullptr, nullptr,
                                      IQ_F32, dev(9), nullptr),
                          IQ_EINVAL);
            EXPECT_REJECT(quantize(d, 0, true, nullptr), IQ_EINVAL);
            EXPECT_REJECT(quantize(d, 0, true, dev(9, 64)), IQ_EALIGN);
            EXPECT_REJECT(iq_quantize(&d, dev(1), dev(2), dev(3), static_cast<float*>(dev(4)), nullptr, dev(6), 7,
                                      dev(9), nullptr),
                          IQ_EINVAL);   // x^ type
            if (l.fmt == IQ_NVFP4)
                EXPECT_REJECT(quantize(d, 0, false), IQ_EINVAL);   // the global scale is an output
            // flags belong to their own format
            EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, l.cols, -1, 0x80u)), IQ_EUNSUPPORTED);
            if (l.fmt != IQ_MXFP4)
                EXPECT_REJECT(quantize(desc(l.fmt, l.gran, dt, 4, l.cols, -1, IQ_FLAG_MX_ROUND_UP)), IQ_EUNSUPPORTED);
            // absmax on its own
            EXPECT_ONE_LAUNCH(iq_amax(&d, dev(1), static_cast<float*>(dev(4)), dev(9), nullptr));
            EXPECT(iqk::last_amax_rows == 37 && iqk::last_amax_cols == l.cols, "amax sizes");
            EXPECT_REJECT(iq_amax(&(const iq_desc&)desc(l.fmt, l.gran, dt, big, 64), dev(1),
                                  static_cast<float*>(dev(4)), dev(9), nullptr),
                          IQ_EUNSUPPORTED);
        }
    // bad enums
    EXPECT_REJECT(quantize(desc(7, IQ_PER_BLOCK, IQ_F32, 4, 128)), IQ_EINVAL);
    EXPECT_REJECT(quantize(desc(-1, IQ_PER_BLOCK, IQ_F32, 4, 128)), IQ_EINVAL);
    EXPECT_REJECT(quantize(desc(IQ_INT8, 3, IQ_F32, 4, 128)), IQ_EINVAL);
    EXPECT_REJECT(quantize(desc(IQ_INT8, IQ_PER_ROW, 2, 4, 128)), IQ_EINVAL);
    EXPECT_REJECT(quantize(desc(IQ_MXFP4, IQ_PER_ROW, IQ_F32, 4, 128)), IQ_EINVAL);
    EXPECT_REJECT(quantize(desc(IQ_INT8, IQ_PER_BLOCK, IQ_F32, 4, 128)), IQ_EINVAL);
    EXPECT_REJECT(iq_quantize(nullptr, dev(1), dev(2), dev(3), nullptr, nullptr, nullptr, IQ_F32, dev(9), nullptr),
                  IQ_EINVAL);
    // the two MXFP4 rules exclude each other
    EXPECT_REJECT(quantize(desc(IQ_MXFP4, IQ_PER_BLOCK, IQ_F32, 4, 128, -1,
                                IQ_FLAG_MX_ROUND_UP | IQ_FLAG_MX_ROUND_NEAREST)),
                  IQ_EUNSUPPORTED);

    // static scaling: per tensor and NVFP4 only
    {
        const iq_desc t = desc(IQ_FP8_E4M3, IQ_PER_TENSOR, IQ_BF16, 16, 64);
        EXPECT_ONE_LAUNCH(iq_quantize_static(&t, dev(1), static_cast<const float*>(dev(7)), dev(2), dev(3), nullptr,
                                             nullptr, nullptr, IQ_F32, dev(9), nullptr));
        EXPECT_REJECT(iq_quantize_static(&t, dev(1), nullptr, dev(2), dev(3), nullptr, nullptr, nullptr, IQ_F32,
                                         dev(9), nullptr),
                      IQ_EINVAL);
        const iq_desc r = desc(IQ_FP8_E4M3, IQ_PER_ROW, IQ_BF16, 16, 64);
        EXPECT_REJECT(iq_quantize_static(&r, dev(1), static_cast<const float*>(dev(7)), dev(2), dev(3), nullptr,
                                         nullptr, nullptr, IQ_F32, dev(9), nullptr),
                      IQ_EINVAL);
    }
    // asymmetric INT4: only through its own entry points, cols a multiple of 256
    {
        const iq_desc z = desc(IQ_INT4_ZP, IQ_PER_BLOCK, IQ_BF16, 9, 512);
        EXPECT_ONE_LAUNCH(iq_quantize_zp(&z, dev(1), dev(2), static_cast<float*>(dev(3)),
                                         static_cast<uint8_t*>(dev(4)), nullptr, nullptr, IQ_F32, dev(9), nullptr));
        EXPECT_REJECT(quantize(z), IQ_EINVAL);
        EXPECT_REJECT(iq_quantize_noalloc(&z, dev(1), dev(2), dev(3), nullptr, nullptr, nullptr, IQ_F32, nullptr),
                      IQ_EINVAL);
        const iq_desc z128 = desc(IQ_INT4_ZP, IQ_PER_BLOCK, IQ_BF16, 9, 384);
        EXPECT_REJECT(iq_quantize_zp(&z128, dev(1), dev(2), static_cast<float*>(dev(3)),
                                     static_cast<uint8_t*>(dev(4)), nullptr, nullptr, IQ_F32, dev(9), nullptr),
                      IQ_EINVAL);
        EXPECT(iq_shifts_bytes(&z) == 9 * 2, "shift bytes");
        EXPECT_ONE_LAUNCH(iq_dequantize_zp(&z, dev(2), static_cast<const float*>(dev(3)),
                                           static_cast<const uint8_t*>(dev(4)), dev(6), IQ_F32, nullptr));
        // Puzzle 12's consumer
        EXPECT_ONE_LAUNCH(iq_zp_gemm(&z, dev(2), static_cast<const float*>(dev(3)), static_cast<const uint8_t*>(dev(4)),
                                     dev(1), IQ_BF16, 100, static_cast<float*>(dev(5)), nullptr));
        EXPECT_REJECT(iq_zp_gemm(&z, dev(2), static_cast<const float*>(dev(3)), static_cast<const uint8_t*>(dev(4)),
                                 dev(1), IQ_BF16, big, static_cast<float*>(dev(5)), nullptr),
                      IQ_EUNSUPPORTED);
        EXPECT_REJECT(iq_zp_gemm(&z, dev(2), static_cast<const float*>(dev(3)), static_cast<const uint8_t*>(dev(4)),
                                 dev(1), IQ_BF16, -1, static_cast<float*>(dev(5)), nullptr),
                      IQ_EINVAL);
    }
    // FP4 GEMMs
    {
        const iq_desc w = desc(IQ_MXFP4, IQ_PER_BLOCK, IQ_BF16, 256, 1024);
        EXPECT_ONE_LAUNCH(iq_mx_gemm(&w, dev(1), dev(2), dev(3), dev(4), 64, static_cast<float*>(dev(5)), nullptr));
        EXPECT_ONE_LAUNCH(iq_mxw_gemm(&w, dev(1), dev(2), dev(3), IQ_BF16, 64, static_cast<float*>(dev(5)), nullptr));
        EXPECT_REJECT(iq_mx_gemm(&w, dev(1), dev(2), dev(3), dev(4), big, static_cast<float*>(dev(5)), nullptr),
                      IQ_EUNSUPPORTED);
        EXPECT_REJECT(iq_mxw_gemm(&w, dev(1), dev(2), dev(3), IQ_F32, 64, static_cast<float*>(dev(5)), nullptr),
                      IQ_EUNSUPPORTED);
        const iq_desc k96 = desc(IQ_MXFP4, IQ_PER_BLOCK, IQ_BF16, 256, 96);
        EXPECT_REJECT(iq_mx_gemm(&k96, dev(1), dev(2), dev(3), dev(4), 64, static_cast<float*>(dev(5)), nullptr),
                      IQ_EINVAL);
        const iq_desc huge = desc(IQ_MXFP4, IQ_PER_BLOCK, IQ_BF16, big, 1024);
        EXPECT_REJECT(iq_mx_gemm(&huge, dev(1), dev(2), dev(3), dev(4), 64, static_cast<float*>(dev(5)), nullptr),
                      IQ_EUNSUPPORTED);
    }
    EXPECT(iq_abi_version() == IQ_ABI_VERSION, "abi version");
    for (int s = -1; s <= 5; ++s) EXPECT(iq_status_str(static_cast<iq_status>(s)) != nullptr, "status string");
    std::printf("%s %ld checks, %d launches\n", failures ? "FAILED" : "ok", checks, iqk::launches);
    return failures ? 1 : 0;
}
