// Internal interface between the C ABI (iq_api.cpp) and the kernel launchers
// (iq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace iqk {

// Formats and granularities use the public enum values of iq.h.
enum { F_INT8 = 0, F_E4M3 = 1, F_E5M2 = 2, F_MXFP4 = 3, F_NVFP4 = 4, F_INT4 = 5, F_INT4ZP = 6 };
enum { G_TENSOR = 0, G_ROW = 1, G_BLOCK = 2 };
enum { D_F32 = 0, D_BF16 = 1 };
// Scale-rule variants, the public flag values.
enum : uint32_t { R_MX_NEAREST = 0x1u, R_MX_UP = 0x2u, R_NV_RNE = 0x4u };

constexpr int kThreads = 256;        // threads per workgroup of every streaming kernel
constexpr int kChunk = 8;            // elements per chunk (one 16-byte BF16 load)
constexpr int kTileChunksPerThread = 4;
constexpr int kTileChunks = kThreads * kTileChunksPerThread;  // chunks per workgroup iteration
constexpr int kMaxGrid = 2048;       // workgroups of the persistent streaming kernels

// Per-workgroup partial statistics, folded in a fixed order by the workgroup
// of the launch that finishes last.
struct alignas(16) Partial {
    double sum_x2, sum_err2, sum_abs_err;
    float max_abs_err;
    uint32_t n_saturated, n_zero_flush, n_nonfinite;
    uint32_t pad[2];
};
static_assert(sizeof(Partial) == 48, "partial layout");

// Arrival counters of one launch: workgroups count on their group's counter
// (kTicketGroup workgroups per group), the last of each group on the
// launch-wide counter, so no counter takes more than kTicketGroup atomics.
// Counters sit kTicketStride uint32 apart (separate 64-byte lines).
constexpr int kTicketGroup = 64;
constexpr int kTicketStride = 16;
constexpr size_t kTicketBytes = sizeof(uint32_t) * kTicketStride * (1 + kMaxGrid / kTicketGroup);

// Workspace layout.  The last workgroup of a launch folds the partials and
// sets every counter it used back to zero (each group's last arrival resets
// its group counter), so a zero-filled workspace stays ready for the next
// call.
struct Workspace {
    static constexpr size_t kStatsTicketOff = 0;                             // kTicketBytes
    static constexpr size_t kAmaxTicketOff = kStatsTicketOff + kTicketBytes;  // kTicketBytes
    static constexpr size_t kAmaxOff = kAmaxTicketOff + kTicketBytes;        // uint2 per workgroup
    static constexpr size_t kPartialOff = kAmaxOff + sizeof(uint32_t) * 2 * kMaxGrid;
    static constexpr size_t kBytes = kPartialOff + sizeof(Partial) * kMaxGrid;
};

struct QuantArgs {
    int fmt, gran, in_dtype;
    int64_t rows, cols, ld;
    const void* x;
    void* codes;
    void* scales;
    float* global_scale;
    uint8_t* shifts;      // asymmetric INT4: packed 4-bit shifts (else null)
    void* stats;          // iq_stats*, may be null
    void* xhat;           // may be null
    int xhat_dtype;
    uint32_t rule;        // R_* bits valid for fmt, 0 for the default rules
    const float* static_amax;  // per-tensor / NVFP4: caller-supplied absmax (null: measured)
    void* workspace;
};

struct DequantArgs {
    int fmt, gran;
    int64_t rows, cols;
    const void* codes;
    const void* scales;
    const float* global_scale;
    const uint8_t* shifts;   // asymmetric INT4 only
    void* xhat;
    int xhat_dtype;
};

// Puzzle 12 consumer: z [n0, n1] = dequantized asymmetric INT4 weights [n0, K]
// times the token-major BF16 activations x [n1, K], transposed.
struct ZpGemmLaunch {
    const void* codes;
    const float* scales;
    const uint8_t* shifts;
    const void* x;
    float* z;
    int64_t n0, n1, K;
};

// FP4 GEMM: z [n0, n1] = MXFP4 weights [n0, K] times MXFP4 activations
// [n1, K], transposed (codes K/2 bytes and E8M0 scales K/32 bytes per row).
struct MxGemmLaunch {
    const void* codes_w;
    const void* scales_w;
    const void* codes_a;
    const void* scales_a;
    float* z;
    int64_t n0, n1, K;
};

// MXFP4 weights [n0, K] times token-major BF16 activations x [n1, K], transposed.
struct MxwGemmLaunch {
    const void* codes;
    const void* scales;
    const void* x;
    float* z;
    int64_t n0, n1, K;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);
hipError_t launch_zp_gemm(const ZpGemmLaunch& g, hipStream_t stream);
hipError_t launch_mx_gemm(const MxGemmLaunch& g, hipStream_t stream);
hipError_t launch_mxw_gemm(const MxwGemmLaunch& g, hipStream_t stream);
hipError_t launch_amax(int in_dtype, int64_t rows, int64_t cols, int64_t ld, const void* x,
                       float* amax_out, void* workspace, hipStream_t stream);

// The library-held workspace of the current device (kScratchBytes, zero at
// load, tickets left at zero by every call): its device address.
constexpr size_t kScratchBytes = 128 * 1024;
hipError_t scratch_workspace(void** device_address);

}  // namespace iqk
