// Reference streaming kernels for the benchmark harness (not part of libiq).
// They bound what any kernel that streams HBM can reach on this chip:
//   read-only, write-only, copy, and read:write mixes of 2:1 and 4:1 bytes
//   (the ratios of the 1-byte and the 4-bit quantizers of a BF16 input),
// each with NR 16-byte words read and NW words written per lane and
// iteration, so the depth of loads in flight per lane is a template
// parameter (4, 8 or 16 words).  Every load and store instruction of a
// workgroup covers 4 KiB of consecutive bytes (1 KiB per wave).  A
// non-temporal variant matches the cache policy of the quantize kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

namespace {

template <bool NT> __device__ __forceinline__ u4v ld16(const u4v* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT> __device__ __forceinline__ void st16(u4v v, u4v* p) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// One workgroup iteration reads NR * 256 words and writes NW * 256 words;
// `iters` iterations cover the buffers exactly.  Read-only kernels fold the
// loaded words into a value that is stored only if it equals `magic` (the
// caller passes a value the data cannot produce), so no load is dead.
template <int NR, int NW, bool NT>
__global__ __launch_bounds__(256) void k_stream(const u4v* __restrict__ src, u4v* __restrict__ dst, uint64_t iters,
                                                uint32_t magic) {
    const uint32_t t = threadIdx.x;
    u4v acc = {0u, 0u, 0u, 0u};
    for (uint64_t it = blockIdx.x; it < iters; it += gridDim.x) {
        u4v r[NR > 0 ? NR : 1];
#pragma unroll
        for (int j = 0; j < NR; ++j) r[j] = ld16<NT>(src + (it * NR + j) * 256 + t);
        if (NW == 0) {
#pragma unroll
            for (int j = 0; j < NR; ++j) acc ^= r[j];
        } else {
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                u4v w;
                if (NR == 0) {
                    w = u4v{magic, (uint32_t)it, (uint32_t)j, t};
                } else {
                    constexpr int P = (NW > 0 && NR >= NW) ? NR / NW : 1;   // words folded into each written word
                    w = r[j * P];
#pragma unroll
                    for (int k = 1; k < P; ++k) w ^= r[j * P + k];
                }
                st16<NT>(w, dst + (it * NW + j) * 256 + t);
            }
        }
    }
    if (NW == 0 && (acc.x ^ acc.y ^ acc.z ^ acc.w) == magic) dst[blockIdx.x * 256 + t] = acc;
}

template <int NR, int NW>
int launch(bool nt, const void* src, void* dst, uint64_t iters, int grid, hipStream_t s) {
    const u4v* a = static_cast<const u4v*>(src);
    u4v* b = static_cast<u4v*>(dst);
    if (nt) k_stream<NR, NW, true><<<grid, 256, 0, s>>>(a, b, iters, 0xA5A5F00Du);
    else k_stream<NR, NW, false><<<grid, 256, 0, s>>>(a, b, iters, 0xA5A5F00Du);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Words per lane and iteration for (kind, depth): depth is the number of
// words in flight on the heavier side.
struct Shape { int nr, nw; };
Shape shape_of(int kind, int depth) {
    switch (kind) {
    case 0: return {depth, 0};             // read only
    case 1: return {0, depth};             // write only
    case 2: return {depth, depth};         // copy
    case 3: return {depth, depth / 2};     // read 2 : write 1
    default: return {depth, depth / 4};    // read 4 : write 1
    }
}

}  // namespace

extern "C" {
// Stream `bytes` of the larger side (the read side, or the written bytes for
// the write-only kind) through the kernel of (kind, depth):
//   kind 0 read-only, 1 write-only, 2 copy, 3 read:write 2:1, 4 read:write 4:1
//   depth 4, 8 or 16 words of 16 bytes per lane
// src must hold `bytes` (kinds 0, 2-4) and dst the written bytes (bytes for
// kinds 1 and 2, bytes/2 for kind 3, bytes/4 for kind 4; one 4 KiB word
// row per workgroup for kind 0).  bytes must be a multiple of 16 * 256 *
// depth; pointers 16-byte aligned device pointers.  Returns 0 on success.
int iqb_stream(int kind, int depth, int nontemporal, const void* src, void* dst, uint64_t bytes, int grid,
               hipStream_t stream) {
    if (kind < 0 || kind > 4 || !(depth == 4 || depth == 8 || depth == 16) || grid <= 0 || !dst) return 1;
    if (kind != 1 && !src) return 1;
    const uint64_t per_iter = (uint64_t)16 * 256 * depth;
    if (bytes == 0 || bytes % per_iter) return 1;
    const uint64_t iters = bytes / per_iter;
    const Shape sh = shape_of(kind, depth);
    const bool nt = nontemporal != 0;
#define IQB_CASE(R, W) if (sh.nr == R && sh.nw == W) return launch<R, W>(nt, src, dst, iters, grid, stream)
    IQB_CASE(4, 0); IQB_CASE(8, 0); IQB_CASE(16, 0);
    IQB_CASE(0, 4); IQB_CASE(0, 8); IQB_CASE(0, 16);
    IQB_CASE(4, 4); IQB_CASE(8, 8); IQB_CASE(16, 16);
    IQB_CASE(4, 2); IQB_CASE(8, 4); IQB_CASE(16, 8);
    IQB_CASE(4, 1); IQB_CASE(8, 2); IQB_CASE(16, 4);
#undef IQB_CASE
    return 1;
}
}
