// Reference streaming kernels for the benchmark harness (not part of libiq):
// a 16-byte non-temporal copy, the practical HBM ceiling for a kernel that
// reads and writes once, and a fill used to evict the memory-side cache
// between timed repetitions.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_copy16(const u4v* __restrict__ src, u4v* __restrict__ dst, uint64_t n16) {
    const uint64_t stride = (uint64_t)gridDim.x * 256 * 4;
    for (uint64_t base = (uint64_t)blockIdx.x * 1024 + threadIdx.x; base < n16; base += stride) {
        u4v v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint64_t i = base + (uint64_t)j * 256;
            if (i < n16) v[j] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint64_t i = base + (uint64_t)j * 256;
            if (i < n16) __builtin_nontemporal_store(v[j], dst + i);
        }
    }
}

__global__ __launch_bounds__(256) void k_fill16(u4v* __restrict__ dst, uint64_t n16, uint32_t value) {
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    u4v v = {value, value, value, value};
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = v;
}

extern "C" {
// n_bytes must be a multiple of 16; src/dst 16-byte aligned device pointers.
int iqb_copy(const void* src, void* dst, uint64_t n_bytes, int grid, hipStream_t stream) {
    if ((n_bytes & 15) || !src || !dst || grid <= 0) return 1;
    k_copy16<<<grid, 256, 0, stream>>>(static_cast<const u4v*>(src), static_cast<u4v*>(dst), n_bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
int iqb_fill(void* dst, uint64_t n_bytes, uint32_t value, hipStream_t stream) {
    if ((n_bytes & 15) || !dst) return 1;
    k_fill16<<<4096, 256, 0, stream>>>(static_cast<u4v*>(dst), n_bytes / 16, value);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
}
