// stream.hip -- read-only bandwidth probe on gfx950 (a measurement helper,
// not a step of the method): it streams a buffer from device memory once and
// folds it into a checksum, so the achievable HBM read rate at a given size
// can be measured beside the GEMV that streams the same number of bytes.
#include "device.hpp"
#include "launch.hpp"

namespace awq4 {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                                     uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    uint32_t acc = 0;
    // four independent 16-byte loads in flight per thread and iteration
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        const u32x4 e = a ^ b ^ c ^ d;
        acc ^= e[0] ^ e[1] ^ e[2] ^ e[3];
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    int64_t blocks = (n16 + kStreamThreads - 1) / kStreamThreads;
    if (blocks > kStreamMaxBlocks) blocks = kStreamMaxBlocks;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kStreamThreads), 0, st, (const u32x4 *)src,
                       n16, sink);
    return hipGetLastError();
}

}  // namespace awq4
