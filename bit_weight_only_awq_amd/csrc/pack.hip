// pack.hip -- pack / unpack 4-bit values into 32-bit words on gfx950.
//
// AWQ_LAYOUT_N8 (first-generation AWQ GEMM format; vLLM pull request "Speed up
// AWQ 2.5x with updated kernel", list of packing differences): a word packs
// the 8 columns 8j..8j+7 of one row; nibble i holds column 8j + MAP_N8[i].
// W4A8_LAYOUT_K8 (this library's W4A8 layout): a word packs k = 8kb..8kb+7 of
// one column; nibble i holds k = 8kb + MAP_K8[i], two's complement.
// AWQ_LAYOUT_V2 (the newer packing of the same list): identity order along a
// row, ceil(cols/8) words per row, unused nibbles skipped (see below).
// Out-of-range inputs are clamped, and counted when a counter is given
// (a missing clamp in packing was a real bug on the QQQ page, "Support W4A8
// quantization for vllm").
#include "device.hpp"
#include "launch.hpp"

namespace awq4 {

__constant__ int MAP_N8[8] = {0, 2, 4, 6, 1, 3, 5, 7};
__constant__ int MAP_K8[8] = {0, 4, 1, 5, 2, 6, 3, 7};

__device__ __forceinline__ void count_clamped(int32_t *clamp_count, int bad) {
    // one atomic per wave at most
    uint64_t any = __ballot(bad != 0);
    if (!any) return;
    int tot = bad;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if ((threadIdx.x & 63) == __builtin_ctzll(any)) atomicAdd(clamp_count, tot);
}

__global__ void pack_n8_kernel(const uint8_t *__restrict__ vals, uint32_t *__restrict__ out, int64_t words,
                               int32_t *clamp_count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (i < words) {
        const u32x2 v = *(const u32x2 *)(vals + 8 * i);  // the 8 columns of word i
        uint32_t w = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int c = MAP_N8[n];
            uint32_t q = (v[c >> 2] >> (8 * (c & 3))) & 0xFFu;
            if (q > 15u) {
                q = 15u;
                ++bad;
            }
            w |= q << (4 * n);
        }
        out[i] = w;
    }
    if (clamp_count) count_clamped(clamp_count, bad);
}

__global__ void unpack_n8_kernel(const uint32_t *__restrict__ in, uint8_t *__restrict__ vals, int64_t words) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const uint32_t w = in[i];
    u32x2 v = {0, 0};
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int c = MAP_N8[n];
        v[c >> 2] |= ((w >> (4 * n)) & 0xFu) << (8 * (c & 3));
    }
    *(u32x2 *)(vals + 8 * i) = v;
}

// K8: word (kb, n) gathers column n of rows 8kb..8kb+7 (one byte per row).
__global__ void pack_k8_kernel(const int8_t *__restrict__ vals, uint32_t *__restrict__ out, int64_t kblocks, int64_t N,
                               int32_t *clamp_count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (i < kblocks * N) {
        const int64_t kb = i / N, n = i - kb * N;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int q = vals[(8 * kb + MAP_K8[e]) * N + n];
            if (q < -8) {
                q = -8;
                ++bad;
            } else if (q > 7) {
                q = 7;
                ++bad;
            }
            w |= ((uint32_t)q & 0xFu) << (4 * e);
        }
        out[i] = w;
    }
    if (clamp_count) count_clamped(clamp_count, bad);
}

__global__ void unpack_k8_kernel(const uint32_t *__restrict__ in, int8_t *__restrict__ vals, int64_t kblocks, int64_t N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= kblocks * N) return;
    const int64_t kb = i / N, n = i - kb * N;
    const uint32_t w = in[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int nib = (int)((w >> (4 * e)) & 0xFu);
        vals[(8 * kb + MAP_K8[e]) * N + n] = (int8_t)((nib ^ 8) - 8);
    }
}

// Second AWQ packing (AWQ_LAYOUT_V2; the same pull request's list of
// differences: identity order map, zero points packed along the groups with
// the unused nibbles skipped): nibble e of word [r][j] holds element 8j + e
// of row r; a row of `cols` values takes ceil(cols / 8) words, and the
// nibbles past the last value are 0.
__global__ void pack_v2_kernel(const uint8_t *__restrict__ vals, uint32_t *__restrict__ out, int64_t rows,
                               int64_t cols, int32_t *clamp_count) {
    const int64_t wc = (cols + 7) / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int bad = 0;
    if (i < rows * wc) {
        const int64_t r = i / wc, j = i - r * wc;
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t c = 8 * j + e;
            if (c >= cols) break;  // skipped
            uint32_t q = vals[r * cols + c];
            if (q > 15u) {
                q = 15u;
                ++bad;
            }
            w |= q << (4 * e);
        }
        out[i] = w;
    }
    if (clamp_count) count_clamped(clamp_count, bad);
}

__global__ void unpack_v2_kernel(const uint32_t *__restrict__ in, uint8_t *__restrict__ vals, int64_t rows,
                                 int64_t cols) {
    const int64_t wc = (cols + 7) / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * wc) return;
    const int64_t r = i / wc, j = i - r * wc;
    const uint32_t w = in[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t c = 8 * j + e;
        if (c >= cols) break;
        vals[r * cols + c] = (uint8_t)((w >> (4 * e)) & 0xFu);
    }
}

// Repacking the second format into the first (the format of the GEMM and
// GEMV kernels): qweight words keep their place and have their nibbles
// reordered from the identity order to MAP_N8; zero points move from
// [N, ceil(G'/8)] words along the groups (G' = K / G groups) to [G', N/8]
// words along the columns.
__global__ void repack_v2_qweight(const uint32_t *__restrict__ in, uint32_t *__restrict__ out, int64_t words) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const uint32_t w = in[i];
    uint32_t o = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) o |= ((w >> (4 * MAP_N8[n])) & 0xFu) << (4 * n);
    out[i] = o;
}

__global__ void repack_v2_qzeros(const uint32_t *__restrict__ in, uint32_t *__restrict__ out, int64_t groups,
                                 int64_t N) {
    const int64_t nw = N / 8, zw = (groups + 7) / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= groups * nw) return;
    const int64_t g = i / nw, j = i - g * nw;
    uint32_t o = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int64_t col = 8 * j + MAP_N8[n];
        o |= ((in[col * zw + g / 8] >> (4 * (g % 8))) & 0xFu) << (4 * n);
    }
    out[i] = o;
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_repack_v2(const int32_t *qweight_v2, const int32_t *qzeros_v2, int32_t *qweight, int32_t *qzeros,
                            int64_t N, int64_t K, int G, hipStream_t st) {
    const int64_t words = K * (N / 8);
    hipLaunchKernelGGL(repack_v2_qweight, dim3(blocks_for(words)), dim3(256), 0, st, (const uint32_t *)qweight_v2,
                       (uint32_t *)qweight, words);
    if (qzeros_v2) {
        const int64_t groups = K / G;
        hipLaunchKernelGGL(repack_v2_qzeros, dim3(blocks_for(groups * (N / 8))), dim3(256), 0, st,
                           (const uint32_t *)qzeros_v2, (uint32_t *)qzeros, groups, N);
    }
    return hipGetLastError();
}

hipError_t launch_pack(const void *vals, int32_t *packed, int64_t rows, int64_t cols, int layout,
                       int32_t *clamp_count, hipStream_t st) {
    if (layout == 2) {
        const int64_t words = rows * ((cols + 7) / 8);
        if (words == 0) return hipSuccess;
        hipLaunchKernelGGL(pack_v2_kernel, dim3(blocks_for(words)), dim3(256), 0, st, (const uint8_t *)vals,
                           (uint32_t *)packed, rows, cols, clamp_count);
    } else if (layout == 0) {
        const int64_t words = rows * (cols / 8);
        if (words == 0) return hipSuccess;
        hipLaunchKernelGGL(pack_n8_kernel, dim3(blocks_for(words)), dim3(256), 0, st, (const uint8_t *)vals,
                           (uint32_t *)packed, words, clamp_count);
    } else {
        const int64_t words = (rows / 8) * cols;
        if (words == 0) return hipSuccess;
        hipLaunchKernelGGL(pack_k8_kernel, dim3(blocks_for(words)), dim3(256), 0, st, (const int8_t *)vals,
                           (uint32_t *)packed, rows / 8, cols, clamp_count);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const int32_t *packed, void *vals, int64_t rows, int64_t cols, int layout, hipStream_t st) {
    if (layout == 2) {
        const int64_t words = rows * ((cols + 7) / 8);
        if (words == 0) return hipSuccess;
        hipLaunchKernelGGL(unpack_v2_kernel, dim3(blocks_for(words)), dim3(256), 0, st, (const uint32_t *)packed,
                           (uint8_t *)vals, rows, cols);
    } else if (layout == 0) {
        const int64_t words = rows * (cols / 8);
        if (words == 0) return hipSuccess;
        hipLaunchKernelGGL(unpack_n8_kernel, dim3(blocks_for(words)), dim3(256), 0, st, (const uint32_t *)packed,
                           (uint8_t *)vals, words);
    } else {
        const int64_t words = (rows / 8) * cols;
        if (words == 0) return hipSuccess;
        hipLaunchKernelGGL(unpack_k8_kernel, dim3(blocks_for(words)), dim3(256), 0, st, (const uint32_t *)packed,
                           (int8_t *)vals, rows / 8, cols);
    }
    return hipGetLastError();
}

}  // namespace awq4
