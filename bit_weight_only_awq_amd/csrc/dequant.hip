// dequant.hip -- the AWQ weights dequantised into a dense fp16/bf16 matrix,
// W[k, n] = (q[k,n] - z[k/G,n]) * s[k/G,n] rounded once to the activation type.
//
// Not a step of the 4-bit GEMM itself: it is what a dense vendor GEMM needs as
// its weight operand, and so the first half of the "dequantise, then call the
// dense BLAS GEMM" route that the vLLM pull request "Speed up AWQ 2.5x with
// updated kernel" lists as a TODO for long sequences (its TODO list).  The
// benchmark times it with the vendor GEMM as a comparator of the fused kernels.
//
// Bound by device memory: per word (8 columns of one k) 4 bytes are read and 16
// written.  A thread owns one word-column and 8 consecutive k (inside one
// group, since G is a multiple of 8), so its scales and zero points are read
// once for 8 words; a wave's words and outputs are contiguous along N.
#include "device.hpp"
#include "launch.hpp"
#include "w4a16_ops.hpp"

namespace awq4 {

constexpr int kDequantThreads = 256;

// 1-D grid: blocks (k-block kb = 8 rows) x (column block of 256 word-columns)
template <int DT, bool SYM>
__global__ __launch_bounds__(kDequantThreads) void w4a16_dequant(const uint32_t *__restrict__ qw,
                                                                 const uint16_t *__restrict__ sc,
                                                                 const uint32_t *__restrict__ qz,
                                                                 uint16_t *__restrict__ w, int N, int G,
                                                                 int col_blocks) {
    const int nw = N >> 3;
    const int kb = blockIdx.x / col_blocks, cb = blockIdx.x - kb * col_blocks;
    const int j = cb * kDequantThreads + threadIdx.x;
    if (j >= nw) return;
    const int k0 = 8 * kb;
    const int g = k0 / G;
    const u32x4 s4 = *(const u32x4 *)(sc + (size_t)g * N + 8 * j);
    const uint32_t zw = SYM ? 0x88888888u : qz[(size_t)g * nw + j];
    float s[8];
    int z[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        s[t] = scale_f32<DT>(s4, t);
        z[t] = (int)((zw >> (4 * col_nibble(t))) & 0xFu);
    }
    uint32_t words[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) words[e] = qw[(size_t)(k0 + e) * nw + j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t h[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int t = 2 * p + b;
                const int q = (int)((words[e] >> (4 * col_nibble(t))) & 0xFu);
                // (q - z) * s is exact in fp32 (a 5-bit integer times an 8- or
                // 11-bit significand): the conversion is the one rounding
                h[b] = f32_to_out_bits((float)(q - z[t]) * s[t], DT);
            }
            o[p] = h[0] | (h[1] << 16);
        }
        *(u32x4 *)(w + (size_t)(k0 + e) * N + 8 * j) = o;
    }
}

template <int DT, bool SYM>
static hipError_t launch_dequant_t(const int32_t *qweight, const void *scales, const int32_t *qzeros, void *w,
                                   int64_t N, int64_t K, int G, hipStream_t st) {
    const int nw = (int)(N / 8);
    const int col_blocks = (nw + kDequantThreads - 1) / kDequantThreads;
    const int64_t blocks = (K / 8) * col_blocks;
    hipLaunchKernelGGL((w4a16_dequant<DT, SYM>), dim3((unsigned)blocks), dim3(kDequantThreads), 0, st,
                       (const uint32_t *)qweight, (const uint16_t *)scales, (const uint32_t *)qzeros, (uint16_t *)w,
                       (int)N, G, col_blocks);
    return hipGetLastError();
}

hipError_t launch_w4a16_dequant(const int32_t *qweight, const void *scales, const int32_t *qzeros, void *w, int64_t N,
                                int64_t K, int G, int dtype, hipStream_t st) {
    const bool sym = qzeros == nullptr;
    if (dtype == DT_F16)
        return sym ? launch_dequant_t<DT_F16, true>(qweight, scales, qzeros, w, N, K, G, st)
                   : launch_dequant_t<DT_F16, false>(qweight, scales, qzeros, w, N, K, G, st);
    return sym ? launch_dequant_t<DT_BF16, true>(qweight, scales, qzeros, w, N, K, G, st)
               : launch_dequant_t<DT_BF16, false>(qweight, scales, qzeros, w, N, K, G, st);
}

}  // namespace awq4
