// fp8_ops.hpp -- INT4-FP8 W4A8 matrix-core operands and epilogue, shared by
// the skinny and register-tiled kernels (w4a8_fp8.hip) and the LDS-pipelined
// GEMM (gemm_w4a8_fp8.hip).  The reading of the method (QQQ pull request
// "Support W4A8 quantization for vllm", the authors' INT4-FP8 follow-up) and
// the offset-binary weight codes are described in w4a8_fp8.hip.
#pragma once

#include "device.hpp"

namespace awq4 {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Operands.  B: 32 consecutive k of one column from four consecutive K8 words
// (nibble 2b of a word holds k = b and nibble 2b+1 holds k = 4 + b, so after
// the offset the low nibbles of the four bytes are k 0..3 and the high ones
// k 4..7).
__device__ __forceinline__ i32x8 fp8_b_operand(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    const uint32_t u0 = w0 ^ 0x88888888u, u1 = w1 ^ 0x88888888u, u2 = w2 ^ 0x88888888u, u3 = w3 ^ 0x88888888u;
    i32x8 b;
    b[0] = (int32_t)(u0 & 0x0F0F0F0Fu);
    b[1] = (int32_t)((u0 >> 4) & 0x0F0F0F0Fu);
    b[2] = (int32_t)(u1 & 0x0F0F0F0Fu);
    b[3] = (int32_t)((u1 >> 4) & 0x0F0F0F0Fu);
    b[4] = (int32_t)(u2 & 0x0F0F0F0Fu);
    b[5] = (int32_t)((u2 >> 4) & 0x0F0F0F0Fu);
    b[6] = (int32_t)(u3 & 0x0F0F0F0Fu);
    b[7] = (int32_t)((u3 >> 4) & 0x0F0F0F0Fu);
    return b;
}

__device__ __forceinline__ i32x8 load_a32(const uint8_t *p) {
    const u32x4 lo = *(const u32x4 *)p, hi = *(const u32x4 *)(p + 16);
    return (i32x8){(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                   (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
}

__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
    // A and B in E4M3 (format 0), unit E8M0 scales (127)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Final value of one output from its sum t = sum_k a u 2^-9.
template <int DT>
__device__ __forceinline__ void fp8_store(float t, int m, int n, int N, const float *__restrict__ s1,
                                          const float *__restrict__ asum, const uint16_t *__restrict__ s2,
                                          uint16_t *__restrict__ y, float *__restrict__ acc_out) {
    const float d = __builtin_fmaf(512.0f, t, -8.0f * asum[m]);  // sum a q, one rounding
    y[(size_t)m * N + n] = f32_to_out_bits(d * s1[m] * act_bits_to_f32<DT>(s2[n]), DT);
    if (acc_out) acc_out[(size_t)m * N + n] = d;
}
// The same with sum_k a q already formed (d) and the row's scale s1m.
template <int DT>
__device__ __forceinline__ void fp8_store_d(float d, int m, int n, int N, float s1m, const uint16_t *__restrict__ s2,
                                            uint16_t *__restrict__ y, float *__restrict__ acc_out) {
    y[(size_t)m * N + n] = f32_to_out_bits(d * s1m * act_bits_to_f32<DT>(s2[n]), DT);
    if (acc_out) acc_out[(size_t)m * N + n] = d;
}

}  // namespace awq4
