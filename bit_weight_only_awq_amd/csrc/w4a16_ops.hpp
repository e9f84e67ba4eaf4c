// w4a16_ops.hpp -- W4A16 operand helpers shared by the decode and GEMM
// kernels: zero-point / scale constants of a word-column and the construction
// of matrix-core B operands from paired packed words (see device.hpp for the
// AWQ nibble order and the pairing).
#pragma once

#include "device.hpp"

namespace awq4 {

// Zero-point constants of one word-column for its 8 columns (fp16 path:
// packed -(1024+z) / -(64+z); bf16 path: z as float).
template <int DT>
struct ZeroConsts {
    uint32_t zc[8];
    float zf[8];
};

template <int DT, bool SYM>
__device__ __forceinline__ void zero_consts(ZeroConsts<DT> &c, uint32_t zw) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t z = SYM ? 8u : ((zw >> (4 * col_nibble(t))) & 0xFu);
        if (DT == DT_F16)
            c.zc[t] = col_hi(t) ? zconst_f16<1>(z) : zconst_f16<0>(z);
        else
            c.zf[t] = (float)z;
    }
}

// Scale of column t from the 8 scales of a word-column (16 bytes).
template <int DT>
__device__ __forceinline__ uint32_t scale_bits(u32x4 s4, int t) {
    return (s4[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
}
template <int DT>
__device__ __forceinline__ float scale_f32(u32x4 s4, int t) {
    const uint32_t b = scale_bits<DT>(s4, t);
    return DT == DT_F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

// Exact (q - z) pair of column t from one pair register, as fp16 or bf16.
template <int DT, int t>
__device__ __forceinline__ uint32_t qz_pair(uint32_t src, const ZeroConsts<DT> &c) {
    const uint32_t v = col_shift(t) ? (src >> 8) : src;
    if (DT == DT_F16) {
        const uint32_t mask = col_hi(t) ? 0x00F000F0u : 0x000F000Fu;
        // (v & mask) | 0x64006400 in one three-input bitwise op
        f16x2 h = bit_as<f16x2>(__builtin_amdgcn_bitop3_b32(v, mask, 0x64006400u, 0xEA));
        f16x2 z = bit_as<f16x2>(c.zc[t]);
        f16x2 d;
        if (col_hi(t)) {
            const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
            d = h * sixteenth + z;
        } else {
            d = h + z;
        }
        return bit_as<uint32_t>(d);
    } else {
        const uint32_t m = v & (col_hi(t) ? 0x00F000F0u : 0x000F000Fu);
        const float mul = col_hi(t) ? 0.0625f : 1.0f;
        const float d0 = __builtin_fmaf((float)(m & 0xFFu), mul, -c.zf[t]);          // exact
        const float d1 = __builtin_fmaf((float)((m >> 16) & 0xFFu), mul, -c.zf[t]);  // exact
        return (uint32_t)bit_as<uint16_t>((__bf16)d0) | ((uint32_t)bit_as<uint16_t>((__bf16)d1) << 16);
    }
}

// (q - z) * s pair of column t, rounded once to the activation type.
template <int DT, int t>
__device__ __forceinline__ uint32_t w_pair(uint32_t src, const ZeroConsts<DT> &c, uint32_t sc2, float sf) {
    if (DT == DT_F16) {
        return bit_as<uint32_t>(bit_as<f16x2>(qz_pair<DT, t>(src, c)) * bit_as<f16x2>(sc2));
    } else {
        const uint32_t v = col_shift(t) ? (src >> 8) : src;
        const uint32_t m = v & (col_hi(t) ? 0x00F000F0u : 0x000F000Fu);
        const float sm = col_hi(t) ? sf * 0.0625f : sf;
        const float zs = c.zf[t] * sf;
        const float w0 = __builtin_fmaf((float)(m & 0xFFu), sm, -zs);  // exact, one rounding below
        const float w1 = __builtin_fmaf((float)((m >> 16) & 0xFFu), sm, -zs);
        return (uint32_t)bit_as<uint16_t>((__bf16)w0) | ((uint32_t)bit_as<uint16_t>((__bf16)w1) << 16);
    }
}

template <int DT>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    if (DT == DT_F16) return mfma_f16(a, b, c);
    return mfma_bf16(a, b, c);
}

// Load BLK consecutive packed words of one k-row (zero words out of range).
// NT: streamed exactly once (non-temporal hint).
template <int BLK, bool NT>
__device__ __forceinline__ void load_words(const uint32_t *__restrict__ p, bool valid, uint32_t (&w)[BLK]) {
    if (!valid) {
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = 0;
        return;
    }
    if (BLK == 4) {
        u32x4 v = NT ? __builtin_nontemporal_load((const u32x4 *)p) : *(const u32x4 *)p;
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = v[b];
    } else if (BLK == 2) {
        u32x2 v = NT ? __builtin_nontemporal_load((const u32x2 *)p) : *(const u32x2 *)p;
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = v[b];
    } else {
        w[0] = NT ? __builtin_nontemporal_load(p) : *p;
    }
}

template <int DT>
__device__ __forceinline__ u32x4 pack8_out(f32x4 v0, f32x4 v1) {
    u32x4 o;
    o[0] = (uint32_t)f32_to_out_bits(v0[0], DT) | ((uint32_t)f32_to_out_bits(v0[1], DT) << 16);
    o[1] = (uint32_t)f32_to_out_bits(v0[2], DT) | ((uint32_t)f32_to_out_bits(v0[3], DT) << 16);
    o[2] = (uint32_t)f32_to_out_bits(v1[0], DT) | ((uint32_t)f32_to_out_bits(v1[1], DT) << 16);
    o[3] = (uint32_t)f32_to_out_bits(v1[2], DT) | ((uint32_t)f32_to_out_bits(v1[3], DT) << 16);
    return o;
}

}  // namespace awq4
