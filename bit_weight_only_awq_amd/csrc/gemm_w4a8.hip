// gemm_w4a8.hip -- W4A8 GEMM for large M on gfx950 (int8 matrix cores).
//
// Same method as w4a8.hip (vLLM pull request "Support W4A8 quantization for
// vllm": int4 placed in the upper nibble of an int8, int32 accumulation, s1
// per token and s2 per channel on the output, per-group scales in addition
// for grouped weights -- here integer s3 folded into the int8 weights).
//
// Workgroup tile (32*MT) x 128, K in stages of 64 (one 16x16x64 step); 4
// waves in a 2 x 2 grid, each owning (16*MT) x 64 outputs: MT row tiles x 4
// column MFMAs.  Lane j of a wave reads 16 bytes = 4 consecutive columns of
// two K8 word rows, which give the B operands of its 4 MFMAs (output column
// = 64*wn + 4j + u).  a8 rows, packed words and (grouped) s3 rows are copied
// straight from global memory into LDS by the direct-to-LDS loads: a8 one
// stage ahead in two buffers, words and s3 two stages ahead in three, so one
// wait and one barrier end each stage.
#include "device.hpp"
#include "launch.hpp"

namespace awq4 {

constexpr int W8_N = 128, W8_K = 64;
constexpr int W8_APITCH = W8_K;                  // 64 bytes of a8 per row (4 segments, swizzled)
constexpr int W8_WORDS = (W8_K / 8) * W8_N * 4;  // 8 word rows x 128 columns x 4 B = 4096
constexpr int W8_S3 = 2 * W8_N * 2;              // s3 of the stage's two 32-k halves: 2 x 128 x fp16
constexpr int W8_BBYTES = W8_WORDS + W8_S3;      // 4608 per word buffer
constexpr int W8_ABUFS = 2, W8_BBUFS = 3;

template <int MT>
struct W8Tile {
    static constexpr int M = 32 * MT;
    static constexpr int ABYTES = M * W8_APITCH;
    static constexpr int LDS = W8_ABUFS * ABYTES + W8_BBUFS * W8_BBYTES;
};

// a8 rows: 16-byte segment s of row r is stored at s ^ ((r >> 1) & 3), so the
// 8 rows read by a lane octet fall on 8 distinct 16-byte bank groups.
__device__ __forceinline__ int a8seg(int r, int s) { return s ^ ((r >> 1) & 3); }

__device__ __forceinline__ void dma16_w8(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// int8 B operand of one column from two consecutive K8 words (16 k).
//  per-channel: bytes = 16*q; per-group: bytes = q*s3 (s3 in 1..16), via
//  u = q + 8 in 0..15: u*s3 + (128 - 8*s3) stays in 0..240 per byte, and
//  flipping bit 7 subtracts 128.
template <bool GROUP>
__device__ __forceinline__ u32x4 b8_operand(uint32_t w0, uint32_t w1, uint32_t s3) {
    u32x4 b;
    if (!GROUP) {
        b[0] = (w0 << 4) & 0xF0F0F0F0u;
        b[1] = w0 & 0xF0F0F0F0u;
        b[2] = (w1 << 4) & 0xF0F0F0F0u;
        b[3] = w1 & 0xF0F0F0F0u;
    } else {
        const uint32_t c = (128u - 8u * s3) * 0x01010101u;
        const uint32_t u0 = w0 ^ 0x88888888u, u1 = w1 ^ 0x88888888u;
        b[0] = ((u0 & 0x0F0F0F0Fu) * s3 + c) ^ 0x80808080u;
        b[1] = (((u0 >> 4) & 0x0F0F0F0Fu) * s3 + c) ^ 0x80808080u;
        b[2] = ((u1 & 0x0F0F0F0Fu) * s3 + c) ^ 0x80808080u;
        b[3] = (((u1 >> 4) & 0x0F0F0F0Fu) * s3 + c) ^ 0x80808080u;
    }
    return b;
}

template <int MT, bool GROUP>
__global__ __launch_bounds__(256, 2) void w4a8_gemm_lds(const int8_t *__restrict__ a8, const uint32_t *__restrict__ bq,
                                                       const float *__restrict__ s1, const uint16_t *__restrict__ s2,
                                                       const uint16_t *__restrict__ s3, uint16_t *__restrict__ y,
                                                       int32_t *__restrict__ acc_out, uint64_t *__restrict__ acc64,
                                                       int M, int N, int K, int G, int S) {
    using T = W8Tile<MT>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[T::LDS];
    unsigned char *const Abase = lds;
    unsigned char *const Bbase = lds + W8_ABUFS * T::ABYTES;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
    const int m0 = tm * T::M, n0 = tn * W8_N;
    const int Tst = K / W8_K;
    const int s_lo = (int)((int64_t)Tst * split / S), s_hi = (int)((int64_t)Tst * (split + 1) / S);

    // Copy assignment.  a8: wave w copies rows (M/4) w + 16 i + lane/4, lane%4
    // being the stored segment position; rows past M repeat row M-1 (their
    // outputs are never stored).  Words: wave w copies word rows 2w and 2w+1,
    // lane%32 being the 4-column segment; columns past N repeat the last 4.
    constexpr int AROWS_W = T::M / 4;  // rows per wave
    constexpr int ACOPIES = AROWS_W / 16;
    const int8_t *const ag = a8 + (size_t)m0 * K;
    uint32_t aoff[ACOPIES];
#pragma unroll
    for (int i = 0; i < ACOPIES; ++i) {
        const int r = AROWS_W * wave + 16 * i + (lane >> 2);
        const int m = min(m0 + r, M - 1);
        aoff[i] = (uint32_t)((m - m0) * K + 16 * a8seg(r, lane & 3));
    }
    uint32_t boff;
    {
        const int r = 2 * wave + (lane >> 5);
        const int c = min(n0 + 4 * (lane & 31), N - 4);
        boff = (uint32_t)(r * N + c);
    }
    // s3 (grouped): wave 0 lanes 0..31, half h = lane/16, 8 columns each
    const int s3_h = (lane >> 4) & 1;
    const int s3_c = min(n0 + 8 * (lane & 15), N - 8);

    auto copyA = [&](int st, int buf) {
        const int8_t *src = ag + (size_t)st * W8_K;
        unsigned char *dst = Abase + buf * T::ABYTES + AROWS_W * wave * W8_APITCH;
#pragma unroll
        for (int i = 0; i < ACOPIES; ++i) dma16_w8(src + aoff[i], dst + 16 * i * W8_APITCH);
    };
    auto copyB = [&](int st) {
        unsigned char *dst = Bbase + (st % W8_BBUFS) * W8_BBYTES;
        dma16_w8(bq + (size_t)st * (W8_K / 8) * N + boff, dst + 2 * wave * (W8_N * 4));
        if (GROUP && wave == 0 && lane < 32) {
            const int g = (st * W8_K + 32 * s3_h) / G;
            dma16_w8(s3 + (size_t)g * N + s3_c, dst + W8_WORDS);
        }
    };

    i32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[mt][u] = (i32x4){0, 0, 0, 0};

    const int cl = 64 * wn + 4 * j;  // this lane's first column within the tile
    if (s_lo < s_hi) {
        copyB(s_lo);
        copyA(s_lo, 0);
        if (s_lo + 1 < s_hi) copyB(s_lo + 1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }
    for (int st = s_lo; st < s_hi; ++st) {
        const int abuf = (st - s_lo) & 1;
        if (st + 1 < s_hi) copyA(st + 1, abuf ^ 1);
        if (st + 2 < s_hi) copyB(st + 2);
        const unsigned char *A = Abase + abuf * T::ABYTES;
        const unsigned char *B = Bbase + (st % W8_BBUFS) * W8_BBYTES;
        const u32x4 w0 = *(const u32x4 *)(B + (2 * gq) * (W8_N * 4) + cl * 4);
        const u32x4 w1 = *(const u32x4 *)(B + (2 * gq + 1) * (W8_N * 4) + cl * 4);
        uint32_t g3[4] = {16u, 16u, 16u, 16u};
        if (GROUP) {
            const u32x2 sv = *(const u32x2 *)(B + W8_WORDS + (gq >> 1) * (W8_N * 2) + cl * 2);
#pragma unroll
            for (int u = 0; u < 4; ++u) g3[u] = (uint32_t)f16_bits_to_f32((sv[u >> 1] >> (16 * (u & 1))) & 0xFFFFu);
        }
        u32x4 a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int r = wm * 16 * MT + 16 * mt + j;
            a[mt] = *(const u32x4 *)(A + r * W8_APITCH + a8seg(r, gq) * 16);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 bop = b8_operand<GROUP>(w0[u], w1[u], g3[u]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt][u] = mfma_i8(a[mt], bop, acc[mt][u]);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

    // Epilogue: lane holds rows m0 + 16 MT wm + 16 mt + 4 gq + r, columns
    // n0 + cl + u (u = 0..3, adjacent).  Per-channel accumulators carry the
    // x16 of the upper-nibble int8 and are divided exactly.
    const int nc = n0 + cl;
    if (nc >= N) return;
    float s2f[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) s2f[u] = f16_bits_to_f32(s2[nc + u]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * 16 * MT + 16 * mt + 4 * gq + r;
            if (m >= M) continue;
            const float s1m = s1[m];
            if (S == 1) {
                int32_t v[4];
                uint16_t o[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    v[u] = GROUP ? acc[mt][u][r] : (acc[mt][u][r] >> 4);
                    o[u] = bit_as<uint16_t>((f16)((float)v[u] * s1m * s2f[u]));
                }
                *(u32x2 *)(y + (size_t)m * N + nc) = (u32x2){(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                             (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
                if (acc_out) *(i32x4 *)(acc_out + (size_t)m * N + nc) = (i32x4){v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    int64_t sum;
                    if (splitk_contribute(&acc64[(size_t)m * N + nc + u], acc[mt][u][r], S, &sum)) {
                        const int32_t v = GROUP ? (int32_t)sum : ((int32_t)sum >> 4);
                        y[(size_t)m * N + nc + u] = bit_as<uint16_t>((f16)((float)v * s1m * s2f[u]));
                        if (acc_out) acc_out[(size_t)m * N + nc + u] = v;
                    }
                }
            }
        }
}

template <int MT, bool GROUP>
static hipError_t launch_lds8(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    hipLaunchKernelGGL((w4a8_gemm_lds<MT, GROUP>), dim3(p.tiles_n, p.tiles_m, p.splits), dim3(256), 0, st, a.a8,
                       (const uint32_t *)a.b, a.s1, (const uint16_t *)a.s2, (const uint16_t *)a.s3,
                       (uint16_t *)a.y, a.acc_out, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits);
    return hipGetLastError();
}

hipError_t launch_w4a8_gemm_lds(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    const bool grp = a.s3 != nullptr;
    switch (p.mt) {
        case 4: return grp ? launch_lds8<4, true>(a, p, st) : launch_lds8<4, false>(a, p, st);
        case 8: return grp ? launch_lds8<8, true>(a, p, st) : launch_lds8<8, false>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace awq4
