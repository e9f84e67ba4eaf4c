// w4a8.hip -- QQQ-style W4A8 kernels for gfx950.
//
// Method (vLLM pull request "Support W4A8 quantization for vllm"): activations
// are quantised per token on the fly (row abs-max / 127 as an fp16 scale s1,
// round half to even, clamp to int8); weights are symmetric int4; the int4 is
// turned into an int8 by placing it in the upper nibble (a x16 that the
// epilogue removes exactly); products accumulate in int32 on the matrix
// cores and split-K partials are reduced in int32 through a temporary
// buffer; s1 (per token) and s2 (per output channel) are applied to the
// output.  Grouped weights additionally carry integer group scales s3 that
// multiply the int4 value into an int8 (this library's reading of how the
// per-group and per-channel scales combine; see awq4.h).
//
// Weight layout W4A8_LAYOUT_K8: int32 [K/8, N]; nibble i of word [kb][n]
// holds k = 8kb + {0,4,1,5,2,6,3,7}[i], two's complement, so
//   (w << 4) & 0xF0F0F0F0  -> bytes 0..3 = 16*q for k = 8kb + 0..3
//    w       & 0xF0F0F0F0  -> bytes 0..3 = 16*q for k = 8kb + 4..7
// and two consecutive words give a lane the 16 consecutive k bytes that one
// v_mfma_i32_16x16x64_i8 B operand needs.  Lane j of a wave loads 16 bytes =
// 4 consecutive columns per k-row; column i of those becomes B column j of
// the i-th MFMA (output column = 4*j + i within a 64-column set).
#include "device.hpp"
#include "launch.hpp"

namespace awq4 {

// Rounding an fp32 value to the activation type (nearest even) and back.
template <int DT>
__device__ __forceinline__ float round_to_act(float v) {
    return DT == DT_F16 ? (float)(f16)v : (float)(__bf16)v;
}

// ---------------------------------------------------------------------------
// Activation quantisation, general form (any K): one workgroup (256 threads)
// per row, two passes over the row.  fp16 or bf16 activations (for both,
// the order of finite magnitudes is the order of the low 15 bits).
template <int DT>
__global__ __launch_bounds__(256) void w4a8_quant_kernel(const uint16_t *__restrict__ x, int8_t *__restrict__ a8,
                                                         float *__restrict__ s1, int K) {
    __shared__ uint32_t wmax[4];
    const int m = blockIdx.x;
    const uint16_t *row = x + (size_t)m * K;
    int8_t *out = a8 + (size_t)m * K;
    const int K8 = (K & 7) ? 0 : K;  // vector path only when every row is 16-byte aligned
    // |x| as an integer: for finite fp16 the magnitude order equals the order of the low 15 bits.
    uint32_t mx = 0;
    for (int k = 8 * threadIdx.x; k < K8; k += 8 * 256) {
        u32x4 v = *(const u32x4 *)(row + k);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            mx = max(mx, v[p] & 0x7FFFu);
            mx = max(mx, (v[p] >> 16) & 0x7FFFu);
        }
    }
    for (int k = K8 + threadIdx.x; k < K; k += 256) mx = max(mx, (uint32_t)row[k] & 0x7FFFu);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float amax = act_bits_to_f32<DT>(mx);
    const float q32 = amax / 127.0f;        // correctly rounded fp32 divide
    const float s = round_to_act<DT>(q32);  // to the activation type (nearest even) and back
    if (threadIdx.x == 0) s1[m] = s;
    for (int k = 8 * threadIdx.x; k < K8; k += 8 * 256) {
        u32x4 v = *(const u32x4 *)(row + k);
        u32x2 o = {0, 0};
        if (s != 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                float r = rintf(act_bits_to_f32<DT>(h) / s);
                r = fminf(fmaxf(r, -128.0f), 127.0f);
                o[e >> 2] |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * (e & 3));
            }
        }
        *(u32x2 *)(out + k) = o;
    }
    for (int k = K8 + threadIdx.x; k < K; k += 256) {
        float r = 0.0f;
        if (s != 0.0f) r = fminf(fmaxf(rintf(act_bits_to_f32<DT>(row[k]) / s), -128.0f), 127.0f);
        out[k] = (int8_t)r;
    }
}

// int8 codes of 8 fp16 or bf16 values (one 16-byte chunk) for the scale s,
// given r ~ 1/s: round half to even of x / s, clamped to int8, without a
// divide.  For x and s of one 16-bit type the exact quotient is a half-integer
// or at least 2^-12 (fp16) / 2^-9 (bf16) from one, and x * r (r within a few
// ulps of 1/s) stays within 2^-15 of it.
// One FMA adds 1536, which rounds x * r to a multiple of 2^-13 (the fp32
// spacing in [1024, 2048)): exact ties land on the half-integer, every other
// quotient stays on its own side of it.  The clamp is taken in that shifted
// range; adding 1.5 * 2^23 - 1536 then rounds to an integer (half to even)
// held in the low mantissa bits, so the low byte of the sum's bits is the
// int8 code.  Checked exhaustively against the correctly rounded fp32 divide
// for every reachable s (bf16: every s >= 2^-126, whose reciprocal is a normal
// fp32 value; smaller scales take the divide), every x and reciprocals up to
// 3 ulps off.
template <int DT>
__device__ __forceinline__ u32x2 quant8(u32x4 v, float r) {
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float f = act_bits_to_f32<DT>((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(f, r, 1536.0f), 1536.0f - 128.0f, 1536.0f + 127.0f);
        b[e] = bit_as<uint32_t>(t + (12582912.0f - 1536.0f));
    }
    u32x2 o;
#pragma unroll
    for (int w = 0; w < 2; ++w)  // low bytes of b[4w .. 4w+3]
        o[w] = perm_b32(b[4 * w + 1], b[4 * w], 0x0C0C0400u) | perm_b32(b[4 * w + 3], b[4 * w + 2], 0x04000C0Cu);
    return o;
}

// The same codes through the correctly rounded fp32 divide (bf16 scales
// below 2^-126, whose reciprocal is not a normal fp32 value).
template <int DT>
__device__ __forceinline__ u32x2 quant8_div(u32x4 v, float s) {
    u32x2 o = {0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t h = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const float qf = fminf(fmaxf(rintf(act_bits_to_f32<DT>(h) / s), -128.0f), 127.0f);
        o[e >> 2] |= ((uint32_t)(int32_t)qf & 0xFFu) << (8 * (e & 3));
    }
    return o;
}

// Register-resident quantisation: one workgroup of T threads per row, each
// thread holding NV chunks of 8 values (row length K <= 8 * NV * T, K % 8 ==
// 0), so the row is read from memory once.
// Both types use the divide-free rounding above, except bf16 rows whose
// scale is below 2^-126 (a subnormal fp32 value), which divide.
template <int DT, int NV, int T>
__global__ __launch_bounds__(T) void w4a8_quant_rows(const uint16_t *__restrict__ x, int8_t *__restrict__ a8,
                                                     float *__restrict__ s1, int K) {
    __shared__ uint32_t wmax[T / 64];
    const int m = blockIdx.x;
    const uint16_t *row = x + (size_t)m * K;
    int8_t *out = a8 + (size_t)m * K;
    u32x4 v[NV];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int k = 8 * (threadIdx.x + i * T);
        v[i] = k < K ? *(const u32x4 *)(row + k) : (u32x4){0, 0, 0, 0};
#pragma unroll
        for (int p = 0; p < 4; ++p) mx = max(mx, max(v[i][p] & 0x7FFFu, (v[i][p] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = wmax[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) mx = max(mx, wmax[w]);
    const float amax = act_bits_to_f32<DT>(mx);
    const float q32 = amax / 127.0f;       // correctly rounded fp32 divide, once per row
    const float s = round_to_act<DT>(q32);  // to the activation type (nearest even) and back
    if (threadIdx.x == 0) s1[m] = s;
    const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int k = 8 * (threadIdx.x + i * T);
        if (k >= K) break;
        u32x2 o = {0, 0};
        if (s != 0.0f) {
            o = (DT == DT_F16 || s >= 0x1p-126f) ? quant8<DT>(v[i], r) : quant8_div<DT>(v[i], s);
        }
        *(u32x2 *)(out + k) = o;
    }
}

template <int NV, int T>
static hipError_t launch_quant_rows(const void *x, int8_t *a8, float *s1, int64_t M, int64_t K, int dt,
                                    hipStream_t st) {
    if (dt == DT_BF16)
        hipLaunchKernelGGL((w4a8_quant_rows<DT_BF16, NV, T>), dim3((unsigned)M), dim3(T), 0, st, (const uint16_t *)x,
                           a8, s1, (int)K);
    else
        hipLaunchKernelGGL((w4a8_quant_rows<DT_F16, NV, T>), dim3((unsigned)M), dim3(T), 0, st, (const uint16_t *)x,
                           a8, s1, (int)K);
    return hipGetLastError();
}

hipError_t launch_w4a8_quant(const void *x, int8_t *a8, float *s1, int64_t M, int64_t K, int dt, hipStream_t st) {
    if (K % 8 == 0) {
        if (K <= 8 * 256 * 4) {
            switch ((K + 2047) / 2048) {
                case 1: return launch_quant_rows<1, 256>(x, a8, s1, M, K, dt, st);
                case 2: return launch_quant_rows<2, 256>(x, a8, s1, M, K, dt, st);
                case 3: return launch_quant_rows<3, 256>(x, a8, s1, M, K, dt, st);
                default: return launch_quant_rows<4, 256>(x, a8, s1, M, K, dt, st);
            }
        }
        if (K <= 8 * 1024 * 16) {
            const int64_t nv = (K + 8191) / 8192;
            if (nv <= 2) return launch_quant_rows<2, 1024>(x, a8, s1, M, K, dt, st);
            if (nv <= 3) return launch_quant_rows<3, 1024>(x, a8, s1, M, K, dt, st);
            if (nv <= 4) return launch_quant_rows<4, 1024>(x, a8, s1, M, K, dt, st);
            if (nv <= 6) return launch_quant_rows<6, 1024>(x, a8, s1, M, K, dt, st);
            if (nv <= 8) return launch_quant_rows<8, 1024>(x, a8, s1, M, K, dt, st);
            if (nv <= 12) return launch_quant_rows<12, 1024>(x, a8, s1, M, K, dt, st);
            return launch_quant_rows<16, 1024>(x, a8, s1, M, K, dt, st);
        }
    }
    if (dt == DT_BF16)
        hipLaunchKernelGGL(w4a8_quant_kernel<DT_BF16>, dim3((unsigned)M), dim3(256), 0, st, (const uint16_t *)x, a8, s1,
                           (int)K);
    else
        hipLaunchKernelGGL(w4a8_quant_kernel<DT_F16>, dim3((unsigned)M), dim3(256), 0, st, (const uint16_t *)x, a8, s1,
                           (int)K);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ uint32_t s3_int(const uint16_t *__restrict__ s3, size_t idx) {
    return (uint32_t)act_bits_to_f32<DT>(s3[idx]);
}

// Final value of one output: undo the x16 of per-channel weights, scale, store
// (s2 and y in the activation type).
template <bool GROUP, int DT>
__device__ __forceinline__ void w4a8_store_s(int32_t acc, int m, int n, int N, float s1m,
                                             const uint16_t *__restrict__ s2, uint16_t *__restrict__ y,
                                             int32_t *__restrict__ acc_out) {
    const int32_t a = GROUP ? acc : (acc >> 4);  // exact: per-channel acc is a multiple of 16
    const float v = (float)a * s1m * act_bits_to_f32<DT>(s2[n]);
    y[(size_t)m * N + n] = f32_to_out_bits(v, DT);
    if (acc_out) acc_out[(size_t)m * N + n] = a;
}
template <bool GROUP, int DT>
__device__ __forceinline__ void w4a8_store(int32_t acc, int m, int n, int N, const float *__restrict__ s1,
                                           const uint16_t *__restrict__ s2, uint16_t *__restrict__ y,
                                           int32_t *__restrict__ acc_out) {
    const int32_t a = GROUP ? acc : (acc >> 4);  // exact: per-channel acc is a multiple of 16
    const float v = (float)a * s1[m] * act_bits_to_f32<DT>(s2[n]);
    y[(size_t)m * N + n] = f32_to_out_bits(v, DT);
    if (acc_out) acc_out[(size_t)m * N + n] = a;
}

// ---------------------------------------------------------------------------
// Skinny W4A8 kernel: M <= 16*MT; 4 waves split the K slice of a 64*BLK
// column tile; LDS reduce (int32, exact); split-K over grid y through exact
// counting atomics (device.hpp).
//
// FUSED (M <= 16, the activation rows small enough to read whole per
// workgroup): the kernel takes the fp16 activations x instead of a8 and does
// the per-token quantisation itself, with exactly the arithmetic of
// w4a8_quant_rows.  Every workgroup reduces the abs-max of all M rows (an LDS
// max over its 256 threads), derives s1, and each wave quantises the rows'
// values of its own K range cooperatively (one 8-value chunk per lane at a
// time) into LDS, from where its main loop reads the int8 operands.  The
// int8 activations never go through HBM and the separate launch disappears.
// Workgroup (0, 0) writes s1.  Dynamic LDS: the reduction area, then 32 row
// maxima and 32 scales, then per wave `qa_stride` bytes of int8 rows laid out
// [step][row][64].
template <int BLK, int MT, bool GROUP, bool FUSED, int DT>
__global__ __launch_bounds__(256) void w4a8_skinny(const int8_t *__restrict__ a8, const uint16_t *__restrict__ x16,
                                                   const uint32_t *__restrict__ bq,
                                                   const float *__restrict__ s1, float *__restrict__ s1_out,
                                                   const uint16_t *__restrict__ s2,
                                                   const uint16_t *__restrict__ s3, uint16_t *__restrict__ y,
                                                   int32_t *__restrict__ acc_out, uint64_t *__restrict__ acc64,
                                                   int M, int N, int K, int G, int S, int qa_stride) {
    extern __shared__ int32_t ired[];
    constexpr int COLS = 64 * BLK;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int T = K >> 6;  // 64-k steps
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);
    const int w_lo = s_lo + (s_hi - s_lo) * wave / 4, w_hi = s_lo + (s_hi - s_lo) * (wave + 1) / 4;
    uint32_t *const rmax = (uint32_t *)(ired + 4 * M * COLS);
    float *const srow = (float *)(rmax + 32);
    unsigned char *const qa = (unsigned char *)(srow + 32) + (size_t)wave * qa_stride;
    int ncol[BLK];
    bool ok[BLK];
#pragma unroll
    for (int b = 0; b < BLK; ++b) {
        ncol[b] = tile * COLS + 64 * b + 4 * j;
        ok[b] = ncol[b] < N;  // N % 8 == 0 and the 4 columns start at a multiple of 4
    }
    // words of 64-k step st for this lane's 4 columns of each set (zero past N)
    auto load_w = [&](int st, u32x4 (&w0)[BLK], u32x4 (&w1)[BLK]) {
        const int kb = (st * 64 + 16 * gq) >> 3;
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            if (ok[b]) {
                w0[b] = __builtin_nontemporal_load((const u32x4 *)(bq + (size_t)kb * N + ncol[b]));
                w1[b] = __builtin_nontemporal_load((const u32x4 *)(bq + (size_t)(kb + 1) * N + ncol[b]));
            } else {
                w0[b] = (u32x4){0, 0, 0, 0};
                w1[b] = (u32x4){0, 0, 0, 0};
            }
        }
    };
    if (FUSED) {
        if (threadIdx.x < 32) rmax[threadIdx.x] = 0;
        __syncthreads();
        // |x| as an integer: for finite fp16 and bf16 the magnitude order
        // equals the order of the low 15 bits
        const int K8 = K >> 3;
        for (int m = 0; m < M; ++m) {
            uint32_t mx = 0;
            for (int c = threadIdx.x; c < K8; c += 256) {
                const u32x4 v = *(const u32x4 *)(x16 + (size_t)m * K + 8 * c);
#pragma unroll
                for (int p = 0; p < 4; ++p) mx = max(mx, max(v[p] & 0x7FFFu, (v[p] >> 16) & 0x7FFFu));
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
            if (lane == 0) atomicMax(&rmax[m], mx);
        }
        __syncthreads();
        if (threadIdx.x < M) {
            const float amax = act_bits_to_f32<DT>(rmax[threadIdx.x]);
            const float q32 = amax / 127.0f;       // correctly rounded fp32 divide
            const float sv = round_to_act<DT>(q32);  // to the activation type (nearest even) and back
            srow[threadIdx.x] = sv;
            if (tile == 0 && split == 0) s1_out[threadIdx.x] = sv;
        }
        __syncthreads();
        // this wave's K range, row by row, 8 values per lane and chunk
        const int nst = w_hi - w_lo, per_row = nst * 8;
        for (int c = lane; c < M * per_row; c += 64) {
            const int m = c / per_row, cc = c - m * per_row;
            const u32x4 v = *(const u32x4 *)(x16 + (size_t)m * K + 64 * w_lo + 8 * cc);
            const float sv = srow[m];
            u32x2 o = {0, 0};
            if (sv != 0.0f)
                o = (DT == DT_F16 || sv >= 0x1p-126f) ? quant8<DT>(v, __builtin_amdgcn_rcpf(sv)) : quant8_div<DT>(v, sv);
            *(u32x2 *)(qa + ((size_t)(cc >> 3) * M + m) * 64 + (cc & 7) * 8) = o;
        }
    }
    i32x4 acc[MT][BLK][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int b = 0; b < BLK; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][b][i] = (i32x4){0, 0, 0, 0};

    for (int st = w_lo; st < w_hi; ++st) {
        const int k0 = st * 64 + 16 * gq;  // this lane group's 16 k
        u32x4 w0[BLK], w1[BLK];
        load_w(st, w0, w1);
        u32x4 a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + j;
            if (m >= M) a[mt] = (u32x4){0, 0, 0, 0};
            else if (FUSED) a[mt] = *(const u32x4 *)(qa + ((size_t)(st - w_lo) * M + m) * 64 + 16 * gq);
            else a[mt] = *(const u32x4 *)(a8 + (size_t)m * K + k0);
        }
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            uint32_t g3[4] = {16, 16, 16, 16};
            if (GROUP && ok[b]) {
                const size_t gi = (size_t)(k0 / G) * N + ncol[b];
#pragma unroll
                for (int i = 0; i < 4; ++i) g3[i] = s3_int<DT>(s3, gi + i);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 bop = int8_b_operand<GROUP>(w0[b][i], w1[b][i], g3[i]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][b][i] = mfma_i8(a[mt], bop, acc[mt][b][i]);
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * mt + 4 * gq + r;
            if (m < M) {
#pragma unroll
                for (int b = 0; b < BLK; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ired[((size_t)wave * M + m) * COLS + 64 * b + 4 * j + i] = acc[mt][b][i][r];
            }
        }
    __syncthreads();
    const int total = M * COLS;
    const int n_base = tile * COLS;
    // split-K: per-element counting atomics (one round trip at the end)
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int m = idx / COLS, c = idx - m * COLS;
        const int32_t v = ired[(size_t)(0 * M + m) * COLS + c] + ired[(size_t)(1 * M + m) * COLS + c] +
                          ired[(size_t)(2 * M + m) * COLS + c] + ired[(size_t)(3 * M + m) * COLS + c];
        const int n = n_base + c;
        if (n >= N) continue;
        int64_t sum;
        const float s1m = FUSED ? srow[m] : s1[m];
        if (S == 1)
            w4a8_store_s<GROUP, DT>(v, m, n, N, s1m, s2, y, acc_out);
        else if (splitk_contribute(&acc64[(size_t)m * N + n], v, S, &sum))
            w4a8_store_s<GROUP, DT>((int32_t)sum, m, n, N, s1m, s2, y, acc_out);
    }
}

// ---------------------------------------------------------------------------
// Tiled W4A8 kernel: 2 x 2 waves, wave tile (16*MTW) x 64, workgroup tile
// (32*MTW) x 128; split-K over grid z.
template <int MTW, bool GROUP, int DT>
__global__ __launch_bounds__(256) void w4a8_tiled(const int8_t *__restrict__ a8, const uint32_t *__restrict__ bq,
                                                  const float *__restrict__ s1, const uint16_t *__restrict__ s2,
                                                  const uint16_t *__restrict__ s3, uint16_t *__restrict__ y,
                                                  int32_t *__restrict__ acc_out, uint64_t *__restrict__ acc64,
                                                  int M, int N, int K, int G, int S) {
    constexpr int BM = 32 * MTW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
    const int ncol = tn * 128 + wn * 64 + 4 * j;
    const bool ok = ncol < N;
    const int m0 = tm * BM + wm * 16 * MTW;
    const int T = K >> 6;
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);

    i32x4 acc[MTW][4];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = (i32x4){0, 0, 0, 0};
    bool row_ok[MTW];
    const int8_t *arow[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        const int m = m0 + 16 * mt + j;
        row_ok[mt] = m < M;
        arow[mt] = a8 + (size_t)(row_ok[mt] ? m : 0) * K + 16 * gq;
    }

    for (int st = s_lo; st < s_hi; ++st) {
        const int k0 = st * 64 + 16 * gq;
        const int kb = k0 >> 3;
        u32x4 w0 = {0, 0, 0, 0}, w1 = {0, 0, 0, 0};
        if (ok) {
            w0 = *(const u32x4 *)(bq + (size_t)kb * N + ncol);
            w1 = *(const u32x4 *)(bq + (size_t)(kb + 1) * N + ncol);
        }
        u32x4 a[MTW];
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
            a[mt] = row_ok[mt] ? *(const u32x4 *)(arow[mt] + st * 64) : (u32x4){0, 0, 0, 0};
        uint32_t g3[4] = {16, 16, 16, 16};
        if (GROUP && ok) {
            const size_t gi = (size_t)(k0 / G) * N + ncol;
#pragma unroll
            for (int i = 0; i < 4; ++i) g3[i] = s3_int<DT>(s3, gi + i);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 bop = int8_b_operand<GROUP>(w0[i], w1[i], g3[i]);
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) acc[mt][i] = mfma_i8(a[mt], bop, acc[mt][i]);
        }
    }

    if (S == 1) {
        if (!ok) return;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * gq + r;
                if (m < M) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) w4a8_store<GROUP, DT>(acc[mt][i][r], m, ncol + i, N, s1, s2, y, acc_out);
                }
            }
        return;
    }
    // Split-K by partial tiles exchanged through agent-scope atomics
    // (device.hpp); int32 partials, so the sum is exact in any order.
    uint32_t *const cnt = (uint32_t *)acc64 + (tn + gridDim.x * tm);
    uint64_t *const part = (uint64_t *)((char *)acc64 + split_counters_bytes((int64_t)gridDim.x * gridDim.y));
    const size_t slot = (size_t)M * N / 2;  // 64-bit words per split
    auto at = [&](int sp, int m) { return part + sp * slot + ((size_t)m * N + ncol) / 2; };
    if (ok) {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * gq + r;
                if (m < M) part_put(at(split, m), (i32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]});
            }
    }
    if (!split_tile_last_atomic(cnt, S) || !ok) return;
    // the last split sums the partials one row tile (4 of the lane's rows)
    // at a time, then clears them
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        auto row = [&](int r) { return m0 + 16 * mt + 4 * gq + r; };
        auto addr = [&](int sp, int r) { return at(sp, row(r)); };
        auto valid = [&](int r) { return row(r) < M; };
        i32x4 v[4];
        part_sum<4, 1>(v, S, addr, valid);
        part_clear_all<4>(S, addr, valid);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!valid(r)) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) w4a8_store<GROUP, DT>(v[r][i], row(r), ncol + i, N, s1, s2, y, acc_out);
        }
    }
}

// ---------------------------------------------------------------------------
// int8 rows of one wave's K range in the fused skinny kernel: at most
// ceil(ceil(T / S) / 4) steps of M rows x 64 bytes
int64_t w4a8_fused_qa_stride(int64_t M, int64_t K, int splits) {
    const int64_t T = K / 64, per_wg = (T + splits - 1) / splits;
    return ((per_wg + 3) / 4) * M * 64;
}
size_t w4a8_fused_lds_bytes(int64_t M, int64_t K, int blk, int splits) {
    return (size_t)4 * M * 64 * blk * sizeof(int32_t) + 64 * sizeof(uint32_t) +
           4 * (size_t)w4a8_fused_qa_stride(M, K, splits);
}

template <int BLK, int MT, bool GROUP, bool FUSED, int DT>
static hipError_t launch_skinny8(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    const int qa_stride = FUSED ? (int)w4a8_fused_qa_stride(a.M, a.K, p.splits) : 0;
    const size_t lds = FUSED ? w4a8_fused_lds_bytes(a.M, a.K, BLK, p.splits)
                             : (size_t)4 * a.M * 64 * BLK * sizeof(int32_t);  // wave partials only
    hipLaunchKernelGGL((w4a8_skinny<BLK, MT, GROUP, FUSED, DT>), dim3(p.tiles_n, p.splits), dim3(256), lds, st, a.a8,
                       (const uint16_t *)a.x, (const uint32_t *)a.b, a.s1, a.s1_out, (const uint16_t *)a.s2,
                       (const uint16_t *)a.s3, (uint16_t *)a.y, a.acc_out, p.acc, (int)a.M, (int)a.N, (int)a.K,
                       a.G, p.splits, qa_stride);
    return hipGetLastError();
}

template <int MTW, bool GROUP, int DT>
static hipError_t launch_tiled8(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    hipLaunchKernelGGL((w4a8_tiled<MTW, GROUP, DT>), dim3(p.tiles_n, p.tiles_m, p.splits), dim3(256), 0, st, a.a8,
                       (const uint32_t *)a.b, a.s1, (const uint16_t *)a.s2, (const uint16_t *)a.s3,
                       (uint16_t *)a.y, a.acc_out, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G,
                       p.splits);
    return hipGetLastError();
}

template <bool GROUP, int DT>
static hipError_t launch_w4a8_t(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    if (p.kind == 0) {
        switch (p.blk * 10 + p.mt) {
            case 11: return launch_skinny8<1, 1, GROUP, false, DT>(a, p, st);
            case 21: return launch_skinny8<2, 1, GROUP, false, DT>(a, p, st);
            case 12: return launch_skinny8<1, 2, GROUP, false, DT>(a, p, st);
            case 14: return launch_skinny8<1, 4, GROUP, false, DT>(a, p, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.mt) {
        case 1: return launch_tiled8<1, GROUP, DT>(a, p, st);
        case 2: return launch_tiled8<2, GROUP, DT>(a, p, st);
        case 4: return launch_tiled8<4, GROUP, DT>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_w4a8(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    if (p.kind == 2) return launch_w4a8_gemm_lds(a, p, st);
    const bool grp = a.s3 != nullptr;
    if (a.dtype == DT_BF16)
        return grp ? launch_w4a8_t<true, DT_BF16>(a, p, st) : launch_w4a8_t<false, DT_BF16>(a, p, st);
    return grp ? launch_w4a8_t<true, DT_F16>(a, p, st) : launch_w4a8_t<false, DT_F16>(a, p, st);
}

// The fused quantisation of one fp16 or bf16 token (the same codes as
// w4a8_quant_rows, through the same rounding).
template <int DT>
static hipError_t launch_w4a8_fused_t(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    const bool grp = a.s3 != nullptr;
    if (p.blk == 2)
        return grp ? launch_skinny8<2, 1, true, true, DT>(a, p, st) : launch_skinny8<2, 1, false, true, DT>(a, p, st);
    return grp ? launch_skinny8<1, 1, true, true, DT>(a, p, st) : launch_skinny8<1, 1, false, true, DT>(a, p, st);
}

hipError_t launch_w4a8_fused(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    if (p.kind != 0 || p.mt != 1) return hipErrorInvalidValue;
    return a.dtype == DT_BF16 ? launch_w4a8_fused_t<DT_BF16>(a, p, st) : launch_w4a8_fused_t<DT_F16>(a, p, st);
}

}  // namespace awq4
