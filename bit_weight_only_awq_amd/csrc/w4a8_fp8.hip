// w4a8_fp8.hip -- INT4-FP8 W4A8 on gfx950: per-token OCP FP8 (E4M3)
// activations x symmetric int4 weights on the fp8 matrix cores.
//
// The QQQ pull request "Support W4A8 quantization for vllm" names "INT4-FP8
// QQQ (W4A8)" as its authors' next step and says nothing more; this library's
// reading is the int8 recipe of that page with E4M3 codes and 448 (the largest
// finite E4M3 value) in place of int8 codes and 127, rounded to nearest even
// and saturated at +-448, per-channel weight scales:
//   s1[m]    = act(amax_m / 448)                  (fp32 divide, rounded to the activation type)
//   a[m,k]   = e4m3(clamp(x[m,k] / s1[m], +-448))  (fp32 divide)
//   y[m,n]   = act((sum_k a[m,k] q[k,n]) * s1[m] * s2[n])
//
// Weights: the W4A8 K-packed layout.  The matrix cores take the weights as
// E4M3 *codes equal to the offset-binary nibble u = q + 8*: a code u in 0..15
// is the value u * 2^-9 (subnormal below 8, the lowest binade from 8 on), so
// the B operand is two masks per packed word, as for int8, and the products
// a * u * 2^-9 are exact.  The epilogue turns the sum back into
// sum a q = 2^9 * sum(a u 2^-9) - 8 * sum_k a, with the row sums of the
// activation codes (asum) that the quantiser writes beside s1.
//
// Matrix-core operand model (v_mfma_scale_f32_16x16x128_f8f6f4, unit scales):
// lane l supplies row / column l % 16 and 32 consecutive k, chunk l / 16, as
// eight registers of four codes; the C layout is that of the 16x16 MFMAs.
#include "device.hpp"
#include "fp8_ops.hpp"
#include "launch.hpp"

namespace awq4 {

// E4M3 code of |q| <= 448 (not NaN), round to nearest, ties to even.
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    const uint32_t u = bit_as<uint32_t>(q);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a < 0x3C800000u) {
        // below 2^-6: multiples of 2^-9 (the scaling by 512 is exact)
        code = (uint32_t)__builtin_rintf(bit_as<float>(a) * 512.0f);
    } else {
        // round the fp32 significand to 3 bits (nearest even), then rebias
        // the exponent from 127 to 7; a carry moves into the exponent
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - ((127u - 7u) << 3);
    }
    return sign | code;
}

// Value of an E4M3 code in units of 2^-9 (an exact integer, |v| <= 229376).
__device__ __forceinline__ int32_t e4m3_units(uint32_t c) {
    const int32_t e = (c >> 3) & 15, m = c & 7;
    const int32_t v = e == 0 ? m : (8 + m) << (e - 1);
    return (c & 0x80u) ? -v : v;
}

template <int DT>
__device__ __forceinline__ float round_act_f(float v) {
    return DT == DT_F16 ? (float)(f16)v : (float)(__bf16)v;
}

// ---------------------------------------------------------------------------
// The quotient x / s without a divide per value.  Per row: r = RN(1 / s') by
// one divide; per value q0 = RN(x' r), e = x' - q0 s' (exact, one FMA) and
// q = RN(q0 + e r), Markstein's correction, which is the correctly rounded
// quotient when nothing underflows; x' and s' are x and s times 2^64 on bf16
// rows with s < 2^-60 (exact, the same quotient), so that every x whose
// quotient can reach the smallest E4M3 subnormal stays far above the range
// where e would round.  Checked on the host for every scale the quantiser can
// produce and every fp16 / bf16 value it can meet: the E4M3 code of the
// clamped q equals that of the clamped correctly rounded quotient in every
// case.  Rows with s = 0, s below 2^-126 (bf16 only) or s not finite take
// the divide.
template <int DT>
struct Fp8Quotient {
    float sc, ss, r;
    bool exact_divide;
    __device__ __forceinline__ explicit Fp8Quotient(float s) {
        sc = (DT == DT_BF16 && s < 0x1p-60f) ? 0x1p64f : 1.0f;
        ss = s * sc;
        exact_divide = !(s >= 0x1p-126f && s <= 3.4028234663852886e38f);
        r = exact_divide ? 0.0f : 1.0f / ss;
    }
    // clamp(x / s, +-448) for exact_divide == false.  The sign is x's: the
    // correction can turn a zero quotient's sign (-0 + 0 = +0), and the E4M3
    // code keeps it.
    __device__ __forceinline__ float q(float x) const {
        const float xs = DT == DT_BF16 ? x * sc : x;
        const float q0 = xs * r;
        const float e = __builtin_fmaf(-q0, ss, xs);
        return __builtin_amdgcn_fmed3f(__builtin_copysignf(__builtin_fmaf(e, r, q0), x), -448.0f, 448.0f);
    }
};

// E4M3 codes of the clamped quotients of four 16-bit activation patterns
// (h01: values 0, 1 in its halves; h23: values 2, 3), one byte each, by the
// matrix-core generation's fp32 -> OCP E4M3 conversion (round to nearest
// even; the same code as e4m3_code for every |q| <= 448, both signs,
// subnormals included -- checked on the device over all such fp32 values).
template <int DT>
__device__ __forceinline__ uint32_t fp8_codes4(const Fp8Quotient<DT> &f, uint32_t h01, uint32_t h23) {
    const float q0 = f.q(act_bits_to_f32<DT>(h01 & 0xFFFFu)), q1 = f.q(act_bits_to_f32<DT>(h01 >> 16));
    const float q2 = f.q(act_bits_to_f32<DT>(h23 & 0xFFFFu)), q3 = f.q(act_bits_to_f32<DT>(h23 >> 16));
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, lo, true);
}

// Sum of the values of eight E4M3 codes (one a byte of lo, hi), in units of
// 2^-9, through the hardware's fp8 -> fp32 decode (the same OCP E4M3 format
// as the encode above).  Exact: every value is a multiple of 2^-9 of
// magnitude at most 448, so every partial sum of the eight is a multiple of
// 2^-9 below 2^24 units and fp32 holds it.
__device__ __forceinline__ int32_t e4m3_units8(uint32_t lo, uint32_t hi) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    const float v = ((a[0] + a[1]) + (b[0] + b[1])) + ((c[0] + c[1]) + (d[0] + d[1]));
    return (int32_t)(v * 512.0f);
}

// ---------------------------------------------------------------------------
// Quantisation: one workgroup of 256 threads per row, two passes over the row
// (abs-max, then codes).  The row sum of the codes' values is accumulated
// exactly as an integer in units of 2^-9 and rounded once to fp32.
template <int DT>
__global__ __launch_bounds__(256) void w4a8_fp8_quant(const uint16_t *__restrict__ x, uint8_t *__restrict__ a,
                                                      float *__restrict__ s1, float *__restrict__ asum, int K) {
    __shared__ uint32_t wmax[4];
    __shared__ long long wsum[4];
    const int m = blockIdx.x;
    const uint16_t *row = x + (size_t)m * K;
    uint8_t *out = a + (size_t)m * K;
    const int K8 = (K & 7) ? 0 : K;
    uint32_t mx = 0;
    for (int k = 8 * threadIdx.x; k < K8; k += 8 * 256) {
        const u32x4 v = *(const u32x4 *)(row + k);
#pragma unroll
        for (int p = 0; p < 4; ++p) mx = max(mx, max(v[p] & 0x7FFFu, (v[p] >> 16) & 0x7FFFu));
    }
    for (int k = K8 + threadIdx.x; k < K; k += 256) mx = max(mx, (uint32_t)row[k] & 0x7FFFu);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float amax = act_bits_to_f32<DT>(mx);
    const float s = round_act_f<DT>(amax / 448.0f);  // correctly rounded fp32 divide, then the activation type
    const Fp8Quotient<DT> fq(s);
    long long sum = 0;
    auto code_of = [&](uint32_t h) -> uint32_t {
        if (s == 0.0f) return 0u;
        if (!fq.exact_divide) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fq.q(act_bits_to_f32<DT>(h)), 0.0f, 0,
                                                                              false) & 0xFFu;
        const float q = fminf(fmaxf(act_bits_to_f32<DT>(h) / s, -448.0f), 448.0f);
        return e4m3_code(q);
    };
    if (s != 0.0f && !fq.exact_divide) {
        // (per thread at most 512 values of at most 229376 units: int32)
        int32_t part = 0;
        for (int k = 8 * threadIdx.x; k < K8; k += 8 * 256) {
            const u32x4 v = *(const u32x4 *)(row + k);
            const u32x2 o = {fp8_codes4<DT>(fq, v[0], v[1]), fp8_codes4<DT>(fq, v[2], v[3])};
            part += e4m3_units8(o[0], o[1]);
            *(u32x2 *)(out + k) = o;
        }
        sum = part;
    } else {
        for (int k = 8 * threadIdx.x; k < K8; k += 8 * 256) {
            const u32x4 v = *(const u32x4 *)(row + k);
            u32x2 o = {0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t c = code_of((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
                sum += e4m3_units(c);
                o[e >> 2] |= c << (8 * (e & 3));
            }
            *(u32x2 *)(out + k) = o;
        }
    }
    for (int k = K8 + threadIdx.x; k < K; k += 256) {
        const uint32_t c = code_of(row[k]);
        sum += e4m3_units(c);
        out[k] = (uint8_t)c;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        const long long tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        s1[m] = s;
        asum[m] = (float)tot * 0x1p-9f;  // one rounding (int64 -> fp32), then an exact power of two
    }
}

// Register-resident form: one workgroup of T threads per row, each thread
// holding NV chunks of 8 values (K % 8 == 0, K <= 8 * NV * T), so the row is
// read from memory once and a single token's row is spread over up to 1024
// threads.
template <int DT, int NV, int T>
__global__ __launch_bounds__(T) void w4a8_fp8_quant_rows(const uint16_t *__restrict__ x, uint8_t *__restrict__ a,
                                                         float *__restrict__ s1, float *__restrict__ asum, int K) {
    __shared__ uint32_t wmax[T / 64];
    __shared__ long long wsum[T / 64];
    const int m = blockIdx.x;
    const uint16_t *row = x + (size_t)m * K;
    uint8_t *out = a + (size_t)m * K;
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
    const float s = round_act_f<DT>(act_bits_to_f32<DT>(mx) / 448.0f);
    const Fp8Quotient<DT> fq(s);
    long long sum = 0;
    if (!fq.exact_divide) {
        int32_t part = 0;  // at most 8 NV values of at most 229376 units
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int k = 8 * (threadIdx.x + i * T);
            if (k >= K) break;
            const u32x2 o = {fp8_codes4<DT>(fq, v[i][0], v[i][1]), fp8_codes4<DT>(fq, v[i][2], v[i][3])};
            part += e4m3_units8(o[0], o[1]);
            *(u32x2 *)(out + k) = o;
        }
        sum = part;
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int k = 8 * (threadIdx.x + i * T);
            if (k >= K) break;
            u32x2 o = {0, 0};
            if (s != 0.0f) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float q = fminf(
                        fmaxf(act_bits_to_f32<DT>((v[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu) / s, -448.0f), 448.0f);
                    const uint32_t c = e4m3_code(q);
                    sum += e4m3_units(c);
                    o[e >> 2] |= c << (8 * (e & 3));
                }
            }
            *(u32x2 *)(out + k) = o;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        long long tot = 0;
#pragma unroll
        for (int w = 0; w < T / 64; ++w) tot += wsum[w];
        s1[m] = s;
        asum[m] = (float)tot * 0x1p-9f;
    }
}

template <int NV, int T>
static hipError_t launch_fp8_rows(const void *x, uint8_t *a, float *s1, float *asum, int64_t M, int64_t K, int dt,
                                  hipStream_t st) {
    if (dt == DT_BF16)
        hipLaunchKernelGGL((w4a8_fp8_quant_rows<DT_BF16, NV, T>), dim3((unsigned)M), dim3(T), 0, st,
                           (const uint16_t *)x, a, s1, asum, (int)K);
    else
        hipLaunchKernelGGL((w4a8_fp8_quant_rows<DT_F16, NV, T>), dim3((unsigned)M), dim3(T), 0, st,
                           (const uint16_t *)x, a, s1, asum, (int)K);
    return hipGetLastError();
}

hipError_t launch_w4a8_fp8_quant(const void *x, uint8_t *a, float *s1, float *asum, int64_t M, int64_t K, int dt,
                                 hipStream_t st) {
    if (K % 8 == 0 && K <= 8 * 1024 * 8) {
        if (K <= 8 * 256 * 2) return launch_fp8_rows<2, 256>(x, a, s1, asum, M, K, dt, st);
        if (K <= 8 * 1024 * 2) return launch_fp8_rows<2, 1024>(x, a, s1, asum, M, K, dt, st);
        if (K <= 8 * 1024 * 4) return launch_fp8_rows<4, 1024>(x, a, s1, asum, M, K, dt, st);
        return launch_fp8_rows<8, 1024>(x, a, s1, asum, M, K, dt, st);
    }
    if (dt == DT_BF16)
        hipLaunchKernelGGL(w4a8_fp8_quant<DT_BF16>, dim3((unsigned)M), dim3(256), 0, st, (const uint16_t *)x, a, s1,
                           asum, (int)K);
    else
        hipLaunchKernelGGL(w4a8_fp8_quant<DT_F16>, dim3((unsigned)M), dim3(256), 0, st, (const uint16_t *)x, a, s1,
                           asum, (int)K);
    return hipGetLastError();
}

// Fixed-point resolution of the split-K sum of t: 2^-20 (range 2^27 > 13.2 K).
constexpr double kFp8Fixed = 1048576.0;

// ---------------------------------------------------------------------------
// Skinny kernel: M <= 16*MT; 4 waves split the K slice of a 64*BLK column tile
// (128-k steps); LDS reduce in wave order; split-K over grid y through the
// counting fixed-point accumulators (device.hpp).
//
// FUSED (one token, M == 1): the quantisation runs inside the kernel.  Every
// workgroup reads the whole activation row for its abs-max, derives s1 as
// the quantiser does (workgroup (0, 0) writes it out), and quantises only its
// own K slice into LDS, from where the main loop reads the codes; the E4M3
// codes never travel through device memory and the separate launch goes.
// The epilogue needs d = sum_k a q = 512 t - 8 asum (t the matrix-core sum,
// asum the row sum of the codes' values), and d is linear in the K slices:
// each workgroup contributes 512 t_s - 8 asum_s of its own slice, so none of
// them needs the whole row's asum.  In the fixed point of the split-K sum
// (2^-20 of t) the asum part, 32 U_s (U_s = asum_s in units of 2^-9), is exact;
// d is then formed once, exactly, and rounded once to fp32 (the two-launch
// path rounds t to fp32 before forming d: the two differ by at most one fp32
// rounding of d).  Dynamic LDS: the reduction area, then the slice's codes.
template <int BLK, int MT, int DT, bool FUSED = false>
__global__ __launch_bounds__(256) void w4a8_fp8_skinny(const uint8_t *__restrict__ a, const uint32_t *__restrict__ bq,
                                                       const float *__restrict__ s1, const float *__restrict__ asum,
                                                       const uint16_t *__restrict__ s2, uint16_t *__restrict__ y,
                                                       float *__restrict__ acc_out, uint64_t *__restrict__ acc64,
                                                       int M, int N, int K, int S,
                                                       const uint16_t *__restrict__ x16 = nullptr,
                                                       float *__restrict__ s1_out = nullptr) {
    extern __shared__ float fred[];
    constexpr int COLS = 64 * BLK;
    static_assert(!FUSED || MT == 1, "the fused quantisation takes one row");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int T = K >> 7;  // 128-k steps
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);
    const int w_lo = s_lo + (s_hi - s_lo) * wave / 4, w_hi = s_lo + (s_hi - s_lo) * (wave + 1) / 4;
    int ncol[BLK];
    bool ok[BLK];
#pragma unroll
    for (int b = 0; b < BLK; ++b) {
        ncol[b] = tile * COLS + 64 * b + 4 * j;
        ok[b] = ncol[b] < N;
    }
    // FUSED: the row's scale, this workgroup's codes (LDS, after the
    // reduction area) and their value sum in units of 2^-9
    uint8_t *const qa = (uint8_t *)(fred + (size_t)4 * M * COLS);
    float s1v = 0.0f;
    int64_t uwg = 0;
    if constexpr (FUSED) {
        __shared__ uint32_t wmax[4];
        __shared__ long long wsum[4];
        uint32_t mx = 0;
        for (int c = threadIdx.x; c < (K >> 3); c += 256) {
            const u32x4 v = *(const u32x4 *)(x16 + 8 * c);
#pragma unroll
            for (int p = 0; p < 4; ++p) mx = max(mx, max(v[p] & 0x7FFFu, (v[p] >> 16) & 0x7FFFu));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
        if (lane == 0) wmax[wave] = mx;
        __syncthreads();
        mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
        // the quantiser's own expressions (w4a8_fp8_quant_rows), so s1 and
        // every code come out the same
        const float s = round_act_f<DT>(act_bits_to_f32<DT>(mx) / 448.0f);
        const Fp8Quotient<DT> fq(s);
        const int k_lo = 128 * s_lo, nc = 16 * (s_hi - s_lo);  // chunks of 8 values
        int32_t part = 0;  // at most ceil(nc / 256) <= 16 chunks of at most 1835008 units
        for (int c = threadIdx.x; c < nc; c += 256) {
            const u32x4 v = *(const u32x4 *)(x16 + k_lo + 8 * c);
            u32x2 o = {0, 0};
            if (!fq.exact_divide) {
                o = (u32x2){fp8_codes4<DT>(fq, v[0], v[1]), fp8_codes4<DT>(fq, v[2], v[3])};
                part += e4m3_units8(o[0], o[1]);
            } else if (s != 0.0f) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float q = fminf(
                        fmaxf(act_bits_to_f32<DT>((v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) / s, -448.0f), 448.0f);
                    const uint32_t cd = e4m3_code(q);
                    part += e4m3_units(cd);
                    o[e >> 2] |= cd << (8 * (e & 3));
                }
            }
            *(u32x2 *)(qa + 8 * c) = o;
        }
        long long sum = part;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
        if (lane == 0) wsum[wave] = sum;
        __syncthreads();
        uwg = (int64_t)wsum[0] + wsum[1] + wsum[2] + wsum[3];
        s1v = s;
        if (tile == 0 && split == 0 && threadIdx.x == 0) s1_out[0] = s;
    }

    f32x4 acc[MT][BLK][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int b = 0; b < BLK; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][b][i] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int st = w_lo; st < w_hi; ++st) {
        const int k0 = st * 128 + 32 * gq;  // this lane group's 32 k
        const int kb = k0 >> 3;
        u32x4 w[BLK][4];
#pragma unroll
        for (int b = 0; b < BLK; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[b][e] = ok[b] ? __builtin_nontemporal_load((const u32x4 *)(bq + (size_t)(kb + e) * N + ncol[b]))
                                : (u32x4){0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        i32x8 av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + j;
            if (m >= M) av[mt] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
            else if (FUSED) av[mt] = *(const i32x8 *)(qa + (k0 - 128 * s_lo));
            else av[mt] = load_a32(a + (size_t)m * K + k0);
        }
#pragma unroll
        for (int b = 0; b < BLK; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const i32x8 bop = fp8_b_operand(w[b][0][i], w[b][1][i], w[b][2][i], w[b][3][i]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][b][i] = mfma_fp8(av[mt], bop, acc[mt][b][i]);
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
                    for (int i = 0; i < 4; ++i) fred[((size_t)wave * M + m) * COLS + 64 * b + 4 * j + i] = acc[mt][b][i][r];
            }
        }
    __syncthreads();
    const int total = M * COLS;
    const int n_base = tile * COLS;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int m = idx / COLS, c = idx - m * COLS;
        const int n = n_base + c;
        if (n >= N) continue;
        const float v = ((fred[(size_t)(0 * M + m) * COLS + c] + fred[(size_t)(1 * M + m) * COLS + c]) +
                         fred[(size_t)(2 * M + m) * COLS + c]) + fred[(size_t)(3 * M + m) * COLS + c];
        if (FUSED) {
            // 512 t - 8 asum of this K slice (U in units of 2^-9: 8 asum = U / 64)
            if (S == 1) {
                fp8_store_d<DT>((float)((double)v * 512.0 - (double)uwg * (1.0 / 64.0)), m, n, N, s1v, s2, y,
                                acc_out);
            } else {
                const double lim = (double)(kBias - 1);
                const double fv = __builtin_rint(fmin(fmax((double)v * kFp8Fixed, -lim), lim)) - 32.0 * (double)uwg;
                const int64_t fx = (int64_t)fmin(fmax(fv, -lim), lim);
                int64_t sum;
                if (splitk_contribute(&acc64[(size_t)m * N + n], fx, S, &sum))
                    fp8_store_d<DT>((float)((double)sum * (512.0 / kFp8Fixed)), m, n, N, s1v, s2, y, acc_out);
            }
        } else if (S == 1) {
            fp8_store<DT>(v, m, n, N, s1, asum, s2, y, acc_out);
        } else {
            const double lim = (double)(kBias - 1);
            const int64_t fx = (int64_t)__builtin_rint(fmin(fmax((double)v * kFp8Fixed, -lim), lim));
            int64_t sum;
            if (splitk_contribute(&acc64[(size_t)m * N + n], fx, S, &sum))
                fp8_store<DT>((float)((double)sum * (1.0 / kFp8Fixed)), m, n, N, s1, asum, s2, y, acc_out);
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel: 2 x 2 waves, wave tile (16*MTW) x 64, workgroup tile
// (32*MTW) x 128; 128-k steps; split-K over grid z through per-tile fp32
// partials summed in split order (device.hpp).
template <int MTW, int DT>
__global__ __launch_bounds__(256) void w4a8_fp8_tiled(const uint8_t *__restrict__ a, const uint32_t *__restrict__ bq,
                                                      const float *__restrict__ s1, const float *__restrict__ asum,
                                                      const uint16_t *__restrict__ s2, uint16_t *__restrict__ y,
                                                      float *__restrict__ acc_out, uint64_t *__restrict__ ws, int M,
                                                      int N, int K, int S) {
    constexpr int BM = 32 * MTW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
    const int ncol = tn * 128 + wn * 64 + 4 * j;
    const bool ok = ncol < N;
    const int m0 = tm * BM + wm * 16 * MTW;
    const int T = K >> 7;
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);
    f32x4 acc[MTW][4];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    bool row_ok[MTW];
    const uint8_t *arow[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        const int m = m0 + 16 * mt + j;
        row_ok[mt] = m < M;
        arow[mt] = a + (size_t)(row_ok[mt] ? m : 0) * K + 32 * gq;
    }
    for (int st = s_lo; st < s_hi; ++st) {
        const int kb = (st * 128 + 32 * gq) >> 3;
        u32x4 w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = ok ? *(const u32x4 *)(bq + (size_t)(kb + e) * N + ncol)
                      : (u32x4){0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        i32x8 av[MTW];
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
            av[mt] = row_ok[mt] ? load_a32(arow[mt] + st * 128) : (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x8 bop = fp8_b_operand(w[0][i], w[1][i], w[2][i], w[3][i]);
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt) acc[mt][i] = mfma_fp8(av[mt], bop, acc[mt][i]);
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
                    for (int i = 0; i < 4; ++i) fp8_store<DT>(acc[mt][i][r], m, ncol + i, N, s1, asum, s2, y, acc_out);
                }
            }
        return;
    }
    // Split-K by partial tiles exchanged through agent-scope atomics
    // (device.hpp), fp32, summed in split order.
    uint32_t *const cnt = (uint32_t *)ws + (tn + gridDim.x * tm);
    uint64_t *const part = (uint64_t *)((char *)ws + split_counters_bytes((int64_t)gridDim.x * gridDim.y));
    const size_t slot = (size_t)M * N / 2;  // 64-bit words per split
    auto at = [&](int sp, int m) { return part + sp * slot + ((size_t)m * N + ncol) / 2; };
    if (ok) {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * gq + r;
                if (m < M) part_put(at(split, m), (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]});
            }
    }
    if (!split_tile_last_atomic(cnt, S) || !ok) return;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        auto row = [&](int r) { return m0 + 16 * mt + 4 * gq + r; };
        auto addr = [&](int sp, int r) { return at(sp, row(r)); };
        auto valid = [&](int r) { return row(r) < M; };
        f32x4 v[4];
        part_sum<4, 1>(v, S, addr, valid);
        part_clear_all<4>(S, addr, valid);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!valid(r)) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) fp8_store<DT>(v[r][i], row(r), ncol + i, N, s1, asum, s2, y, acc_out);
        }
    }
}

template <int BLK, int MT, int DT>
static hipError_t launch_fp8_skinny(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st) {
    const size_t lds = (size_t)4 * g.M * 64 * BLK * sizeof(float);
    hipLaunchKernelGGL((w4a8_fp8_skinny<BLK, MT, DT>), dim3(p.tiles_n, p.splits), dim3(256), lds, st, g.a,
                       (const uint32_t *)g.b, g.s1, g.asum, (const uint16_t *)g.s2, (uint16_t *)g.y, g.acc_out, p.acc,
                       (int)g.M, (int)g.N, (int)g.K, p.splits);
    return hipGetLastError();
}

template <int MTW, int DT>
static hipError_t launch_fp8_tiled(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st) {
    hipLaunchKernelGGL((w4a8_fp8_tiled<MTW, DT>), dim3(p.tiles_n, p.tiles_m, p.splits), dim3(256), 0, st, g.a,
                       (const uint32_t *)g.b, g.s1, g.asum, (const uint16_t *)g.s2, (uint16_t *)g.y, g.acc_out, p.acc,
                       (int)g.M, (int)g.N, (int)g.K, p.splits);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_fp8_dt(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st) {
    if (p.kind == 0) {
        switch (p.blk * 10 + p.mt) {
            case 11: return launch_fp8_skinny<1, 1, DT>(g, p, st);
            case 21: return launch_fp8_skinny<2, 1, DT>(g, p, st);
            case 12: return launch_fp8_skinny<1, 2, DT>(g, p, st);
            case 14: return launch_fp8_skinny<1, 4, DT>(g, p, st);
            default: return hipErrorInvalidValue;
        }
    }
    if (p.kind == 2) return launch_w4a8_fp8_lds(g, p, st);
    if (p.splits > 1 && p.acc == nullptr) return hipErrorInvalidValue;
    switch (p.mt) {
        case 2: return launch_fp8_tiled<2, DT>(g, p, st);
        case 4: return launch_fp8_tiled<4, DT>(g, p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_w4a8_fp8(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st) {
    return g.dtype == DT_BF16 ? launch_fp8_dt<DT_BF16>(g, p, st) : launch_fp8_dt<DT_F16>(g, p, st);
}

// The fused single-token form (w4a8_fp8_skinny<..., FUSED>): its dynamic LDS,
// the reduction area and the largest K slice's codes.
size_t w4a8_fp8_fused_lds_bytes(int64_t K, int blk, int splits) {
    const int64_t T = K / 128, per = (T + splits - 1) / splits;
    return (size_t)4 * 64 * blk * sizeof(float) + (size_t)per * 128;
}
bool w4a8_fp8_fuses_quant(int64_t M, int64_t K, const W4A8Plan &p) {
    return M == 1 && p.kind == 0 && p.mt == 1 && w4a8_fp8_fused_lds_bytes(K, p.blk, p.splits) <= 64 * 1024;
}

template <int BLK, int DT>
static hipError_t launch_fp8_fused_t(const W4A8Fp8Args &g, const void *x, float *s1_out, const W4A8Plan &p,
                                     hipStream_t st) {
    const size_t lds = w4a8_fp8_fused_lds_bytes(g.K, BLK, p.splits);
    hipLaunchKernelGGL((w4a8_fp8_skinny<BLK, 1, DT, true>), dim3(p.tiles_n, p.splits), dim3(256), lds, st,
                       (const uint8_t *)nullptr, (const uint32_t *)g.b, (const float *)nullptr,
                       (const float *)nullptr, (const uint16_t *)g.s2, (uint16_t *)g.y, g.acc_out, p.acc, 1,
                       (int)g.N, (int)g.K, p.splits, (const uint16_t *)x, s1_out);
    return hipGetLastError();
}

hipError_t launch_w4a8_fp8_fused(const W4A8Fp8Args &g, const void *x, float *s1_out, const W4A8Plan &p,
                                 hipStream_t st) {
    if (!w4a8_fp8_fuses_quant(g.M, g.K, p) || (p.splits > 1 && p.acc == nullptr)) return hipErrorInvalidValue;
    if (g.dtype == DT_BF16)
        return p.blk == 2 ? launch_fp8_fused_t<2, DT_BF16>(g, x, s1_out, p, st)
                          : launch_fp8_fused_t<1, DT_BF16>(g, x, s1_out, p, st);
    return p.blk == 2 ? launch_fp8_fused_t<2, DT_F16>(g, x, s1_out, p, st)
                      : launch_fp8_fused_t<1, DT_F16>(g, x, s1_out, p, st);
}

}  // namespace awq4
