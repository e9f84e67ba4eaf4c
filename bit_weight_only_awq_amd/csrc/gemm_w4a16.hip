// gemm_w4a16.hip -- prefill GEMM for AWQ W4A16 on gfx950 (large M).
//
// Same method as w4a16.hip (vLLM pull request "Speed up AWQ 2.5x with updated
// kernel": first-generation AWQ packing and the context-phase GEMM; AutoAWQ
// pull request "Marlin symmetric quantization and inference": z = 8 when no
// zero points): Y = X . W with W[k,n] = (q - z) * s rounded once to the
// activation type, fp32 accumulation on the matrix cores.
//
// Workgroup tile 128 (M) x 256 (N), K in stages of 64; 4 waves in a 2 x 2
// grid, each owning 64 x 128 outputs (4 row tiles x 8 column MFMAs of
// 16x16x32).  Per stage, X (fp16/bf16) and the packed weight words are staged
// through LDS with double buffering: the global loads of stage s+1 (and the
// scales / zero points it needs) are issued before stage s is computed, and
// written to the other LDS buffer afterwards, so one barrier per stage
// suffices.  Each wave dequantises its own B operands from the packed words in
// LDS (lane j: one word-column, 8 consecutive k; see device.hpp), which keeps
// the LDS traffic for B at 4 bits per weight.
#include "device.hpp"
#include "launch.hpp"
#include "w4a16_ops.hpp"

namespace awq4 {

constexpr int GB_M = 128, GB_N = 256, GB_K = 64;
constexpr int GA_PITCH = GB_K * 2 + 16;          // bytes per X row in LDS (16 B pad: conflict-free row reads)
constexpr int GA_BYTES = GB_M * GA_PITCH;        // 18432
constexpr int GB_PITCH = (GB_N / 8) * 4;         // bytes per k-row of packed words (32 words)
constexpr int GB_BYTES = GB_K * GB_PITCH;        // 8192
constexpr int G_STAGE = GA_BYTES + GB_BYTES;     // 26624; two stages = 53248 bytes of LDS

// Packed-word LDS swizzle: 16-byte segment s of k-row r is stored at segment
// s ^ 4*((r >> 3) & 1), so lane groups reading rows 8 apart use both halves
// of the banks.
__device__ __forceinline__ int gseg(int r, int s) { return s ^ (((r >> 3) & 1) << 2); }

template <int DT, bool SYM>
__global__ __launch_bounds__(256, 2) void w4a16_gemm(const uint16_t *__restrict__ x, const uint32_t *__restrict__ qw,
                                                     const uint16_t *__restrict__ sc,
                                                     const uint32_t *__restrict__ qz, uint16_t *__restrict__ y,
                                                     uint64_t *__restrict__ acc64, int M, int N, int K, int G,
                                                     int S) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * G_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int nw = N >> 3;
    const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
    const int m0 = tm * GB_M, wc0 = tn * (GB_N / 8);
    const int T = K / GB_K;
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);

    // global -> register prefetch assignment: 8 threads per 128-byte row
    const int ld_row = tid >> 3, ld_seg = tid & 7;
    // the word-column this lane dequantises and owns in the output
    const int wcol = wc0 + wn * 16 + j;
    const bool col_ok = wcol < nw;

    u32x4 pa[4], pb[2], ps4[2];
    uint32_t pzw[2];
    auto gload = [&](int st) {
        const int k0 = st * GB_K;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + ld_row + 32 * i;
            pa[i] = m < M ? *(const u32x4 *)(x + (size_t)m * K + k0 + ld_seg * 8) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int wc = wc0 + ld_seg * 4;  // nw % 4 == 0: all four words valid or none
            pb[i] = wc < nw ? *(const u32x4 *)(qw + (size_t)(k0 + ld_row + 32 * i) * nw + wc) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int g = (k0 + 32 * ks) / G;
            ps4[ks] = col_ok ? *(const u32x4 *)(sc + (size_t)g * N + 8 * wcol) : (u32x4){0, 0, 0, 0};
            pzw[ks] = (!SYM && col_ok) ? qz[(size_t)g * nw + wcol] : 0x88888888u;
        }
    };
    auto swrite = [&](int buf) {
        unsigned char *A = lds + buf * G_STAGE;
        unsigned char *B = A + GA_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)(A + (ld_row + 32 * i) * GA_PITCH + ld_seg * 16) = pa[i];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = ld_row + 32 * i;
            *(u32x4 *)(B + r * GB_PITCH + gseg(r, ld_seg) * 16) = pb[i];
        }
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    ZeroConsts<DT> zc;
    uint32_t sc2[8];
    float sf[8];
    int gcur = -1;
    u32x4 cs4[2];
    uint32_t czw[2];

    if (s_lo < s_hi) {
        gload(s_lo);
        swrite(0);
        cs4[0] = ps4[0];
        cs4[1] = ps4[1];
        czw[0] = pzw[0];
        czw[1] = pzw[1];
    }
    __syncthreads();
    for (int st = s_lo; st < s_hi; ++st) {
        const int buf = (st - s_lo) & 1;
        const bool more = st + 1 < s_hi;
        if (more) gload(st + 1);
        const unsigned char *A = lds + buf * G_STAGE;
        const unsigned char *B = A + GA_BYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int g = (st * GB_K + 32 * ks) / G;
            if (g != gcur) {
                gcur = g;
                zero_consts<DT, SYM>(zc, czw[ks]);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint32_t b = scale_bits<DT>(cs4[ks], t);
                    sc2[t] = b | (b << 16);
                    sf[t] = scale_f32<DT>(cs4[ks], t);
                }
            }
            u32x4 a[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                a[mt] = *(const u32x4 *)(A + (wm * 64 + 16 * mt + j) * GA_PITCH + (32 * ks + 8 * gq) * 2);
            uint32_t w[8];
            const int c = wn * 16 + j;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 32 * ks + 8 * gq + e;
                w[e] = *(const uint32_t *)(B + r * GB_PITCH + gseg(r, c >> 2) * 16 + (c & 3) * 4);
            }
            uint32_t px[4], py[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                px[p] = pair_x(w[2 * p], w[2 * p + 1]);
                py[p] = pair_y(w[2 * p], w[2 * p + 1]);
            }
#define AWQ4_COL(T_)                                                                                  \
    {                                                                                                 \
        u32x4 bop;                                                                                    \
        _Pragma("unroll") for (int p = 0; p < 4; ++p) bop[p] =                                        \
            w_pair<DT, T_>(col_src_y(T_) ? py[p] : px[p], zc, sc2[T_], sf[T_]);                       \
        _Pragma("unroll") for (int mt = 0; mt < 4; ++mt) acc[mt][T_] = mma<DT>(a[mt], bop, acc[mt][T_]); \
    }
            AWQ4_COL(0) AWQ4_COL(1) AWQ4_COL(2) AWQ4_COL(3) AWQ4_COL(4) AWQ4_COL(5) AWQ4_COL(6) AWQ4_COL(7)
#undef AWQ4_COL
        }
        if (more) {
            swrite(buf ^ 1);
            cs4[0] = ps4[0];
            cs4[1] = ps4[1];
            czw[0] = pzw[0];
            czw[1] = pzw[1];
        }
        __syncthreads();
    }

    // Epilogue: lane holds rows m0 + 64wm + 16mt + 4gq + r, columns 8*wcol + t.
    if (!col_ok) return;
    const int n0 = 8 * wcol;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * 64 + 16 * mt + 4 * gq + r;
            if (m >= M) continue;
            if (S == 1) {
                f32x4 v0 = {acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                f32x4 v1 = {acc[mt][4][r], acc[mt][5][r], acc[mt][6][r], acc[mt][7][r]};
                *(u32x4 *)(y + (size_t)m * N + n0) = pack8_out<DT>(v0, v1);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    int64_t sum;
                    if (splitk_contribute(&acc64[(size_t)m * N + n0 + t], to_fixed<DT>(acc[mt][t][r]), S, &sum))
                        y[(size_t)m * N + n0 + t] = f32_to_out_bits(from_fixed<DT>(sum), DT);
                }
            }
        }
}

template <int DT, bool SYM>
static hipError_t launch_gemm_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    dim3 grid(p.tiles_n, p.tiles_m, p.splits);
    hipLaunchKernelGGL((w4a16_gemm<DT, SYM>), grid, dim3(256), 0, st, (const uint16_t *)a.x,
                       (const uint32_t *)a.qweight, (const uint16_t *)a.scales, (const uint32_t *)a.qzeros,
                       (uint16_t *)a.y, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits);
    return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16) return sym ? launch_gemm_t<DT_F16, true>(a, p, st) : launch_gemm_t<DT_F16, false>(a, p, st);
    return sym ? launch_gemm_t<DT_BF16, true>(a, p, st) : launch_gemm_t<DT_BF16, false>(a, p, st);
}

}  // namespace awq4
