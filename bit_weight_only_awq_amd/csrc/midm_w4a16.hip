// midm_w4a16.hip -- AWQ W4A16 for mid-size M (16 < M <= 64) on gfx950.
//
// Method as in w4a16.hip (vLLM pull request "Speed up AWQ 2.5x with updated
// kernel": the first-generation AWQ order map; w = (q - z) * s, z = 8 when
// symmetric per the AutoAWQ pull request "Marlin symmetric quantization and
// inference").
//
// At these sizes the LDS-pipelined GEMM walks few tiles through many K stages,
// one workgroup per CU, each stage waiting on copy latency.  This kernel is
// the decode kernel's shape widened to up to four 16-row tiles: a wave owns
// one K chunk (32*CS consecutive k inside one group) of a 128-column tile and
// issues all its loads before using any -- the scales and zero points, its MT
// row tiles of X (from L2: every column tile reads the same rows), then every
// packed word of the chunk -- so the whole layer's weights are in flight at
// once.  The B operands are built as in the decode kernel (fp16: the masked
// nibble pair read as fp16 subnormals, zero point and scale applied once per
// chunk on the fp32 sums with row sums from one MFMA against ones; bf16: the
// exact integer q - z, scaled once per chunk), each feeding MT MFMAs.
// The WV waves of a workgroup (WV consecutive chunks) add their partial tiles
// through LDS in a fixed tree (waves [h, 2h) hand theirs to waves [0, h),
// h = WV/2, WV/4, ..., 1), so the result does not depend on timing; the
// workgroups along K then exchange fp32 partial tiles through agent-scope
// atomic stores and loads (device.hpp: split_tile_last_atomic), and the last
// one of a column tile adds them in split order.  One workgroup covers
// WV*32*CS k, so the partial tiles (S x M x N x 4 bytes) stay about the size
// of the weights rather than a multiple of them.
#include "device.hpp"
#include "launch.hpp"
#include "w4a16_ops.hpp"

namespace awq4 {

template <int MT, int CS, int WV, int DT, bool SYM>
__global__ __launch_bounds__(64 * WV, 1) void w4a16_midm(const uint16_t *__restrict__ x,
                                                        const uint32_t *__restrict__ qw,
                                                        const uint16_t *__restrict__ sc,
                                                        const uint32_t *__restrict__ qz, uint16_t *__restrict__ y,
                                                        uint64_t *__restrict__ ws, int M, int N, int K, int G) {
    constexpr int CK = 32 * CS;
    constexpr int ROWS = 16 * MT, COLS = 128;
    // tree reduction area: WV/2 partial tiles of ROWS x COLS floats
    __shared__ __attribute__((aligned(16))) float red[(WV / 2) * ROWS * COLS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int nw = N >> 3;
    const int tile = blockIdx.x;
    const int wcol = tile * 16 + j;
    const bool col_ok = wcol < nw;
    const int wld = col_ok ? wcol : nw - 1;  // past the last word-column: in-bounds words, sums never stored
    const int chunk = blockIdx.y * WV + wave;
    const bool active = chunk < K / CK;

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (active) {
        const int k0 = chunk * CK;
        const int g = k0 / G;  // the chunk lies inside one group
        const u32x4 s4 = *(const u32x4 *)(sc + (size_t)g * N + 8 * wld);
        const uint32_t zw = SYM ? 0x88888888u : qz[(size_t)g * nw + wld];
        u32x4 a[MT][CS];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = 16 * mt + j;
            const int xr = row < M ? row : 0;  // rows past M read row 0 and are zeroed below
#pragma unroll
            for (int s = 0; s < CS; ++s) a[mt][s] = *(const u32x4 *)(x + (size_t)xr * K + k0 + 32 * s + 8 * gq);
        }
        // keep the issue order: scales, zero points and X first, then the
        // weight stream (the scheduler would otherwise sink the small loads
        // next to their late use)
        __builtin_amdgcn_sched_barrier(0);
        uint32_t w[CS][8];
#pragma unroll
        for (int s = 0; s < CS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t tmp[1];
                load_words<1, true>(qw + (size_t)(k0 + 32 * s + 8 * gq + e) * nw + wld, true, tmp);
                w[s][e] = tmp[0];
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (16 * mt + j >= M) {
#pragma unroll
                for (int s = 0; s < CS; ++s) a[mt][s] = (u32x4){0, 0, 0, 0};
            }

        if (DT == DT_F16) {
            const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
            f32x4 rs[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                rs[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < CS; ++s) rs[mt] = mfma_f16(a[mt][s], ones, rs[mt]);
            }
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                uint32_t px[4], py[4], px8[4], py8[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    px[p] = pair_x(w[s][2 * p], w[s][2 * p + 1]);
                    py[p] = pair_y(w[s][2 * p], w[s][2 * p + 1]);
                    px8[p] = px[p] >> 8;
                    py8[p] = py[p] >> 8;
                }
                static_for<8>([&](auto tc) {
                    constexpr int T = decltype(tc)::value;
                    u32x4 bop;
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const uint32_t src = col_src_y(T) ? (col_shift(T) ? py8[p] : py[p])
                                                          : (col_shift(T) ? px8[p] : px[p]);
                        bop[p] = src & (col_hi(T) ? 0x00F000F0u : 0x000F000Fu);
                    }
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt][T] = mfma_f16(a[mt][s], bop, acc[mt][T]);
                });
            }
            float at[8], bt[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float st = scale_f32<DT>(s4, t);
                const float zt = SYM ? 8.0f : (float)((zw >> (4 * col_nibble(t))) & 0xFu);
                at[t] = st * (col_hi(t) ? 1048576.0f : 16777216.0f);  // s * 2^20 or s * 2^24
                bt[t] = st * zt;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        acc[mt][t][r] = __builtin_fmaf(acc[mt][t][r], at[t], -bt[t] * rs[mt][r]);
        } else {
            ZeroConsts<DT> zc;
            zero_consts<DT, SYM>(zc, zw);
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                uint32_t px[4], py[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    px[p] = pair_x(w[s][2 * p], w[s][2 * p + 1]);
                    py[p] = pair_y(w[s][2 * p], w[s][2 * p + 1]);
                }
                static_for<8>([&](auto tc) {
                    constexpr int T = decltype(tc)::value;
                    u32x4 bop;
#pragma unroll
                    for (int p = 0; p < 4; ++p) bop[p] = qz_pair<DT, T>(col_src_y(T) ? py[p] : px[p], zc);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) acc[mt][T] = mma<DT>(a[mt][s], bop, acc[mt][T]);
                });
            }
            float st[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) st[t] = scale_f32<DT>(s4, t);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < 8; ++t) acc[mt][t][r] *= st[t];
        }
    }

    // Lane holds rows 16 mt + 4 gq + r and columns 8 j + t of the tile.
    auto slot_of = [&](int sl, int mt, int r) {
        return red + ((size_t)sl * ROWS + 16 * mt + 4 * gq + r) * COLS + 8 * j;
    };
#pragma unroll
    for (int h = WV / 2; h >= 1; h >>= 1) {
        if (wave >= h && wave < 2 * h) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float *d = slot_of(wave - h, mt, r);
                    *(f32x4 *)d = (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                    *(f32x4 *)(d + 4) = (f32x4){acc[mt][4][r], acc[mt][5][r], acc[mt][6][r], acc[mt][7][r]};
                }
        }
        __syncthreads();
        if (wave < h) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float *d = slot_of(wave, mt, r);
                    const f32x4 v0 = *(const f32x4 *)d, v1 = *(const f32x4 *)(d + 4);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        acc[mt][t][r] += v0[t];
                        acc[mt][4 + t][r] += v1[t];
                    }
                }
        }
        __syncthreads();
    }
    // wave 0 holds the workgroup's sum: park it for all threads
    if (wave == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *d = slot_of(0, mt, r);
                *(f32x4 *)d = (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                *(f32x4 *)(d + 4) = (f32x4){acc[mt][4][r], acc[mt][5][r], acc[mt][6][r], acc[mt][7][r]};
            }
    }
    __syncthreads();

    const int S = gridDim.y;
    const int total = M * COLS, n_base = tile * COLS;
    if (S == 1) {
        for (int idx = threadIdx.x; idx < total; idx += 64 * WV) {
            const int m = idx / COLS, c = idx - m * COLS, n = n_base + c;
            if (n < N) y[(size_t)m * N + n] = f32_to_out_bits(red[idx], DT);
        }
        return;
    }
    float *const part = (float *)((char *)ws + split_counters_bytes(gridDim.x));
    const size_t slot = (size_t)M * N;
    for (int idx = threadIdx.x; idx < total; idx += 64 * WV) {
        const int m = idx / COLS, c = idx - m * COLS, n = n_base + c;
        if (n < N)
            __hip_atomic_store(&part[blockIdx.y * slot + (size_t)m * N + n], red[idx], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!split_tile_last_atomic((uint32_t *)ws + tile, S)) return;
    // the last workgroup of the column tile: partials summed in split order
    // (loads of a batch of splits issued together), then cleared
    constexpr int kBatch = 8;
    for (int idx = threadIdx.x; idx < total; idx += 64 * WV) {
        const int m = idx / COLS, c = idx - m * COLS, n = n_base + c;
        if (n >= N) continue;
        float *p = part + (size_t)m * N + n;
        float v = 0.f;
        for (int s0 = 0; s0 < S; s0 += kBatch) {
            float b[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                b[i] = s0 + i < S ? __hip_atomic_load(&p[(size_t)(s0 + i) * slot], __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : 0.f;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) v += b[i];
        }
        for (int s = 0; s < S; ++s)
            __hip_atomic_store(&p[(size_t)s * slot], 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        y[(size_t)m * N + n] = f32_to_out_bits(v, DT);
    }
}

template <int MT, int CS, int DT, bool SYM>
static hipError_t launch_midm_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    constexpr int WV = 8;
    if (p.splits > 1 && p.acc == nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((w4a16_midm<MT, CS, WV, DT, SYM>), dim3(p.tiles_n, p.splits), dim3(64 * WV), 0, st,
                       (const uint16_t *)a.x, (const uint32_t *)a.qweight, (const uint16_t *)a.scales,
                       (const uint32_t *)a.qzeros, (uint16_t *)a.y, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G);
    return hipGetLastError();
}

template <int MT, int CS>
static hipError_t launch_midm_dt(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16)
        return sym ? launch_midm_t<MT, CS, DT_F16, true>(a, p, st) : launch_midm_t<MT, CS, DT_F16, false>(a, p, st);
    return sym ? launch_midm_t<MT, CS, DT_BF16, true>(a, p, st) : launch_midm_t<MT, CS, DT_BF16, false>(a, p, st);
}

// p.mt: 16-row tiles (2: M <= 32, 4: M <= 64); p.cs: 32-k steps per wave chunk (1 or 2)
hipError_t launch_w4a16_midm(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    switch (p.mt * 10 + p.cs) {
        case 21: return launch_midm_dt<2, 1>(a, p, st);
        case 22: return launch_midm_dt<2, 2>(a, p, st);
        case 41: return launch_midm_dt<4, 1>(a, p, st);
        case 42: return launch_midm_dt<4, 2>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace awq4
