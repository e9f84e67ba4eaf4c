// w4a16.hip -- AWQ W4A16 kernels for gfx950: Y = X . dequant(qweight, qzeros, scales).
//
// Method (vLLM pull request "Speed up AWQ 2.5x with updated kernel": the
// GEMM/GEMV dispatch snippet and the list of packing differences; AutoAWQ pull
// request "Marlin symmetric quantization and inference": the symmetric form
// without zero points): w[k,n] = (q[k,n] - z[k/G,n]) * s[k/G,n], with q, z
// nibbles of the first-generation AWQ order map and z = 8 when qzeros is
// absent.
//
// Design (both kernels): no transpose through LDS.  A lane loads the packed
// words of ONE word-column (8 output columns) at 8 consecutive k, pairs
// consecutive-k words byte-wise with v_perm so that every 16-bit half holds
// one k, and extracts column t from the pairs with one mask, giving the
// matrix-core B operand of 8 consecutive k of that column directly.  Column t
// of the word of lane j becomes B column j of the t-th MFMA, so one set of 8
// MFMAs covers the 16 word-columns of a wave (128 output columns) and
// output column = 8 * word_column(j) + t.  Dequantisation stays exact up to
// one rounding (see device.hpp).
//
//  * skinny kernel (decode, M <= 32): a workgroup of 4 waves owns 128*BLK
//    output columns; its waves split a K slice, are reduced through LDS in a
//    fixed order, and workgroups along K (split-K) are combined by the last
//    one to arrive.  Weight loads are 4*BLK bytes per lane per k-row, fully
//    coalesced per wave.
//  * tiled kernel (prefill): a workgroup of 4 waves (2 x 2) owns a
//    (2*16*MTW) x 256 output tile; each wave runs the full K of its slice with
//    MTW row tiles x 8 column MFMAs per 32-k step; optional split-K over the
//    grid's z dimension.
#include "device.hpp"
#include "launch.hpp"

namespace awq4 {

// Per-group dequant constants of one word-column for the 8 columns t.
template <int DT, bool SYM>
struct GroupConsts {
    uint32_t zc[8];  // fp16: packed zero constant
    uint32_t sc[8];  // fp16: packed scale
    float sf[8];     // bf16: effective scale (s or s/16)
    float zs[8];     // bf16: z*s
};

template <int DT, bool SYM>
__device__ __forceinline__ void load_group(GroupConsts<DT, SYM> &c, const uint16_t *__restrict__ sc,
                                           const uint32_t *__restrict__ qz, int N, int nw, int g, int wcol,
                                           bool valid) {
    u32x4 s4 = {0, 0, 0, 0};
    uint32_t zw = 0x88888888u;
    if (valid) {
        s4 = *(const u32x4 *)(sc + (size_t)g * N + 8 * wcol);
        if (!SYM) zw = qz[(size_t)g * nw + wcol];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t sb = (s4[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;  // scale of column 8*wcol + t
        uint32_t z = (zw >> (4 * col_nibble(t))) & 0xFu;
        if (DT == DT_F16) {
            c.zc[t] = col_hi(t) ? zconst_f16<1>(z) : zconst_f16<0>(z);
            c.sc[t] = sb | (sb << 16);
        } else {
            float s = bf16_bits_to_f32(sb);
            c.sf[t] = col_hi(t) ? s * 0.0625f : s;
            c.zs[t] = (float)z * s;
        }
    }
}

// B operand (8 consecutive k of column t) from the pair registers px/py.
template <int DT, bool SYM, int t>
__device__ __forceinline__ u32x4 make_b(const uint32_t (&px)[4], const uint32_t (&py)[4],
                                        const GroupConsts<DT, SYM> &c) {
    u32x4 b;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t src = col_src_y(t) ? py[p] : px[p];
        uint32_t v = col_shift(t) ? (src >> 8) : src;
        if (DT == DT_F16) {
            b[p] = col_hi(t) ? dq_f16<1>(v, c.zc[t], c.sc[t]) : dq_f16<0>(v, c.zc[t], c.sc[t]);
        } else {
            b[p] = dq_bf16(v, col_hi(t) ? 0x00F000F0u : 0x000F000Fu, c.sf[t], c.zs[t]);
        }
    }
    return b;
}

template <int DT>
__device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    if (DT == DT_F16) return mfma_f16(a, b, c);
    return mfma_bf16(a, b, c);
}

// Load BLK consecutive packed words of one k-row (zero words out of range).
// The skinny kernel streams each word exactly once (non-temporal hint); the
// tiled kernel re-reads words from other row tiles and keeps them cacheable.
template <int BLK, bool NT = true>
__device__ __forceinline__ void load_words(const uint32_t *__restrict__ p, bool valid, uint32_t (&w)[BLK]) {
    if (!valid) {
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = 0;
        return;
    }
    if (!NT) {
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = p[b];
        return;
    }
    if (BLK == 4) {
        u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = v[b];
    } else if (BLK == 2) {
        u32x2 v = __builtin_nontemporal_load((const u32x2 *)p);
#pragma unroll
        for (int b = 0; b < BLK; ++b) w[b] = v[b];
    } else {
        w[0] = __builtin_nontemporal_load(p);
    }
}

// ===========================================================================
// Skinny kernel: M <= 16*MT, grid (col tiles, splits), 256 threads.
// Dynamic LDS: 3 * M * (128*BLK) floats.
template <int BLK, int MT, int DT, bool SYM>
__global__ __launch_bounds__(256) void w4a16_skinny(const uint16_t *__restrict__ x, const uint32_t *__restrict__ qw,
                                                    const uint16_t *__restrict__ sc,
                                                    const uint32_t *__restrict__ qz, uint16_t *__restrict__ y,
                                                    float *__restrict__ part, int *__restrict__ counters, int M,
                                                    int N, int K, int G, int S) {
    extern __shared__ float red[];
    constexpr int COLS = 128 * BLK;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int nw = N >> 3;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int wcol0 = tile * 16 * BLK + j * BLK;  // lane's first word-column
    const bool col_ok = wcol0 < nw;
    const int T = K >> 5;
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);
    const int w_lo = s_lo + (s_hi - s_lo) * wave / 4, w_hi = s_lo + (s_hi - s_lo) * (wave + 1) / 4;

    f32x4 acc[MT][BLK][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int b = 0; b < BLK; ++b)
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[mt][b][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    GroupConsts<DT, SYM> gc[BLK];
    int gcur = -1;
    for (int st = w_lo; st < w_hi; ++st) {
        const int k0 = st * 32;
        uint32_t w[8][BLK];
#pragma unroll
        for (int e = 0; e < 8; ++e) load_words<BLK>(qw + (size_t)(k0 + 8 * gq + e) * nw + wcol0, col_ok, w[e]);
        u32x4 a[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + j;
            a[mt] = (m < M) ? *(const u32x4 *)(x + (size_t)m * K + k0 + 8 * gq) : (u32x4){0, 0, 0, 0};
        }
        const int g = k0 / G;
        if (g != gcur) {
            gcur = g;
#pragma unroll
            for (int b = 0; b < BLK; ++b) load_group<DT, SYM>(gc[b], sc, qz, N, nw, g, wcol0 + b, col_ok);
        }
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            uint32_t px[4], py[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                px[p] = pair_x(w[2 * p][b], w[2 * p + 1][b]);
                py[p] = pair_y(w[2 * p][b], w[2 * p + 1][b]);
            }
#define AWQ4_COL(T_)                                                                  \
    {                                                                                 \
        u32x4 bop = make_b<DT, SYM, T_>(px, py, gc[b]);                               \
        _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) acc[mt][b][T_] =            \
            mma<DT>(a[mt], bop, acc[mt][b][T_]);                                      \
    }
            AWQ4_COL(0) AWQ4_COL(1) AWQ4_COL(2) AWQ4_COL(3) AWQ4_COL(4) AWQ4_COL(5) AWQ4_COL(6) AWQ4_COL(7)
#undef AWQ4_COL
        }
    }

    // Reduce the 4 waves: waves 1..3 park their partials in LDS
    // (red[wave-1][m][c], c = local column); wave 0 adds them, in wave order,
    // to its own registers and writes 8 consecutive columns per store.
    if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mt * 16 + 4 * gq + r;
                if (m < M) {
#pragma unroll
                    for (int b = 0; b < BLK; ++b) {
                        float *dst = red + ((size_t)(wave - 1) * M + m) * COLS + 8 * (j * BLK + b);
                        *(f32x4 *)dst = (f32x4){acc[mt][b][0][r], acc[mt][b][1][r], acc[mt][b][2][r], acc[mt][b][3][r]};
                        *(f32x4 *)(dst + 4) = (f32x4){acc[mt][b][4][r], acc[mt][b][5][r], acc[mt][b][6][r], acc[mt][b][7][r]};
                    }
                }
            }
    }
    __syncthreads();
    if (wave == 0 && col_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mt * 16 + 4 * gq + r;
                if (m >= M) continue;
#pragma unroll
                for (int b = 0; b < BLK; ++b) {
                    f32x4 v0 = {acc[mt][b][0][r], acc[mt][b][1][r], acc[mt][b][2][r], acc[mt][b][3][r]};
                    f32x4 v1 = {acc[mt][b][4][r], acc[mt][b][5][r], acc[mt][b][6][r], acc[mt][b][7][r]};
#pragma unroll
                    for (int w = 0; w < 3; ++w) {
                        const float *src = red + ((size_t)w * M + m) * COLS + 8 * (j * BLK + b);
                        v0 += *(const f32x4 *)src;
                        v1 += *(const f32x4 *)(src + 4);
                    }
                    const int n0 = 8 * (wcol0 + b);
                    if (S == 1) {
                        u32x4 o;
                        o[0] = (uint32_t)f32_to_out_bits(v0[0], DT) | ((uint32_t)f32_to_out_bits(v0[1], DT) << 16);
                        o[1] = (uint32_t)f32_to_out_bits(v0[2], DT) | ((uint32_t)f32_to_out_bits(v0[3], DT) << 16);
                        o[2] = (uint32_t)f32_to_out_bits(v1[0], DT) | ((uint32_t)f32_to_out_bits(v1[1], DT) << 16);
                        o[3] = (uint32_t)f32_to_out_bits(v1[2], DT) | ((uint32_t)f32_to_out_bits(v1[3], DT) << 16);
                        *(u32x4 *)(y + (size_t)m * N + n0) = o;
                    } else {
                        float *dst = part + ((size_t)split * M + m) * N + n0;
                        *(f32x4 *)dst = v0;
                        *(f32x4 *)(dst + 4) = v1;
                    }
                }
            }
    }
    if (S == 1) return;
    if (!splitk_arrive(&counters[tile], S)) return;
    // Last workgroup of this column tile: sum the S partials in split order.
    const int n_base = tile * COLS;
    const int total = M * COLS;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int m = idx / COLS, c = idx - m * COLS;
        const int n = n_base + c;
        if (n >= N) continue;
        float v = 0.f;
        for (int s = 0; s < S; ++s) v += __builtin_nontemporal_load(&part[((size_t)s * M + m) * N + n]);
        y[(size_t)m * N + n] = f32_to_out_bits(v, DT);
    }
}

// ===========================================================================
// Tiled kernel: grid (ceil(N/256), ceil(M/BM), S), 256 threads = 2 x 2 waves,
// wave tile (16*MTW) x 128, BM = 32*MTW.
template <int MTW, int DT, bool SYM>
__global__ __launch_bounds__(256) void w4a16_tiled(const uint16_t *__restrict__ x, const uint32_t *__restrict__ qw,
                                                   const uint16_t *__restrict__ sc, const uint32_t *__restrict__ qz,
                                                   uint16_t *__restrict__ y, float *__restrict__ part,
                                                   int *__restrict__ counters, int M, int N, int K, int G, int S) {
    constexpr int BM = 32 * MTW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int nw = N >> 3;
    const int tn = blockIdx.x, tm = blockIdx.y, split = blockIdx.z;
    const int wcol = tn * 32 + wn * 16 + j;  // this lane's word-column
    const bool col_ok = wcol < nw;
    const int m0 = tm * BM + wm * 16 * MTW;
    const int T = K >> 5;
    const int s_lo = (int)((int64_t)T * split / S), s_hi = (int)((int64_t)T * (split + 1) / S);

    f32x4 acc[MTW][8];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const uint16_t *xrow[MTW];
    bool row_ok[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        const int m = m0 + 16 * mt + j;
        row_ok[mt] = m < M;
        xrow[mt] = x + (size_t)(row_ok[mt] ? m : 0) * K + 8 * gq;
    }

    GroupConsts<DT, SYM> gc;
    int gcur = -1;
    for (int st = s_lo; st < s_hi; ++st) {
        const int k0 = st * 32;
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t tmp[1];
            load_words<1, false>(qw + (size_t)(k0 + 8 * gq + e) * nw + wcol, col_ok, tmp);
            w[e] = tmp[0];
        }
        u32x4 a[MTW];
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
            a[mt] = row_ok[mt] ? *(const u32x4 *)(xrow[mt] + k0) : (u32x4){0, 0, 0, 0};
        const int g = k0 / G;
        if (g != gcur) {
            gcur = g;
            load_group<DT, SYM>(gc, sc, qz, N, nw, g, wcol, col_ok);
        }
        uint32_t px[4], py[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            px[p] = pair_x(w[2 * p], w[2 * p + 1]);
            py[p] = pair_y(w[2 * p], w[2 * p + 1]);
        }
#define AWQ4_COL(T_)                                                                                  \
    {                                                                                                 \
        u32x4 bop = make_b<DT, SYM, T_>(px, py, gc);                                                  \
        _Pragma("unroll") for (int mt = 0; mt < MTW; ++mt) acc[mt][T_] = mma<DT>(a[mt], bop, acc[mt][T_]); \
    }
        AWQ4_COL(0) AWQ4_COL(1) AWQ4_COL(2) AWQ4_COL(3) AWQ4_COL(4) AWQ4_COL(5) AWQ4_COL(6) AWQ4_COL(7)
#undef AWQ4_COL
    }

    // Epilogue: lane holds rows m0 + 16mt + 4gq + r, columns 8*wcol + t.
    const int n0 = 8 * wcol;
    if (S == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * gq + r;
                if (m < M) {
                    u32x4 o;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        o[p] = (uint32_t)f32_to_out_bits(acc[mt][2 * p][r], DT) |
                               ((uint32_t)f32_to_out_bits(acc[mt][2 * p + 1][r], DT) << 16);
                    *(u32x4 *)(y + (size_t)m * N + n0) = o;
                }
            }
        return;
    }
    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * gq + r;
                if (m < M) {
                    float *dst = part + ((size_t)split * M + m) * N + n0;
                    *(f32x4 *)dst = (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                    *(f32x4 *)(dst + 4) = (f32x4){acc[mt][4][r], acc[mt][5][r], acc[mt][6][r], acc[mt][7][r]};
                }
            }
    }
    if (!splitk_arrive(&counters[tm * gridDim.x + tn], S)) return;
    if (!col_ok) return;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 16 * mt + 4 * gq + r;
            if (m >= M) continue;
            f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < S; ++s) {
                const float *src = part + ((size_t)s * M + m) * N + n0;
                v0 += __builtin_nontemporal_load((const f32x4 *)src);
                v1 += __builtin_nontemporal_load((const f32x4 *)(src + 4));
            }
            u32x4 o;
            o[0] = (uint32_t)f32_to_out_bits(v0[0], DT) | ((uint32_t)f32_to_out_bits(v0[1], DT) << 16);
            o[1] = (uint32_t)f32_to_out_bits(v0[2], DT) | ((uint32_t)f32_to_out_bits(v0[3], DT) << 16);
            o[2] = (uint32_t)f32_to_out_bits(v1[0], DT) | ((uint32_t)f32_to_out_bits(v1[1], DT) << 16);
            o[3] = (uint32_t)f32_to_out_bits(v1[2], DT) | ((uint32_t)f32_to_out_bits(v1[3], DT) << 16);
            *(u32x4 *)(y + (size_t)m * N + n0) = o;
        }
}

// ===========================================================================
// Host launchers.

template <int BLK, int MT, int DT, bool SYM>
static hipError_t launch_skinny_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    dim3 grid(p.tiles_n, p.splits);
    size_t lds = (size_t)3 * a.M * 128 * BLK * sizeof(float);
    hipLaunchKernelGGL((w4a16_skinny<BLK, MT, DT, SYM>), grid, dim3(256), lds, st, (const uint16_t *)a.x,
                       (const uint32_t *)a.qweight, (const uint16_t *)a.scales, (const uint32_t *)a.qzeros,
                       (uint16_t *)a.y, p.partials, p.counters, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits);
    return hipGetLastError();
}

template <int BLK, int MT>
static hipError_t launch_skinny_dt(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16) return sym ? launch_skinny_t<BLK, MT, DT_F16, true>(a, p, st)
                                      : launch_skinny_t<BLK, MT, DT_F16, false>(a, p, st);
    return sym ? launch_skinny_t<BLK, MT, DT_BF16, true>(a, p, st) : launch_skinny_t<BLK, MT, DT_BF16, false>(a, p, st);
}

hipError_t launch_w4a16_skinny(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    switch (p.blk * 10 + p.mt) {
        case 11: return launch_skinny_dt<1, 1>(a, p, st);
        case 21: return launch_skinny_dt<2, 1>(a, p, st);
        case 41: return launch_skinny_dt<4, 1>(a, p, st);
        case 12: return launch_skinny_dt<1, 2>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

template <int MTW, int DT, bool SYM>
static hipError_t launch_tiled_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    dim3 grid(p.tiles_n, p.tiles_m, p.splits);
    hipLaunchKernelGGL((w4a16_tiled<MTW, DT, SYM>), grid, dim3(256), 0, st, (const uint16_t *)a.x,
                       (const uint32_t *)a.qweight, (const uint16_t *)a.scales, (const uint32_t *)a.qzeros,
                       (uint16_t *)a.y, p.partials, p.counters, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits);
    return hipGetLastError();
}

template <int MTW>
static hipError_t launch_tiled_dt(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16) return sym ? launch_tiled_t<MTW, DT_F16, true>(a, p, st)
                                      : launch_tiled_t<MTW, DT_F16, false>(a, p, st);
    return sym ? launch_tiled_t<MTW, DT_BF16, true>(a, p, st) : launch_tiled_t<MTW, DT_BF16, false>(a, p, st);
}

hipError_t launch_w4a16_tiled(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    switch (p.mt) {
        case 1: return launch_tiled_dt<1>(a, p, st);
        case 2: return launch_tiled_dt<2>(a, p, st);
        case 4: return launch_tiled_dt<4>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace awq4
