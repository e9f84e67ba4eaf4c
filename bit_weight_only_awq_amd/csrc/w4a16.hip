// w4a16.hip -- AWQ W4A16 kernels for gfx950: Y = X . dequant(qweight, qzeros, scales).
//
// Method (vLLM pull request "Speed up AWQ 2.5x with updated kernel": the
// GEMM/GEMV dispatch snippet and the list of packing differences; AutoAWQ pull
// request "Marlin symmetric quantization and inference": the symmetric form
// without zero points): w[k,n] = (q[k,n] - z[k/G,n]) * s[k/G,n], with q, z
// nibbles of the first-generation AWQ order map and z = 8 when qzeros is
// absent.
//
// Operand construction (both kernels): no transpose through LDS.  A lane
// loads the packed words of ONE word-column (8 output columns) at 8
// consecutive k, pairs consecutive-k words byte-wise with v_perm so that every
// 16-bit half holds one k, and extracts column t from the pairs with one mask:
// that is the matrix-core B operand of 8 consecutive k of column t.  Column t
// of the word of lane j becomes B column j of the t-th MFMA, so one set of 8
// MFMAs covers the 16 word-columns of a wave (128 output columns), and output
// column = 8 * word_column(j) + t.
//
//  * decode kernel (M <= 16): a wave owns one K chunk (32*CS values inside one
//    quantisation group) of a 128*BLK column tile and issues every weight load
//    of the chunk before using any, so the whole weight stream is in flight
//    across the GPU.  fp16: the B operand is the masked nibble pair read as
//    fp16 subnormals (exact on the matrix cores, one AND per pair); zero point
//    and scale are applied once per chunk on the fp32 sums.  bf16: the B
//    operand is the exact integer 128 + q (the nibble ORed into the mantissa
//    of 128.0), zero point and scale applied once per chunk in the same
//    way.  The 4 waves of a
//    workgroup (4 consecutive chunks) are reduced through LDS, workgroups
//    along K through counting fixed-point atomics (fp16) or per-tile fp32
//    partials (bf16; device.hpp).
//  * tiled kernel (prefill): a workgroup of 4 waves (2 x 2) owns a
//    (2*16*MTW) x 256 output tile; each wave runs the full K of its slice with
//    MTW row tiles x 8 column MFMAs per 32-k step, B = (q - z) * s rounded
//    once to the activation type; optional split-K over the grid's z.
#include "device.hpp"
#include "launch.hpp"
#include "w4a16_ops.hpp"

namespace awq4 {

// Workgroup epilogue of the decode kernels: every wave parks its M x COLS
// partial in LDS (red[wave][m][c]); after one barrier each thread adds the
// WAVES partials of its elements in wave order (a fixed order, so the result
// is deterministic) and either writes the output (no split) or hands the sum
// to the split-K reduction (device.hpp):
//  - fp16 outputs: one counting fixed-point accumulator per element (steps of
//    2^-28, a sixteenth of the finest fp16 spacing, with range 2^19 beyond the
//    largest fp16; one device-scope round trip per workgroup);
//  - bf16 outputs: per-tile fp32 partials summed in split order by the last
//    workgroup of the tile, exchanged through agent-scope atomic stores and
//    loads (no L2 write-back per workgroup; device.hpp).  bf16 keeps binary32's exponent range, so no
//    fixed-point step suits every output: a step fine enough for |y| ~ 1e-3
//    leaves no range for large outputs, and a coarse one loses small outputs.
template <int BLK, int DT, int WAVES = 4>
__device__ __forceinline__ void decode_epilogue(f32x4 (&acc)[BLK][8], float *red, uint16_t *__restrict__ y,
                                                uint64_t *__restrict__ acc64, int M, int N, int wave, int gq,
                                                int j, int tile) {
    constexpr int COLS = 128 * BLK;
    const int total = M * COLS;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * gq + r;
        if (m < M) {
#pragma unroll
            for (int b = 0; b < BLK; ++b) {
                float *dst = red + (size_t)wave * total + (size_t)m * COLS + 8 * (j * BLK + b);
                *(f32x4 *)dst = (f32x4){acc[b][0][r], acc[b][1][r], acc[b][2][r], acc[b][3][r]};
                *(f32x4 *)(dst + 4) = (f32x4){acc[b][4][r], acc[b][5][r], acc[b][6][r], acc[b][7][r]};
            }
        }
    }
    __syncthreads();
    const int n_base = tile * COLS;
    const int S = gridDim.y;
    // bf16 split-K: workspace = tile counters, then fp32 partials [S][M][N]
    float *const part = (float *)((char *)acc64 + split_counters_bytes(gridDim.x));
    const size_t slot = (size_t)M * N;
    for (int idx = threadIdx.x; idx < total; idx += 64 * WAVES) {
        const int m = idx / COLS, c = idx - m * COLS;
        const int n = n_base + c;
        if (n >= N) continue;
        float v = red[idx];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += red[(size_t)w * total + idx];
        if (S == 1) {
            y[(size_t)m * N + n] = f32_to_out_bits(v, DT);
        } else if (DT == DT_F16) {
            int64_t sum;
            if (splitk_contribute(&acc64[(size_t)m * N + n], to_fixed<DT>(v), S, &sum))
                y[(size_t)m * N + n] = f32_to_out_bits(from_fixed<DT>(sum), DT);
        } else {
            __hip_atomic_store(&part[blockIdx.y * slot + (size_t)m * N + n], v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (DT == DT_F16 || S == 1) return;
    if (!split_tile_last_atomic((uint32_t *)acc64 + tile, S)) return;
    // the last workgroup of the tile: partials summed in split order, then
    // cleared (the workspace is zero again after the call).  The loads of a
    // batch of splits are all issued before the first is added, so the sum
    // costs one memory round trip per batch rather than one per split.
    // (Each load is a split's base address, the same for the whole
    // workgroup, plus the element's 32-bit byte offset: a split holds
    // M * N * 4 < 2^31 bytes.)
    constexpr int kBatch = 32;
    for (int idx = threadIdx.x; idx < total; idx += 64 * WAVES) {
        const int m = idx / COLS, c = idx - m * COLS;
        const int n = n_base + c;
        if (n >= N) continue;
        const uint32_t off = ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 4u;
        auto at = [&](int sp) { return (float *)((char *)(part + (size_t)sp * slot) + off); };
        float v = 0.f;
        for (int s0 = 0; s0 < S; s0 += kBatch) {
            float b[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                b[i] = s0 + i < S ? __hip_atomic_load(at(s0 + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) v += b[i];
        }
        for (int sp = 0; sp < S; ++sp) __hip_atomic_store(at(sp), 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        y[(size_t)m * N + n] = f32_to_out_bits(v, DT);
    }
}

// ===========================================================================
// Decode kernel.  grid = (column tiles, ceil(chunks / WAVES)), 64*WAVES
// threads.  Dynamic LDS: WAVES * M * (128*BLK) floats.  Workspace (when gridDim.y > 1):
// fp16, one counting accumulator per output element, acc64[M][N]; bf16, one
// arrival counter per column tile and fp32 partials [S][M][N] (device.hpp).
// The launch bound asks for 4 waves per SIMD (<= 128 registers) at CS <= 2:
// the whole weight stream of a layer must be in flight at once, and this fits
// without spills (measured faster than the compiler's own 3-wave allocation).
// CS = 4 (one 128-k group per wave, about 140 registers, 3 waves per SIMD)
// halves the workgroup count for layers whose CS = 2 grid would not be
// resident all at once, so that they still run as a single round.  WAVES = 8
// (the same waves per SIMD in half as many workgroups) halves the K splits,
// and so the per-element atomics, which grow with M.
template <int BLK, int CS, int DT, bool SYM, int WAVES>
__global__ __launch_bounds__(64 * WAVES, (CS >= 4 ? 2 : 4) * 4 / WAVES) void w4a16_decode(const uint16_t *__restrict__ x, const uint32_t *__restrict__ qw,
                                                    const uint16_t *__restrict__ sc,
                                                    const uint32_t *__restrict__ qz, uint16_t *__restrict__ y,
                                                    uint64_t *__restrict__ acc64, int M, int N, int K, int G) {
    extern __shared__ float red[];
    constexpr int CK = 32 * CS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, gq = lane >> 4;
    const int nw = N >> 3;
    const int tile = blockIdx.x;
    const int wcol0 = tile * 16 * BLK + j * BLK;  // lane's first word-column
    const bool col_ok = wcol0 < nw;
    // lanes past the last word-column load the last in-bounds words instead
    // (their sums are never stored), so that every load is unconditional
    const int wld = col_ok ? wcol0 : nw - BLK;
    const int chunk = blockIdx.y * WAVES + wave;
    const bool active = chunk < K / CK;

    f32x4 acc[BLK][8];
#pragma unroll
    for (int b = 0; b < BLK; ++b)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[b][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (active) {
        const int k0 = chunk * CK;
        const int g = k0 / G;  // the chunk lies inside one group
        // every load of the chunk is issued before any is used; the scales,
        // zero points and activations go first, so that they do not queue
        // behind the weight stream
        u32x4 s4[BLK];
        uint32_t zw[BLK];
#pragma unroll
        for (int b = 0; b < BLK; ++b) {
            s4[b] = *(const u32x4 *)(sc + (size_t)g * N + 8 * (wld + b));
            zw[b] = SYM ? 0x88888888u : qz[(size_t)g * nw + wld + b];
        }
        u32x4 a[CS];
        const int xr = j < M ? j : 0;  // rows past M read row 0 and are zeroed below
#pragma unroll
        for (int s = 0; s < CS; ++s) a[s] = *(const u32x4 *)(x + (size_t)xr * K + k0 + 32 * s + 8 * gq);
        // keep the issue order: the scheduler would otherwise sink the small
        // loads next to their late use, a whole memory round trip later
        __builtin_amdgcn_sched_barrier(0);
        uint32_t w[CS][8][BLK];
#pragma unroll
        for (int s = 0; s < CS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                load_words<BLK, true>(qw + (size_t)(k0 + 32 * s + 8 * gq + e) * nw + wld, true, w[s][e]);
        __builtin_amdgcn_sched_barrier(0);
        if (j >= M) {
#pragma unroll
            for (int s = 0; s < CS; ++s) a[s] = (u32x4){0, 0, 0, 0};
        }

        if (DT == DT_F16) {
            // B operand = the masked nibble pair itself, read as fp16
            // subnormals q * 2^-24 (or 16q * 2^-24 for an upper nibble): the
            // matrix core multiplies them exactly.  The zero point and scale
            // are applied per chunk:  s * (2^24 * sum(x q 2^-24) - z * sum(x)),
            // with sum(x) from one extra MFMA against an all-ones operand.
            const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
            f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < CS; ++s) rs = mfma_f16(a[s], ones, rs);
#pragma unroll
            for (int b = 0; b < BLK; ++b) {
#pragma unroll
                for (int s = 0; s < CS; ++s) {
                    uint32_t px[4], py[4], px8[4], py8[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        px[p] = pair_x(w[s][2 * p][b], w[s][2 * p + 1][b]);
                        py[p] = pair_y(w[s][2 * p][b], w[s][2 * p + 1][b]);
                        px8[p] = px[p] >> 8;
                        py8[p] = py[p] >> 8;
                    }
#define AWQ4_COL(T_)                                                                                \
    {                                                                                               \
        u32x4 bop;                                                                                  \
        _Pragma("unroll") for (int p = 0; p < 4; ++p) {                                             \
            const uint32_t src = col_src_y(T_) ? (col_shift(T_) ? py8[p] : py[p])                   \
                                               : (col_shift(T_) ? px8[p] : px[p]);                  \
            bop[p] = src & (col_hi(T_) ? 0x00F000F0u : 0x000F000Fu);                                \
        }                                                                                           \
        acc[b][T_] = mfma_f16(a[s], bop, acc[b][T_]);                                               \
    }
                    AWQ4_COL(0) AWQ4_COL(1) AWQ4_COL(2) AWQ4_COL(3) AWQ4_COL(4) AWQ4_COL(5) AWQ4_COL(6) AWQ4_COL(7)
#undef AWQ4_COL
                }
                float at[8], bt[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float st = scale_f32<DT>(s4[b], t);
                    const float zt = SYM ? 8.0f : (float)((zw[b] >> (4 * col_nibble(t))) & 0xFu);
                    at[t] = st * (col_hi(t) ? 1048576.0f : 16777216.0f);  // s * 2^20 or s * 2^24
                    bt[t] = st * zt;
                }
                // only the first min(M, 4) of a lane's rows can be live (the
                // rows past M are zero and never stored): a uniform bound
                // instead of a per-lane row test
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (r < M) {
#pragma unroll
                        for (int t = 0; t < 8; ++t) acc[b][t][r] = __builtin_fmaf(acc[b][t][r], at[t], -bt[t] * rs[r]);
                    }
            }
        } else {
            // B operand = the exact integer 128 + q as bf16: the nibble ORed
            // into the mantissa of 128.0 (one bitwise op per pair; an upper
            // nibble is shifted down first).  The zero point and scale are
            // applied per chunk on the fp32 sums: s * (sum(x (128 + q)) -
            // (128 + z) * sum(x)), with sum(x) from one extra MFMA against an
            // all-ones operand.  Every product is exact in fp32, and the
            // sums of a chunk keep 2^-24 relative to 128 sum|x|, far below
            // the bf16 output's rounding.
            const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
            f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < CS; ++s) rs = mfma_bf16(a[s], ones, rs);
#pragma unroll
            for (int b = 0; b < BLK; ++b) {
#pragma unroll
                for (int s = 0; s < CS; ++s) {
                    // the pair registers shifted by 0, 4, 8 and 12 bits: the
                    // wanted nibble of column t then sits at bits 0 and 16
                    uint32_t px[4][4], py[4][4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        px[p][0] = pair_x(w[s][2 * p][b], w[s][2 * p + 1][b]);
                        py[p][0] = pair_y(w[s][2 * p][b], w[s][2 * p + 1][b]);
#pragma unroll
                        for (int h = 1; h < 4; ++h) {
                            px[p][h] = px[p][0] >> (4 * h);
                            py[p][h] = py[p][0] >> (4 * h);
                        }
                    }
#define AWQ4_COL(T_)                                                                                \
    {                                                                                               \
        constexpr int sh = (col_shift(T_) + 4 * col_hi(T_)) / 4;                                    \
        u32x4 bop;                                                                                  \
        _Pragma("unroll") for (int p = 0; p < 4; ++p) bop[p] = __builtin_amdgcn_bitop3_b32(        \
            col_src_y(T_) ? py[p][sh] : px[p][sh], 0x000F000Fu, 0x43004300u, 0xEA);                 \
        acc[b][T_] = mfma_bf16(a[s], bop, acc[b][T_]);                                              \
    }
                    AWQ4_COL(0) AWQ4_COL(1) AWQ4_COL(2) AWQ4_COL(3) AWQ4_COL(4) AWQ4_COL(5) AWQ4_COL(6) AWQ4_COL(7)
#undef AWQ4_COL
                }
                float st[8], bt[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    st[t] = scale_f32<DT>(s4[b], t);
                    const float zt = SYM ? 8.0f : (float)((zw[b] >> (4 * col_nibble(t))) & 0xFu);
                    bt[t] = st[t] * (128.0f + zt);  // exact: 8 + 8 significant bits
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (r < M) {
#pragma unroll
                        for (int t = 0; t < 8; ++t) acc[b][t][r] = __builtin_fmaf(acc[b][t][r], st[t], -bt[t] * rs[r]);
                    }
            }
        }
    }

    decode_epilogue<BLK, DT, WAVES>(acc, red, y, acc64, M, N, wave, gq, j, tile);
}

// ===========================================================================
// Tiled kernel: grid (ceil(N/256), ceil(M/BM), S), 256 threads = 2 x 2 waves,
// wave tile (16*MTW) x 128, BM = 32*MTW.
template <int MTW, int DT, bool SYM>
__global__ __launch_bounds__(256) void w4a16_tiled(const uint16_t *__restrict__ x, const uint32_t *__restrict__ qw,
                                                   const uint16_t *__restrict__ sc, const uint32_t *__restrict__ qz,
                                                   uint16_t *__restrict__ y, uint64_t *__restrict__ acc64, int M,
                                                   int N, int K, int G, int S) {
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

    ZeroConsts<DT> zc;
    uint32_t sc2[8];
    float sf[8];
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
            uint32_t zw = 0x88888888u;
            u32x4 s4 = {0, 0, 0, 0};
            if (col_ok) {
                s4 = *(const u32x4 *)(sc + (size_t)g * N + 8 * wcol);
                if (!SYM) zw = qz[(size_t)g * nw + wcol];
            }
            zero_consts<DT, SYM>(zc, zw);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t b = scale_bits<DT>(s4, t);
                sc2[t] = b | (b << 16);
                sf[t] = scale_f32<DT>(s4, t);
            }
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
                    f32x4 v0 = {acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                    f32x4 v1 = {acc[mt][4][r], acc[mt][5][r], acc[mt][6][r], acc[mt][7][r]};
                    *(u32x4 *)(y + (size_t)m * N + n0) = pack8_out<DT>(v0, v1);
                }
            }
        return;
    }
    // Split-K by partial tiles exchanged through agent-scope atomics
    // (device.hpp): store this split's partials, then the last workgroup of
    // the tile sums all splits in split order.
    uint32_t *const cnt = (uint32_t *)acc64 + (tn + gridDim.x * tm);
    uint64_t *const part = (uint64_t *)((char *)acc64 + split_counters_bytes((int64_t)gridDim.x * gridDim.y));
    const size_t slot = (size_t)M * N / 2;  // 64-bit words per split
    auto at = [&](int sp, int m) { return part + sp * slot + ((size_t)m * N + n0) / 2; };
    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * mt + 4 * gq + r;
                if (m >= M) continue;
                part_put(at(split, m), (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]});
                part_put(at(split, m) + 2, (f32x4){acc[mt][4][r], acc[mt][5][r], acc[mt][6][r], acc[mt][7][r]});
            }
    }
    if (!split_tile_last_atomic(cnt, S) || !col_ok) return;
    // the last split sums the partials in split order, two of the lane's
    // rows (four 16-byte vectors) at a time, then clears them
#pragma unroll
    for (int b = 0; b < 2 * MTW; ++b) {
        const int mt = b >> 1, r0 = 2 * (b & 1);
        auto row = [&](int i) { return m0 + 16 * mt + 4 * gq + r0 + (i >> 1); };
        auto addr = [&](int sp, int i) { return at(sp, row(i)) + 2 * (i & 1); };
        auto valid = [&](int i) { return row(i) < M; };
        f32x4 v[4];
        part_sum<4, 1>(v, S, addr, valid);
        part_clear_all<4>(S, addr, valid);
#pragma unroll
        for (int r = 0; r < 2; ++r)
            if (valid(2 * r)) *(u32x4 *)(y + (size_t)row(2 * r) * N + n0) = pack8_out<DT>(v[2 * r], v[2 * r + 1]);
    }
}

// ===========================================================================
// Host launchers.

template <int BLK, int CS, int DT, bool SYM, int WAVES>
static hipError_t launch_decode_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    dim3 grid(p.tiles_n, p.splits);
    const size_t lds = (size_t)WAVES * a.M * 128 * BLK * sizeof(float);
    hipLaunchKernelGGL((w4a16_decode<BLK, CS, DT, SYM, WAVES>), grid, dim3(64 * WAVES), lds, st,
                       (const uint16_t *)a.x, (const uint32_t *)a.qweight, (const uint16_t *)a.scales,
                       (const uint32_t *)a.qzeros, (uint16_t *)a.y, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G);
    return hipGetLastError();
}

template <int BLK, int CS, int WAVES>
static hipError_t launch_decode_dt(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16) return sym ? launch_decode_t<BLK, CS, DT_F16, true, WAVES>(a, p, st)
                                      : launch_decode_t<BLK, CS, DT_F16, false, WAVES>(a, p, st);
    return sym ? launch_decode_t<BLK, CS, DT_BF16, true, WAVES>(a, p, st)
               : launch_decode_t<BLK, CS, DT_BF16, false, WAVES>(a, p, st);
}

hipError_t launch_w4a16_decode(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    switch (p.waves * 100 + p.blk * 10 + p.cs) {
        case 411: return launch_decode_dt<1, 1, 4>(a, p, st);
        case 412: return launch_decode_dt<1, 2, 4>(a, p, st);
        case 421: return launch_decode_dt<2, 1, 4>(a, p, st);
        case 422: return launch_decode_dt<2, 2, 4>(a, p, st);
        case 414: return launch_decode_dt<1, 4, 4>(a, p, st);
        case 424: return launch_decode_dt<2, 4, 4>(a, p, st);
        case 811: return launch_decode_dt<1, 1, 8>(a, p, st);
        case 812: return launch_decode_dt<1, 2, 8>(a, p, st);
        case 821: return launch_decode_dt<2, 1, 8>(a, p, st);
        case 822: return launch_decode_dt<2, 2, 8>(a, p, st);
        case 814: return launch_decode_dt<1, 4, 8>(a, p, st);
        case 824: return launch_decode_dt<2, 4, 8>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}


template <int MTW, int DT, bool SYM>
static hipError_t launch_tiled_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    dim3 grid(p.tiles_n, p.tiles_m, p.splits);
    hipLaunchKernelGGL((w4a16_tiled<MTW, DT, SYM>), grid, dim3(256), 0, st, (const uint16_t *)a.x,
                       (const uint32_t *)a.qweight, (const uint16_t *)a.scales, (const uint32_t *)a.qzeros,
                       (uint16_t *)a.y, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits);
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
