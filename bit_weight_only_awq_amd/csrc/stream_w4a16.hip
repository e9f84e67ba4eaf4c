// stream_w4a16.hip -- AWQ W4A16 for 8 < M <= 64 on gfx950: the streaming kernel.
//
// Method as in w4a16.hip (vLLM pull request "Speed up AWQ 2.5x with updated
// kernel": the first-generation AWQ order map; w = (q - z) * s, z = 8 when
// symmetric per the AutoAWQ pull request "Marlin symmetric quantization and
// inference").
//
// A workgroup owns a column tile of 128 outputs and a range of the K
// chunks (32 * CS consecutive k inside one quantisation group); grid y = S
// splits of the chunks.  Its WV waves take the range's chunks in turn (wave
// w: chunks w, w + WV, ..., so at any time the waves read WV consecutive
// chunks of the tile) and keep two chunks' loads in flight in a register
// ring, so that the grid fits the GPU in one round with few K splits and the
// weight stream never drains between chunks.  Lanes are laid out as in the
// decode kernel: lane (j, gq) holds word-column j of the tile (8 outputs) at
// the 8 k-rows 8 gq + e of each 32-k step.  The matrix cores multiply MT
// 16-row tiles of X by B = (q - z) * s rounded once (fp16, four row tiles),
// or by the exact (q - z) with the chunk's sums scaled once in fp32.  The waves' tiles are then added through LDS in wave order and the
// S workgroups of a column tile exchange fp32 partials, the last one adding
// them in split order -- so the result does not depend on timing.
#include "device.hpp"
#include "launch.hpp"
#include "w4a16_ops.hpp"

namespace awq4 {

// Position of column c inside a parked row.  Lane j holds columns 8j .. 8j+7
// of its rows and parks them as two 16-byte halves: half h of every lane sits
// in the h-th half of the row, at the lane's 16-byte slot (4j floats), so the
// 16 lanes of a row write 16 consecutive slots -- all of the LDS banks, no
// two lanes of a write on one bank.  (Columns in plain order put lanes j and
// j+8 on the same banks and the four row groups of a wave on the same ones
// again: eight-way conflicts.)
template <int COLS>
__device__ __forceinline__ int lds_col(int c) {
    return (COLS / 2) * ((c >> 2) & 1) + 4 * (c >> 3) + (c & 3);
}

// The workgroup's M x COLS tile sum -- the SLOTS tiles its waves parked in
// LDS (ROWS x COLS floats each, COLS a row in the order lds_col gives), added
// in slot order -- goes out: written directly when the K range is not split
// (S == 1); otherwise handed over as fp32 partials (one M x N array per
// split after the tile counters), added in split order -- by the reduction
// kernel launched next where they are large (sep), else by the last
// workgroup of the column tile (device.hpp: split_tile_last_atomic), which
// also clears them and writes the output.  Everything moves as quads of columns (N is a
// multiple of 8, so a quad never straddles the last column): 8-byte output
// stores, 16-byte partial loads and stores.  The partials move with the
// cache policy of agent-scope atomic loads and stores (sc1: through to the
// device-wide coherence point), as 16-byte buffer accesses -- half the
// requests of 8-byte atomics; the tail of the kernel is the last workgroups'
// partial traffic, so its request count sets the tail's length.

template <int NT, int DT, int ROWS, int COLS, int SLOTS>
__device__ __forceinline__ void tile_store_or_exchange(const float *red, uint16_t *__restrict__ y,
                                                       uint64_t *__restrict__ ws, int M, int N, int tile, int S,
                                                       int sep) {
    constexpr int QR = COLS / 4;         // quads per row
    constexpr int kQ = ROWS * QR / NT;   // quads per thread, whole tile
    static_assert(kQ >= 1 && kQ * NT == ROWS * QR, "whole quads per thread");
    const int n_base = tile * COLS;
    const int quads = M * QR;
    // thread t takes quads t, t + NT, ...: its sums of the SLOTS parked tiles
    // and their 16-byte index in an [M, N] array
    f32x4 v[kQ];
    bool ok[kQ];
    uint32_t at[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int qi = threadIdx.x + q * NT;
        const int r = qi / QR, c = 4 * (qi % QR);
        ok[q] = qi < quads && n_base + c < N;
        at[q] = ok[q] ? (uint32_t)(r * (N / 4) + (n_base + c) / 4) : 0u;
        v[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (ok[q]) {
            const float *p = red + r * COLS + lds_col<COLS>(c);
            v[q] = *(const f32x4 *)p;
#pragma unroll
            for (int w = 1; w < SLOTS; ++w) v[q] += *(const f32x4 *)(p + w * ROWS * COLS);
        }
    }
    auto out_quad = [&](uint32_t a, f32x4 t) { *(uint2 *)(y + 4 * (size_t)a) = quad_out_bits<DT>(t); };
    if (S == 1) {
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            if (ok[q]) out_quad(at[q], v[q]);
        return;
    }
    // split s's partials: a buffer over its M x N floats (under 2^31 bytes,
    // which the planner ensures)
    char *const part = (char *)ws + split_counters_bytes(gridDim.x);
    const uint32_t slot_bytes = (uint32_t)M * (uint32_t)N * 4u;
    auto split_rsrc = [&](int s) { return buf_rsrc(part + (size_t)s * slot_bytes, slot_bytes); };
    const int own = blockIdx.y;
    // sep: the reduction kernel launched next adds the splits (plain stores,
    // made visible by the kernel boundary); else the column tile's last
    // workgroup adds them below.
    {
        const __amdgpu_buffer_rsrc_t rs = split_rsrc(own);
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            if (ok[q]) {
                if (sep) __builtin_amdgcn_raw_buffer_store_b128(bit_as<u32x4>(v[q]), rs, at[q] * 16u, 0, 0);
                else __builtin_amdgcn_raw_buffer_store_b128(bit_as<u32x4>(v[q]), rs, at[q] * 16u, 0, kPartCoherent);
            }
    }
    if (sep || !split_tile_last_atomic((uint32_t *)ws + tile, S)) return;
    // The last workgroup of the column tile: the other splits' partials of
    // all its quads, kB splits at a time with every load of a batch issued
    // before the first add (one memory round trip per batch), added in split
    // order with its own partial (still in registers) in its place.
    constexpr int kB = 32 / kQ < 1 ? 1 : 32 / kQ > 8 ? 8 : 32 / kQ;
    f32x4 sum[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) sum[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kB) {
        u32x4 b[kQ][kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const int s = s0 + i;
#pragma unroll
            for (int q = 0; q < kQ; ++q) b[q][i] = (u32x4){0u, 0u, 0u, 0u};
            if (s < S && s != own) {
                const __amdgpu_buffer_rsrc_t rs = split_rsrc(s);
#pragma unroll
                for (int q = 0; q < kQ; ++q)
                    if (ok[q]) b[q][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, at[q] * 16u, 0, kPartCoherent);
            }
        }
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const int s = s0 + i;
            if (s >= S) break;
#pragma unroll
            for (int q = 0; q < kQ; ++q) sum[q] += s == own ? v[q] : bit_as<f32x4>(b[q][i]);
        }
    }
    for (int s = 0; s < S; ++s) {
        const __amdgpu_buffer_rsrc_t rs = split_rsrc(s);
#pragma unroll
        for (int q = 0; q < kQ; ++q)
            if (ok[q]) __builtin_amdgcn_raw_buffer_store_b128((u32x4){0u, 0u, 0u, 0u}, rs, at[q] * 16u, 0, kPartCoherent);
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q)
        if (ok[q]) out_quad(at[q], sum[q]);
}

// One chunk's loads: scales and zero points of its group, MT row tiles of X
// (from L2: every column tile reads the same rows), the packed words.
template <int MT, int CS>
struct StreamBuf {
    u32x4 s4;
    uint32_t zw;
    u32x4 a[MT][CS];
    uint32_t w[CS][8];
};

// Per-lane byte offsets of a wave's loads, fixed for the whole kernel; the
// chunk's own offsets (its k0 and group) are uniform, so each load is a
// scalar base plus one of these, with no per-load 64-bit address arithmetic.
template <int MT>
struct StreamOffsets {
    uint32_t w;      // packed word of row 8 gq, word-column wld
    uint32_t s;      // 8 scales of word-column wld
    uint32_t z;      // zero-point word of word-column wld
    uint32_t x[MT];  // X row 16 mt + j (row 0 past M), k offset 8 gq
};

template <int MT, int CS, bool SYM>
__device__ __forceinline__ void stream_issue(StreamBuf<MT, CS> &b, const StreamOffsets<MT> &o,
                                             const uint16_t *__restrict__ x, const uint32_t *__restrict__ qw,
                                             const uint16_t *__restrict__ sc, const uint32_t *__restrict__ qz,
                                             int chunk, int lgG, int N, int nw) {
    const int k0 = chunk * 32 * CS;
    const int g = k0 >> lgG;  // the chunk lies inside one group
    auto at = [](const void *base, uint32_t off) { return (const char *)base + off; };
    b.s4 = *(const u32x4 *)at(sc + (size_t)g * N, o.s);
    b.zw = SYM ? 0x88888888u : *(const uint32_t *)at(qz + (size_t)g * nw, o.z);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < CS; ++s) b.a[mt][s] = *(const u32x4 *)at(x + k0 + 32 * s, o.x[mt]);
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            b.w[s][e] = __builtin_nontemporal_load((const uint32_t *)at(qw + (size_t)(k0 + 32 * s + e) * nw, o.w));
}

// One chunk into the accumulators.
//  fp16 with four row tiles: B = (q - z) * s rounded once to fp16 (the exact
//  (q - z) from the magic-exponent pair, times the column's scale in both
//  halves), the MFMAs accumulating straight into acc -- the weights the LDS
//  GEMM uses.  At 64 rows the fp32 path below costs 128 FMAs a chunk against
//  64 packed multiplies here: gate/up at M = 64 40.3 -> 36.3 us, down 31.3 ->
//  29.4; with one or two row tiles the multiplies cost more than the FMAs
//  they replace (M = 32 gate/up 28.8 -> 29.7 us), so those keep the fp32 path.
//  Otherwise: B = the exact integer (q - z); for each column MFMA the chunk's
//  CS k-steps are summed in a small fp32 temporary that is then scaled by s
//  once and added (no weight is rounded).
template <int MT, int CS, int DT, bool SYM>
__device__ __forceinline__ void stream_compute(const StreamBuf<MT, CS> &b, f32x4 (&acc)[MT][8]) {
    ZeroConsts<DT> zc;
    zero_consts<DT, SYM>(zc, b.zw);
    uint32_t px[CS][4], py[CS][4];
#pragma unroll
    for (int s = 0; s < CS; ++s)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            px[s][p] = pair_x(b.w[s][2 * p], b.w[s][2 * p + 1]);
            py[s][p] = pair_y(b.w[s][2 * p], b.w[s][2 * p + 1]);
        }
    if constexpr (DT == DT_F16 && MT >= 4) {
        static_for<8>([&](auto tc) {
            constexpr int T = decltype(tc)::value;
            const uint32_t sb = scale_bits<DT>(b.s4, T);
            const uint32_t sc2 = sb | (sb << 16);
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                u32x4 bop;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    bop[p] = bit_as<uint32_t>(bit_as<f16x2>(qz_pair<DT, T>(col_src_y(T) ? py[s][p] : px[s][p], zc)) *
                                              bit_as<f16x2>(sc2));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][T] = mma<DT>(b.a[mt][s], bop, acc[mt][T]);
            }
        });
    } else {
        static_for<8>([&](auto tc) {
            constexpr int T = decltype(tc)::value;
            f32x4 t[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) t[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                u32x4 bop;
#pragma unroll
                for (int p = 0; p < 4; ++p) bop[p] = qz_pair<DT, T>(col_src_y(T) ? py[s][p] : px[s][p], zc);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) t[mt] = mma<DT>(b.a[mt][s], bop, t[mt]);
            }
            const float st = scale_f32<DT>(b.s4, T);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][T][r] = __builtin_fmaf(t[mt][r], st, acc[mt][T][r]);
            // two groups of four columns: bounds how many temporaries the
            // scheduler keeps live at once (all eight spill a few registers)
            if (T == 3) __builtin_amdgcn_sched_barrier(0);
        });
    }
}

// Keeps a buffer's loads where they are issued, a chunk ahead of their use:
// the empty asm statement stops the optimiser from sinking them next to it,
// the scheduling barrier stops the instruction scheduler from pulling the
// next chunk's arithmetic, and so its waits, above them.
__device__ __forceinline__ void prefetch_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int MT, int CS, int WV, int DT, bool SYM>
__global__ __launch_bounds__(64 * WV, 1) void w4a16_stream(const uint16_t *__restrict__ x,
                                                          const uint32_t *__restrict__ qw,
                                                          const uint16_t *__restrict__ sc,
                                                          const uint32_t *__restrict__ qz, uint16_t *__restrict__ y,
                                                          uint64_t *__restrict__ ws, int M, int N, int K, int lgG,
                                                          int sep) {
    constexpr int ROWS = 16 * MT, COLS = 128;
    // one parked ROWS x COLS tile per wave (128 KB at 4 row tiles)
    __shared__ __attribute__((aligned(16))) float red[WV * ROWS * COLS];
    const int lane = threadIdx.x & 63;
    // the wave index in a scalar register: the chunk loop below is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, gq = lane >> 4;
    const int nw = N >> 3;
    // A wave reads 64 bytes of each packed k-row; the other half of that
    // 128-byte line belongs to the neighbouring tile.  Neighbouring tiles go
    // to one XCD, so that the line is fetched into one L2 instead of two.
    // (Two word-columns per lane, whole lines per wave, measured slower: the
    // doubled accumulators cost half the waves per CU.)
    const int tile = tile_of_xcd_order(blockIdx.x, gridDim.x);
    const int wcol = tile * 16 + j;
    const int wld = wcol < nw ? wcol : nw - 1;  // past the last word-column: in-bounds words, sums never stored
    // this workgroup's chunks [c_lo, c_hi) and this wave's share of them
    const int S = gridDim.y;
    const int nchunks = K / (32 * CS);
    const int per = (nchunks + S - 1) / S;
    const int c_lo = blockIdx.y * per;
    const int c_hi = min(nchunks, c_lo + per);
    const int n = c_hi - c_lo > wave ? (c_hi - c_lo - wave + WV - 1) / WV : 0;
    // (the per-lane parts stay small: 8 k-rows of packed words, and at most
    // 64 rows of X -- rows past M read row 0, their sums never stored)
    StreamOffsets<MT> off;
    off.w = (uint32_t)(8 * gq * nw + wld) * 4u;
    off.s = (uint32_t)wld * 16u;
    off.z = (uint32_t)wld * 4u;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = 16 * mt + j;
        off.x[mt] = (uint32_t)((row < M ? row : 0) * K + 8 * gq) * 2u;
    }

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Two chunks in flight: chunk i + 2 is issued while chunk i + 1 is
    // computed.  The loop runs while both of its prefetches exist; the last
    // one or two chunks are finished after it, so that no load is issued past
    // the wave's last chunk.
    auto chunk_of = [&](int i) { return c_lo + wave + i * WV; };
    StreamBuf<MT, CS> b0, b1;
    if (n == 1) {
        stream_issue<MT, CS, SYM>(b0, off, x, qw, sc, qz, chunk_of(0), lgG, N, nw);
        stream_compute<MT, CS, DT, SYM>(b0, acc);
    } else if (n >= 2) {
        stream_issue<MT, CS, SYM>(b0, off, x, qw, sc, qz, chunk_of(0), lgG, N, nw);
        stream_issue<MT, CS, SYM>(b1, off, x, qw, sc, qz, chunk_of(1), lgG, N, nw);
        prefetch_fence();
        int i = 0;
        for (; i + 3 < n; i += 2) {
            stream_compute<MT, CS, DT, SYM>(b0, acc);
            stream_issue<MT, CS, SYM>(b0, off, x, qw, sc, qz, chunk_of(i + 2), lgG, N, nw);
            prefetch_fence();
            stream_compute<MT, CS, DT, SYM>(b1, acc);
            stream_issue<MT, CS, SYM>(b1, off, x, qw, sc, qz, chunk_of(i + 3), lgG, N, nw);
            prefetch_fence();
        }
        // chunks i and i + 1 are in flight; n - i is 2 or 3
        stream_compute<MT, CS, DT, SYM>(b0, acc);
        if (i + 2 < n) {
            stream_issue<MT, CS, SYM>(b0, off, x, qw, sc, qz, chunk_of(i + 2), lgG, N, nw);
            prefetch_fence();
            stream_compute<MT, CS, DT, SYM>(b1, acc);
            stream_compute<MT, CS, DT, SYM>(b0, acc);
        } else {
            stream_compute<MT, CS, DT, SYM>(b1, acc);
        }
    }

    // Lane holds rows 16 mt + 4 gq + r and columns 8 j + t of the tile.
    auto slot_of = [&](int sl, int mt, int r) {
        return red + ((size_t)sl * ROWS + 16 * mt + 4 * gq + r) * COLS + 4 * j;  // lds_col(8 j)
    };
    auto park = [&](int sl) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *d = slot_of(sl, mt, r);
                const f32x4(&v)[8] = acc[mt];
                *(f32x4 *)d = (f32x4){v[0][r], v[1][r], v[2][r], v[3][r]};
                *(f32x4 *)(d + COLS / 2) = (f32x4){v[4][r], v[5][r], v[6][r], v[7][r]};
            }
    };
    // every wave parks its tile in a slot of its own, all at once; the
    // exchange below adds the WV slots of each element in wave order (a
    // fixed order: the sum does not depend on timing).  (A tree of wave
    // pairs, half the LDS, took about 3 us at 64 rows: five dependent LDS
    // passes with one or two waves at work in each.)
    park(wave);
    __syncthreads();
    tile_store_or_exchange<64 * WV, DT, ROWS, COLS, WV>(red, y, ws, M, N, tile, S, sep);
}

template <int MT, int CS, int DT, bool SYM>
static hipError_t launch_stream_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    constexpr int WV = kStreamWaves(MT);
    if (p.waves != WV || (p.splits > 1 && p.acc == nullptr)) return hipErrorInvalidValue;
    const int sep = split_reduce_apart(p.splits, 16 * MT);
    hipLaunchKernelGGL((w4a16_stream<MT, CS, WV, DT, SYM>), dim3(p.tiles_n, p.splits), dim3(64 * WV), 0, st,
                       (const uint16_t *)a.x, (const uint32_t *)a.qweight, (const uint16_t *)a.scales,
                       (const uint32_t *)a.qzeros, (uint16_t *)a.y, p.acc, (int)a.M, (int)a.N, (int)a.K,
                       __builtin_ctz((unsigned)a.G), sep);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !sep) return e;
    return launch_w4a16_split_reduce(a, p, p.tiles_n, st);
}

template <int MT, int CS>
static hipError_t launch_stream_dt(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16)
        return sym ? launch_stream_t<MT, CS, DT_F16, true>(a, p, st) : launch_stream_t<MT, CS, DT_F16, false>(a, p, st);
    return sym ? launch_stream_t<MT, CS, DT_BF16, true>(a, p, st) : launch_stream_t<MT, CS, DT_BF16, false>(a, p, st);
}

// p.mt: 16-row tiles (1, 2, 4); p.cs: 32-k steps per chunk (1, 2)
hipError_t launch_w4a16_stream(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    switch (p.mt * 10 + p.cs) {
        case 11: return launch_stream_dt<1, 1>(a, p, st);
        case 12: return launch_stream_dt<1, 2>(a, p, st);
        case 21: return launch_stream_dt<2, 1>(a, p, st);
        case 22: return launch_stream_dt<2, 2>(a, p, st);
        case 41: return launch_stream_dt<4, 1>(a, p, st);
        case 42: return launch_stream_dt<4, 2>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace awq4
