// gemm_w4a8.hip -- W4A8 GEMM for large M on gfx950 (int8 matrix cores).
//
// Same method as w4a8.hip (vLLM pull request "Support W4A8 quantization for
// vllm": int4 placed in the upper nibble of an int8, int32 accumulation, s1
// per token and s2 per channel on the output, per-group scales in addition
// for grouped weights -- here integer s3 folded into the int8 weights).
//
// The int4 -> int8 step costs two VALU instructions per word, so a 64 x 64
// wave tile keeps the VALU far below the matrix cores; what bounds this
// kernel is LDS latency, which the copy ring and the operand prefetch hide.
#include "device.hpp"
#include "launch.hpp"

namespace awq4 {

constexpr int W8_M = 128, W8_K = 64;
constexpr int W8_RING = 4;                         // stages per LDS ring (copied W8_RING - 1 ahead)
constexpr int W8_APITCH = W8_K;                    // 64 bytes of a8 per row (4 segments, swizzled)
constexpr int W8_ABYTES = W8_M * W8_APITCH;        // 8192 per stage

// NW waves per workgroup in a 2 x (NW/2) grid of 64 x 64 wave tiles: the
// workgroup tile is 128 x 32*NW (NW = 4: 128 x 128; NW = 8: 128 x 256, which
// halves the a8 bytes copied per matrix-core instruction).
template <int NW, bool GROUP>
struct W8Layout {
    static constexpr int WN = 32 * NW;                    // workgroup tile width
    static constexpr int WORDS = (W8_K / 8) * WN * 4;     // 8 word rows x WN columns x 4 B
    static constexpr int S3 = 2 * WN * 2;                 // s3 of the stage's two 32-k halves
    static constexpr int BBYTES = WORDS + (GROUP ? S3 : 0);
    static constexpr int OFF_B = W8_RING * W8_ABYTES;
    static constexpr int LDS = OFF_B + W8_RING * BBYTES;  // NW = 4: 49152 / 51200; NW = 8: 65536 / 69632
    static constexpr int A_COPIES = 8 / NW;               // 16-row a8 copies per wave and stage
    static constexpr int COPIES = A_COPIES + 1 + (GROUP ? 1 : 0);  // copies per wave and stage
    static constexpr int WROWS = 256 / WN;                // word rows per wave's word copy
};

// a8 rows: 16-byte segment s of row r is stored at s ^ f(r), f(r) = ((r >> 1)
// ^ (r >> 2)) & 3.  The 16 rows read by one operand load (a row per lane,
// same segment) then fall on distinct 16-byte bank groups whether the LDS
// serves 8 lanes over 32 banks or 16 lanes over 64 banks per cycle: rows
// 2 apart (and rows 4 apart) always get different f.
__device__ __forceinline__ int a8seg(int r, int s) { return s ^ (((r >> 1) ^ (r >> 2)) & 3); }

// Workgroup tile 128 x 32*NW, K in stages of 64 (one 16x16x64 step); NW waves
// in a 2 x NW/2 grid, each owning 64 x 64 outputs: 4 row tiles x 4 column MFMAs.
// KS = 2: two such groups of NW waves share the tile and split its K stages,
// each with its own LDS ring, and add their int32 sums through LDS at the end
// (twice the waves per SIMD when there are no more tiles than CUs).
// Lane j reads 16 bytes = 4 consecutive columns of two K8 word rows, which
// give the B operands of its 4 MFMAs (output column = 64 wn + 4j + u).
// a8 rows, word rows and (grouped) s3 rows are copied into 4-slot LDS rings
// three stages ahead; each stage waits only for the copies older than its
// own, so the next stage is always readable and its operands are loaded while
// the current stage's MFMAs run.
template <int NW, int KS, bool GROUP, int DT>
__global__ __launch_bounds__(64 * NW * KS, 2 / KS) void w4a8_gemm_lds(const int8_t *__restrict__ a8, const uint32_t *__restrict__ bq,
                                                       const float *__restrict__ s1, const uint16_t *__restrict__ s2,
                                                       const uint16_t *__restrict__ s3, uint16_t *__restrict__ y,
                                                       int32_t *__restrict__ acc_out, uint64_t *__restrict__ acc64,
                                                       int M, int N, int K, int G, int S, int sep) {
    using L = W8Layout<NW, GROUP>;
    constexpr int W8_N = L::WN;
    static_assert(KS * L::LDS >= KS * NW * 8 * 64 * 16, "the K-split handover fits in the rings");
    __shared__ __attribute__((aligned(16))) unsigned char lds_all[KS * L::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int grp = KS == 1 ? 0 : wv / NW, wave = wv % NW;
    unsigned char *const lds = lds_all + grp * L::LDS;
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave / (NW / 2), wn = wave % (NW / 2);
    // logical tile of this workgroup (XCD-aware order over the tiles_n x tiles_m grid)
    const int tile = tile_of_xcd_order(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int tn = tile % gridDim.x, tm = tile / gridDim.x, split = blockIdx.z;
    const int m0 = tm * W8_M, n0 = tn * W8_N;
    const int Tst = K / W8_K;
    const int w_lo = (int)((int64_t)Tst * split / S), w_hi = (int)((int64_t)Tst * (split + 1) / S);
    // stages of this group: group 0 the first ceil(n/KS), group 1 the rest;
    // both pass `iters` stage barriers (group 1 adds an idle one if n is odd)
    const int iters = (w_hi - w_lo + KS - 1) / KS;
    const int s_lo = w_lo + grp * iters, s_hi = min(w_hi, s_lo + iters);

    // Copy assignment.  a8: wave w copies rows 16 (A_COPIES w + i) + lane/4
    // (i < A_COPIES), lane%4 being the stored segment position; rows past M
    // repeat row M-1 (their outputs are never stored).  Words: wave w copies
    // word rows WROWS w .. WROWS w + WROWS - 1, lane % (W8_N/4) being the
    // 4-column segment; columns past N repeat the last 4.  s3 (grouped): wave
    // w, lanes 0..7, copies 16-byte segments 8w..8w+7 of the stage's two s3
    // rows (W8_N/8 segments per row).
    uint32_t aoff[L::A_COPIES];
#pragma unroll
    for (int i = 0; i < L::A_COPIES; ++i) {
        const int r = 16 * (L::A_COPIES * wave + i) + (lane >> 2);
        const int m = min(m0 + r, M - 1);
        aoff[i] = (uint32_t)((m - m0) * K + 16 * a8seg(r, lane & 3));
    }
    uint32_t boff;
    {
        const int r = L::WROWS * wave + lane / (W8_N / 4);
        const int c = min(n0 + 4 * (lane % (W8_N / 4)), N - 4);
        boff = (uint32_t)((r * N + c) * 4);
    }
    const int s3_seg = 8 * wave + (lane & 7);
    const int s3_h = s3_seg / (W8_N / 8);  // wave-uniform: the first NW/2 waves copy half 0
    const uint32_t s3_off = (uint32_t)(2 * min(n0 + 8 * (s3_seg % (W8_N / 8)), N - 8));
    const int lg = GROUP ? __builtin_ctz(G) : 0;
    // buffer descriptors (the planner keeps every byte offset under 2^31):
    // a8 rows from m0, the packed words, the s3 rows; per-lane offsets above,
    // the stage's offset as a scalar
    const __amdgpu_buffer_rsrc_t ars = buf_rsrc(a8 + (size_t)m0 * K, (int64_t)(M - m0) * K);
    const __amdgpu_buffer_rsrc_t brs = buf_rsrc(bq, (int64_t)(K / 8) * N * 4);
    const __amdgpu_buffer_rsrc_t grs = buf_rsrc(GROUP ? (const void *)s3 : (const void *)bq,
                                                GROUP ? (int64_t)(K / G) * N * 2 : 0);

    auto copy_stage = [&](int st, int slot) {
        unsigned char *A = lds + slot * W8_ABYTES + 16 * L::A_COPIES * wave * W8_APITCH;
#pragma unroll
        for (int i = 0; i < L::A_COPIES; ++i)
            dma16_buf(ars, aoff[i], (uint32_t)(st * W8_K), A + 16 * i * W8_APITCH);
        unsigned char *B = lds + L::OFF_B + slot * L::BBYTES;
        dma16_buf(brs, boff, (uint32_t)st * (W8_K / 8) * (uint32_t)N * 4, B + L::WROWS * wave * (W8_N * 4));
        if (GROUP && lane < 8) {
            const int g = (st * W8_K + 32 * s3_h) >> lg;
            dma16_buf(grs, s3_off, (uint32_t)g * (uint32_t)N * 2, B + L::WORDS + 16 * s3_seg);
        }
    };

    i32x4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[mt][u] = (i32x4){0, 0, 0, 0};

    const int cl = 64 * wn + 4 * j;  // this lane's first column within the tile
    const uint32_t a_off = (uint32_t)((wm * 64 + j) * W8_APITCH + a8seg(j, gq) * 16);
    const uint32_t w_off = (uint32_t)(L::OFF_B + (2 * gq) * (W8_N * 4) + cl * 4);
    const uint32_t g_off = (uint32_t)(L::OFF_B + L::WORDS + (gq >> 1) * (W8_N * 2) + cl * 2);

    // operands of the stage in ring slot `slot`
    struct Ops {
        u32x4 a[4];
        u32x4 b[4];
    };
    // group scale of column cl + u from the stage's two s3 rows
    auto group_scales = [&](u32x2 sv, uint32_t (&g3)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) g3[u] = (uint32_t)act_bits_to_f32<DT>((sv[u >> 1] >> (16 * (u & 1))) & 0xFFFFu);
    };
    auto load_ops = [&](int slot, Ops &o) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            o.a[mt] = *(const u32x4 *)(lds + slot * W8_ABYTES + a_off + mt * 16 * W8_APITCH);
        // 16-byte aligned (the compiler cannot see it through the ring
        // arithmetic and would split each quad into 4-byte pairs, which
        // collide across lane groups)
        const u32x4 *wq = (const u32x4 *)__builtin_assume_aligned(lds + slot * L::BBYTES + w_off, 16);
        const u32x4 w0 = wq[0];
        const u32x4 w1 = wq[W8_N / 4];
        uint32_t g3[4] = {16u, 16u, 16u, 16u};
        if (GROUP) group_scales(*(const u32x2 *)(lds + slot * L::BBYTES + g_off), g3);
#pragma unroll
        for (int u = 0; u < 4; ++u) o.b[u] = int8_b_operand<GROUP>(w0[u], w1[u], g3[u]);
    };
    // Stage st (its operands already in `o`): 16 MFMAs, each in its own slot.
    // Stage st + 1's packed words are read in the first slots; each a8
    // operand of stage st + 1 is read into `o` right after the MFMA that last
    // uses stage st's (slots 3, 7, 11, 15), and each int8 B operand is built
    // in place after its last use (slots 12..15).  One operand set in place,
    // not two in turn, keeps the kernel at or under 128 VGPRs (four waves per
    // SIMD: two 8-wave workgroups per CU), and no wave waits on its own LDS
    // reads.  Then wait for the copies older than this stage's and cross the
    // barrier.  Copies: stage st + 3 into the slot of stage st - 1 (finished
    // before the last barrier); near the end the last stage is copied again
    // into that slot, never read as data, so every stage issues the same
    // copies and the wait count is fixed.
    auto stage = [&](int st, Ops &o) {
        const unsigned rel = (unsigned)(st - s_lo);
        copy_stage(min(st + W8_RING - 1, s_hi - 1), (int)((rel + W8_RING - 1) % W8_RING));
        const unsigned char *nb = lds + ((rel + 1) % W8_RING) * L::BBYTES;
        const unsigned char *na = lds + ((rel + 1) % W8_RING) * W8_ABYTES + a_off;
        const u32x4 *wq = (const u32x4 *)__builtin_assume_aligned(nb + w_off, 16);
        u32x4 w0, w1;
        u32x2 sv;
        uint32_t g3[4] = {16u, 16u, 16u, 16u};
        static_for<16>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int mt = i >> 2, u = i & 3;
            acc[mt][u] = mfma_i8(o.a[mt], o.b[u], acc[mt][u]);
            if constexpr (i == 1) w0 = wq[0];
            if constexpr (i == 2) w1 = wq[W8_N / 4];
            if constexpr (i == 5 && GROUP) sv = *(const u32x2 *)(nb + g_off);
            if constexpr (i == 9 && GROUP) group_scales(sv, g3);
            if constexpr (u == 3) o.a[mt] = *(const u32x4 *)(na + mt * 16 * W8_APITCH);
            if constexpr (mt == 3) o.b[u] = int8_b_operand<GROUP>(w0[u], w1[u], g3[u]);
            __builtin_amdgcn_sched_barrier(0);
        });
        // copies still allowed in flight: those of stages st + 3 .. st + W8_RING - 1
        constexpr int kInFlight = (W8_RING - 3) * L::COPIES;
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kInFlight & 15) | ((kInFlight >> 4) << 14));
        // no memory fence (it would wait for every copy); the clobber keeps
        // LDS accesses from moving across the barrier
        asm volatile("s_barrier" ::: "memory");
    };

    {
        Ops o;
        if (s_lo < s_hi) {
#pragma unroll
            for (int d = 0; d < W8_RING - 1; ++d)
                if (s_lo + d < s_hi) copy_stage(s_lo + d, d);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (s_lo < s_hi) load_ops(0, o);
        for (int st = s_lo; st < s_hi; ++st) stage(st, o);
    }

    // Epilogue: lane holds rows m0 + 64 wm + 16 mt + 4 gq + r, columns
    // n0 + cl + u (u = 0..3, adjacent).  Per-channel accumulators carry the
    // x16 of the upper-nibble int8 and are divided exactly.
    const int nc = n0 + cl;
    const bool col_ok = nc < N;
    float s2f[4] = {0.f, 0.f, 0.f, 0.f};
    if (col_ok) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s2f[u] = act_bits_to_f32<DT>(s2[nc + u]);
    }
    auto store4 = [&](int m, i32x4 accv) {
        const float s1m = s1[m];
        int32_t v[4];
        uint16_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[u] = GROUP ? accv[u] : (accv[u] >> 4);
            o[u] = f32_to_out_bits((float)v[u] * s1m * s2f[u], DT);
        }
        *(u32x2 *)(y + (size_t)m * N + nc) = (u32x2){(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                     (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
        if (acc_out) *(i32x4 *)(acc_out + (size_t)m * N + nc) = (i32x4){v[0], v[1], v[2], v[3]};
    };
    if constexpr (KS == 2) {
        // (S == 1.)  Group 1's idle stage barrier, then both rings are free:
        // group 0 finishes row tiles 0, 1 of each wave tile and group 1 row
        // tiles 2, 3; each parks the other pair in LDS and adds the pair
        // parked for it (int32: exact in any order).
        for (int k = max(s_hi - s_lo, 0); k < iters; ++k) asm volatile("s_barrier" ::: "memory");
        wait_vm_all();
        __syncthreads();
        i32x4 *const mine = (i32x4 *)lds_all + (size_t)(grp * NW + wave) * 8 * 64 + lane;
        const i32x4 *const theirs = (const i32x4 *)lds_all + (size_t)((grp ^ 1) * NW + wave) * 8 * 64 + lane;
        if (grp == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int u = 0; u < 4; ++u) mine[(4 * h + u) * 64] = acc[2 + h][u];
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int u = 0; u < 4; ++u) mine[(4 * h + u) * 64] = acc[h][u];
        }
        __syncthreads();
        if (!col_ok) return;
        auto finish_pair = [&](auto mt0c) {
            constexpr int mt0 = decltype(mt0c)::value;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[mt0 + h][u] += theirs[(4 * h + u) * 64];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = m0 + wm * 64 + 16 * (mt0 + h) + 4 * gq + r;
                    if (m < M)
                        store4(m, (i32x4){acc[mt0 + h][0][r], acc[mt0 + h][1][r], acc[mt0 + h][2][r],
                                          acc[mt0 + h][3][r]});
                }
        };
        if (grp == 0) finish_pair(std::integral_constant<int, 0>{});
        else finish_pair(std::integral_constant<int, 2>{});
        return;
    }
    if (S == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + 16 * mt + 4 * gq + r;
                if (m < M) store4(m, (i32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]});
            }
        return;
    }
    // Split-K by partial tiles (int32, so the sum is exact in any order):
    // sep = 1, plain 16-byte stores summed by w4a8_split_reduce after the
    // kernel; sep = 0, exchanged through agent-scope atomics (device.hpp) and
    // summed by the tile's last split.
    uint32_t *const cnt = (uint32_t *)acc64 + (tn + gridDim.x * tm);
    uint64_t *const part = (uint64_t *)((char *)acc64 + split_counters_bytes((int64_t)gridDim.x * gridDim.y));
    const size_t slot = (size_t)M * N / 2;  // 64-bit words per split
    auto at = [&](int sp, int m) { return part + sp * slot + ((size_t)m * N + nc) / 2; };
    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + 16 * mt + 4 * gq + r;
                const i32x4 v = (i32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                if (m < M) {
                    if (sep) *(i32x4 *)at(split, m) = v;
                    else part_put(at(split, m), v);
                }
            }
    }
    if (sep || !split_tile_last_atomic(cnt, S) || !col_ok) return;
    // the last split sums the partials one row tile (4 of the lane's rows)
    // at a time, then clears them
    static_for<4>([&](auto bc) {
        constexpr int MT0 = decltype(bc)::value;
        auto row = [&](int r) { return m0 + wm * 64 + 16 * MT0 + 4 * gq + r; };
        auto addr = [&](int sp, int r) { return at(sp, row(r)); };
        auto valid = [&](int r) { return row(r) < M; };
        i32x4 v[4];
        part_sum<4, 1>(v, S, addr, valid);
        part_clear_all<4>(S, addr, valid);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (valid(r)) store4(row(r), v[r]);
    });
}

// The K splits' int32 partials ([S][M][N] after the tile counters) summed
// over the whole GPU, one thread per 4 consecutive outputs, with the GEMM's
// epilogue (the x16 of per-channel weights undone, y = acc s1 s2 rounded
// once, the optional acc_out), then cleared.  A tile's last split would
// otherwise move all S partial tiles through one CU at the rate it moves
// device-coherent data (about 50 GB/s).
template <bool GROUP, int DT>
__global__ __launch_bounds__(256) void w4a8_split_reduce(i32x4 *__restrict__ part, const float *__restrict__ s1,
                                                         const uint16_t *__restrict__ s2, uint16_t *__restrict__ y,
                                                         int32_t *__restrict__ acc_out, int N, int64_t quads, int S) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= quads) return;
    i32x4 *const p = part + q;
    i32x4 v = (i32x4){0, 0, 0, 0};
    constexpr int kB = 8;
    for (int s0 = 0; s0 < S; s0 += kB) {
        i32x4 b[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) b[i] = s0 + i < S ? p[(s0 + i) * quads] : (i32x4){0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < kB; ++i) v += b[i];
    }
    const int64_t m = 4 * q / N;
    const int nc = (int)(4 * q - m * N);
    const float s1m = s1[m];
    int32_t w[4];
    uint16_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        w[u] = GROUP ? v[u] : (v[u] >> 4);
        o[u] = f32_to_out_bits((float)w[u] * s1m * act_bits_to_f32<DT>(s2[nc + u]), DT);
    }
    *(u32x2 *)(y + 4 * q) = (u32x2){(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
    if (acc_out) *(i32x4 *)(acc_out + 4 * q) = (i32x4){w[0], w[1], w[2], w[3]};
    for (int s = 0; s < S; ++s) p[s * quads] = (i32x4){0, 0, 0, 0};
}

template <int NW, int KS, bool GROUP, int DT>
static hipError_t launch_lds8(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    const int sep = p.splits > 1;
    if (sep && (p.acc == nullptr || (a.M * a.N) % 4)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((w4a8_gemm_lds<NW, KS, GROUP, DT>), dim3(p.tiles_n, p.tiles_m, p.splits), dim3(64 * NW * KS),
                       0, st,
                       a.a8,
                       (const uint32_t *)a.b, a.s1, (const uint16_t *)a.s2, (const uint16_t *)a.s3,
                       (uint16_t *)a.y, a.acc_out, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits, sep);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !sep) return e;
    i32x4 *const part = (i32x4 *)((char *)p.acc + split_counters_bytes((int64_t)p.tiles_n * p.tiles_m));
    const int64_t quads = a.M * a.N / 4;
    hipLaunchKernelGGL((w4a8_split_reduce<GROUP, DT>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, part,
                       a.s1, (const uint16_t *)a.s2, (uint16_t *)a.y, a.acc_out, (int)a.N, quads, p.splits);
    return hipGetLastError();
}

template <int NW, int KS>
static hipError_t launch_lds8_nw(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    if (a.dtype == DT_BF16)
        return a.s3 != nullptr ? launch_lds8<NW, KS, true, DT_BF16>(a, p, st)
                               : launch_lds8<NW, KS, false, DT_BF16>(a, p, st);
    return a.s3 != nullptr ? launch_lds8<NW, KS, true, DT_F16>(a, p, st) : launch_lds8<NW, KS, false, DT_F16>(a, p, st);
}

// p.blk: workgroup tile width in 128-column units (1: 128 x 128, 2: 128 x 256);
// p.ksplit: groups of waves splitting K inside a workgroup (128 x 256 tiles
// without a K split only)
hipError_t launch_w4a8_gemm_lds(const W4A8Args &a, const W4A8Plan &p, hipStream_t st) {
    if (p.blk == 2 && p.ksplit == 2) {
        if (p.splits != 1) return hipErrorInvalidValue;
        return launch_lds8_nw<8, 2>(a, p, st);
    }
    return p.blk == 2 ? launch_lds8_nw<8, 1>(a, p, st) : launch_lds8_nw<4, 1>(a, p, st);
}

}  // namespace awq4
