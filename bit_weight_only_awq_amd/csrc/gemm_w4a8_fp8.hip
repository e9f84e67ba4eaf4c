// gemm_w4a8_fp8.hip -- INT4-FP8 W4A8 GEMM for large M on gfx950 (fp8 matrix cores).
//
// Method and operand codes as in w4a8_fp8.hip (the INT4-FP8 reading of the QQQ
// pull request "Support W4A8 quantization for vllm": E4M3 activation codes per
// token, symmetric int4 weights given to the matrix cores as the offset-binary
// codes u = q + 8, i.e. the E4M3 values u * 2^-9, and the epilogue
// sum a q = 2^9 * sum(a u 2^-9) - 8 * sum_k a).
//
// The pipeline is that of the int8 LDS GEMM (gemm_w4a8.hip) with 128-k
// stages, one 16x16x128 fp8 matrix-core step: 128 x 256 workgroup tiles of 8
// waves (2 x 4 wave tiles of 64 x 64: 4 row tiles x 4 column MFMAs); the
// activation codes (128 bytes of each row a stage) and the packed words (16
// K8 word rows) are copied straight into a 4-slot LDS ring three stages
// ahead; each stage waits only for the copies older than its own, and the
// next stage's operands are read while the current stage's MFMAs run, each
// read in a pinned slot.
#include "device.hpp"
#include "fp8_ops.hpp"
#include "launch.hpp"

namespace awq4 {

constexpr int F8_M = 128, F8_N = 256, F8_K = 128, F8_NW = 8;
constexpr int F8_RING = 4;                       // stages per ring (copied F8_RING - 1 ahead)
constexpr int F8_ABYTES = F8_M * F8_K;           // 16384: 128 rows x 128 codes
constexpr int F8_WROWS = F8_K / 8;               // 16 K8 word rows a stage
constexpr int F8_BBYTES = F8_WROWS * F8_N * 4;   // 16384
constexpr int F8_OFF_B = F8_RING * F8_ABYTES;
constexpr int F8_LDS = F8_OFF_B + F8_RING * F8_BBYTES;  // 131072
constexpr int F8_COPIES = 4;                     // 1 KB copies per wave and stage (2 code, 2 word)

// Activation rows: 16-byte segment s of row r is stored at position
// s ^ f8swz(r).  An operand read takes one segment of 16 rows (a row per
// lane); f8swz puts those rows on 16 distinct 16-byte bank groups of a
// 256-byte bank line, and any 8 consecutive rows on 8 distinct groups of a
// 128-byte line.
__device__ __forceinline__ int f8swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int DT>
__global__ __launch_bounds__(64 * F8_NW, 1) void w4a8_fp8_gemm_lds(const uint8_t *__restrict__ a,
                                                                  const uint32_t *__restrict__ bq,
                                                                  const float *__restrict__ s1,
                                                                  const float *__restrict__ asum,
                                                                  const uint16_t *__restrict__ s2,
                                                                  uint16_t *__restrict__ y,
                                                                  float *__restrict__ acc_out,
                                                                  uint64_t *__restrict__ ws, int M, int N, int K,
                                                                  int S, int sep) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[F8_LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int j = lane & 15, gq = lane >> 4;
    const int wm = wave / 4, wn = wave % 4;
    const int tile = tile_of_xcd_order(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int tn = tile % gridDim.x, tm = tile / gridDim.x, split = blockIdx.z;
    const int m0 = tm * F8_M, n0 = tn * F8_N;
    const int Tst = K / F8_K;
    const int s_lo = (int)((int64_t)Tst * split / S), s_hi = (int)((int64_t)Tst * (split + 1) / S);

    // Copy assignment.  Codes: copy i of wave w takes rows 8 (2w + i) + lane/8
    // (one 1 KB block of 8 rows), lane%8 being the stored segment position;
    // rows past M repeat row M-1 (their outputs are never stored).  Words:
    // copy i of wave w takes word row 2w + i, lane giving 4 columns; columns
    // past N repeat the last 4.
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 8 * (2 * wave + i) + (lane >> 3);
        const int m = min(m0 + r, M - 1);
        aoff[i] = (uint32_t)((m - m0) * K + 16 * ((lane & 7) ^ f8swz(r)));
    }
    uint32_t boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 2 * wave + i;
        const int c = min(n0 + 4 * lane, N - 4);
        boff[i] = (uint32_t)((r * N + c) * 4);
    }
    // buffer descriptors (the planner keeps every byte offset under 2^31):
    // the code rows from m0 and the packed words; the stage's offset as a scalar
    const __amdgpu_buffer_rsrc_t ars = buf_rsrc(a + (size_t)m0 * K, (int64_t)(M - m0) * K);
    const __amdgpu_buffer_rsrc_t brs = buf_rsrc(bq, (int64_t)(K / 8) * N * 4);

    auto copy_stage = [&](int st, int slot) {
        unsigned char *A = lds + slot * F8_ABYTES + 2 * wave * 1024;
#pragma unroll
        for (int i = 0; i < 2; ++i) dma16_buf(ars, aoff[i], (uint32_t)(st * F8_K), A + i * 1024);
        unsigned char *B = lds + F8_OFF_B + slot * F8_BBYTES + 2 * wave * (F8_N * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16_buf(brs, boff[i], (uint32_t)st * F8_WROWS * (uint32_t)N * 4, B + i * (F8_N * 4));
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[mt][u] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // lane (j, gq): row tile mt of the wave reads row 64 wm + 16 mt + j,
    // k 32 gq .. 32 gq + 31 (segments 2 gq and 2 gq + 1); columns
    // cl .. cl + 3 of word rows 4 gq .. 4 gq + 3
    const int cl = 64 * wn + 4 * j;
    auto a_addr = [&](int slot, int mt, int h) {
        const int r = 64 * wm + 16 * mt + j;
        return lds + slot * F8_ABYTES + r * F8_K + 16 * ((2 * gq + h) ^ f8swz(r));
    };
    const uint32_t w_off = (uint32_t)(F8_OFF_B + (4 * gq) * (F8_N * 4) + cl * 4);
    auto load_a = [&](int slot, int mt) {
        const u32x4 lo = *(const u32x4 *)a_addr(slot, mt, 0), hi = *(const u32x4 *)a_addr(slot, mt, 1);
        return (i32x8){(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                       (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
    };
    auto word_row = [&](int slot, int e) {
        return *(const u32x4 *)__builtin_assume_aligned(lds + slot * F8_BBYTES + w_off + e * (F8_N * 4), 16);
    };

    // operands of the stage in registers
    struct Ops {
        i32x8 a[4];
        i32x8 b[4];
    };
    auto load_ops = [&](int slot, Ops &o) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o.a[mt] = load_a(slot, mt);
        u32x4 w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = word_row(slot, e);
#pragma unroll
        for (int u = 0; u < 4; ++u) o.b[u] = fp8_b_operand(w[0][u], w[1][u], w[2][u], w[3][u]);
    };
    // Stage st (its operands in `o`): 16 MFMAs, each in its own slot.  Stage
    // st + 1's word rows are read in the first slots; each of its code
    // operands right after the MFMA that last uses stage st's (slots 3, 7,
    // 11, 15), and each B operand is built in place after its last use (slots
    // 12..15).  Then wait for the copies older than this stage's and cross
    // the barrier.  Copies: stage st + 3 into the slot of stage st - 1
    // (finished before the last barrier); near the end the last stage is
    // copied again into that slot, never read as data, so every stage issues
    // the same copies and the wait count is fixed.
    auto stage = [&](int st, Ops &o) {
        const unsigned rel = (unsigned)(st - s_lo);
        copy_stage(min(st + F8_RING - 1, s_hi - 1), (int)((rel + F8_RING - 1) % F8_RING));
        const int nslot = (int)((rel + 1) % F8_RING);
        u32x4 w[4];
        static_for<16>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int mt = i >> 2, u = i & 3;
            acc[mt][u] = mfma_fp8(o.a[mt], o.b[u], acc[mt][u]);
            if constexpr (i >= 1 && i <= 4) w[i - 1] = word_row(nslot, i - 1);
            if constexpr (u == 3) o.a[mt] = load_a(nslot, mt);
            if constexpr (mt == 3) o.b[u] = fp8_b_operand(w[0][u], w[1][u], w[2][u], w[3][u]);
            __builtin_amdgcn_sched_barrier(0);
        });
        // copies still allowed in flight: those of stage st + 3
        constexpr int kInFlight = (F8_RING - 3) * F8_COPIES;
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kInFlight & 15) | ((kInFlight >> 4) << 14));
        // no memory fence (it would wait for every copy); the clobber keeps
        // LDS accesses from moving across the barrier
        asm volatile("s_barrier" ::: "memory");
    };

    {
        Ops o;
        if (s_lo < s_hi) {
#pragma unroll
            for (int d = 0; d < F8_RING - 1; ++d)
                if (s_lo + d < s_hi) copy_stage(s_lo + d, d);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (s_lo < s_hi) load_ops(0, o);
        for (int st = s_lo; st < s_hi; ++st) stage(st, o);
    }

    // Epilogue: lane holds rows m0 + 64 wm + 16 mt + 4 gq + r, columns
    // n0 + cl + u (u = 0..3, adjacent).
    const int nc = n0 + cl;
    const bool col_ok = nc < N;
    auto store4 = [&](int m, f32x4 t) {
        const float s1m = s1[m], am = -8.0f * asum[m];
        float d[4];
        uint16_t o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            d[u] = __builtin_fmaf(512.0f, t[u], am);  // sum a q, one rounding
            o[u] = f32_to_out_bits(d[u] * s1m * act_bits_to_f32<DT>(s2[nc + u]), DT);
        }
        *(u32x2 *)(y + (size_t)m * N + nc) = (u32x2){(uint32_t)o[0] | ((uint32_t)o[1] << 16),
                                                     (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
        if (acc_out) *(f32x4 *)(acc_out + (size_t)m * N + nc) = (f32x4){d[0], d[1], d[2], d[3]};
    };
    if (S == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + 16 * mt + 4 * gq + r;
                if (m < M) store4(m, (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]});
            }
        return;
    }
    // Split-K by fp32 partial tiles, summed in split order: sep = 1, plain
    // 16-byte stores summed by w4a8_fp8_split_reduce after the kernel;
    // sep = 0, exchanged through agent-scope atomics (device.hpp) and summed
    // by the tile's last split.
    uint32_t *const cnt = (uint32_t *)ws + (tn + gridDim.x * tm);
    uint64_t *const part = (uint64_t *)((char *)ws + split_counters_bytes((int64_t)gridDim.x * gridDim.y));
    const size_t slot = (size_t)M * N / 2;  // 64-bit words per split
    auto at = [&](int sp, int m) { return part + sp * slot + ((size_t)m * N + nc) / 2; };
    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 64 + 16 * mt + 4 * gq + r;
                const f32x4 v = (f32x4){acc[mt][0][r], acc[mt][1][r], acc[mt][2][r], acc[mt][3][r]};
                if (m < M) {
                    if (sep) *(f32x4 *)at(split, m) = v;
                    else part_put(at(split, m), v);
                }
            }
    }
    if (sep || !split_tile_last_atomic(cnt, S) || !col_ok) return;
    static_for<4>([&](auto bc) {
        constexpr int MT0 = decltype(bc)::value;
        auto row = [&](int r) { return m0 + wm * 64 + 16 * MT0 + 4 * gq + r; };
        auto addr = [&](int sp, int r) { return at(sp, row(r)); };
        auto valid = [&](int r) { return row(r) < M; };
        f32x4 v[4];
        part_sum<4, 2>(v, S, addr, valid);
        part_clear_all<4>(S, addr, valid);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (valid(r)) store4(row(r), v[r]);
    });
}

// The K splits' fp32 partials ([S][M][N] after the tile counters) summed in
// split order over the whole GPU, one thread per 4 consecutive outputs, with
// the GEMM's epilogue (sum a q = 512 t - 8 sum_k a, one rounding; y = that
// s1 s2 rounded once; the optional acc_out), then cleared.  The same sums as
// a tile's last split would form, without moving every partial through one
// CU at the rate it moves device-coherent data (about 50 GB/s).
template <int DT>
__global__ __launch_bounds__(256) void w4a8_fp8_split_reduce(f32x4 *__restrict__ part, const float *__restrict__ s1,
                                                             const float *__restrict__ asum,
                                                             const uint16_t *__restrict__ s2, uint16_t *__restrict__ y,
                                                             float *__restrict__ acc_out, int N, int64_t quads, int S) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= quads) return;
    f32x4 *const p = part + q;
    f32x4 v = (f32x4){0.f, 0.f, 0.f, 0.f};
    constexpr int kB = 8;
    for (int s0 = 0; s0 < S; s0 += kB) {
        f32x4 b[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) b[i] = s0 + i < S ? p[(s0 + i) * quads] : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kB; ++i)
            if (s0 + i < S) v += b[i];
    }
    const int64_t m = 4 * q / N;
    const int nc = (int)(4 * q - m * N);
    const float s1m = s1[m], am = -8.0f * asum[m];
    float d[4];
    uint16_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        d[u] = __builtin_fmaf(512.0f, v[u], am);
        o[u] = f32_to_out_bits(d[u] * s1m * act_bits_to_f32<DT>(s2[nc + u]), DT);
    }
    *(u32x2 *)(y + 4 * q) = (u32x2){(uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16)};
    if (acc_out) *(f32x4 *)(acc_out + 4 * q) = (f32x4){d[0], d[1], d[2], d[3]};
    for (int s = 0; s < S; ++s) p[s * quads] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

template <int DT>
static hipError_t launch_fp8_lds_t(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st) {
    const int sep = p.splits > 1;
    if (sep && (p.acc == nullptr || (g.M * g.N) % 4)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((w4a8_fp8_gemm_lds<DT>), dim3(p.tiles_n, p.tiles_m, p.splits), dim3(64 * F8_NW), 0, st, g.a,
                       (const uint32_t *)g.b, g.s1, g.asum, (const uint16_t *)g.s2, (uint16_t *)g.y, g.acc_out, p.acc,
                       (int)g.M, (int)g.N, (int)g.K, p.splits, sep);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !sep) return e;
    f32x4 *const part = (f32x4 *)((char *)p.acc + split_counters_bytes((int64_t)p.tiles_n * p.tiles_m));
    const int64_t quads = g.M * g.N / 4;
    hipLaunchKernelGGL((w4a8_fp8_split_reduce<DT>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, part,
                       g.s1, g.asum, (const uint16_t *)g.s2, (uint16_t *)g.y, g.acc_out, (int)g.N, quads, p.splits);
    return hipGetLastError();
}

hipError_t launch_w4a8_fp8_lds(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st) {
    return g.dtype == DT_BF16 ? launch_fp8_lds_t<DT_BF16>(g, p, st) : launch_fp8_lds_t<DT_F16>(g, p, st);
}

}  // namespace awq4
