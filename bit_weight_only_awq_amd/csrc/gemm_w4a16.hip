// gemm_w4a16.hip -- prefill GEMM for AWQ W4A16 on gfx950 (large M).
//
// Same method as w4a16.hip (vLLM pull request "Speed up AWQ 2.5x with updated
// kernel": first-generation AWQ packing and the context-phase GEMM; AutoAWQ
// pull request "Marlin symmetric quantization and inference": z = 8 when no
// zero points): Y = X . W with W[k,n] = (q - z) * s rounded once to the
// activation type, fp32 accumulation on the matrix cores.
//
// Workgroup tile 256 (M) x 128 (N), K in stages of 64 (two 32-k steps); 4
// waves side by side along N, each owning 256 x 32 outputs: 16 row tiles x 2
// column MFMAs of 16x16x32 per k-step.  A wave's 32 columns are 4 packed
// word-columns; the 4 lanes that share a word-column each take two adjacent
// columns of it, so every dequantised B operand feeds 16 MFMAs (about two
// VALU instructions per MFMA in the main loop, which the issue port hides).
//
// Data movement: every stage's X rows and packed words (with the stage's
// scales and zero points) are copied straight from global memory into LDS by
// direct-to-LDS buffer loads, with no register staging, into rings of AB X
// buffers (copied AB - 1 stages ahead) and BB word buffers (BB - 1 ahead).
// The launches use AB = 2, BB = 3 (two workgroups per CU; deeper word
// rings at one workgroup per CU measured slower, also below 128 rows, where
// the mid-size kernel or the two-group K split serves better).  Every stage
// issues the same copies (near the end the last stage is copied again into
// a buffer that is no longer read), so the wait that ends a stage has a fixed
// count: it waits only for what the next stage reads.  Each wave
// software-pipelines its k-steps: while the MFMAs of step q run, it
// dequantises the B operands of step q+1 and reads the X operands six row
// tiles ahead.  One wait and one barrier end each stage.
//
// MT = 16 row tiles per wave (256-row workgroup tiles) or 8 (128 rows, for
// M <= 128, where 256-row tiles would be half padding).
#include "device.hpp"
#include "launch.hpp"
#include "w4a16_ops.hpp"

namespace awq4 {

constexpr int GB_K = 64;
constexpr int GA_PITCH = GB_K * 2;  // 128 bytes per X row (8 segments of 16 B, swizzled)
constexpr int kPrefA = 6;           // X operand reads run this many row tiles ahead of the MFMAs

// LDS ring of one group of WN waves (side by side along N, 32 columns each):
// AB X buffers of 16*MT rows, BB buffers of packed words with the stage's
// scales and zero points
template <int MT, int AB, int BB, int WN>
struct GRing {
    static constexpr int N_TILE = 32 * WN;                // workgroup tile columns
    static constexpr int WC = N_TILE / 8;                 // word-columns per tile
    static constexpr int B_PITCH = WC * 4;                // bytes per k-row of packed words
    static constexpr int B_WORDS = GB_K * B_PITCH;
    static constexpr int M_SCALES = 2 * N_TILE * 2;       // scales of both k-steps
    static constexpr int M_ZEROS = 2 * WC * 4;            // zero words of both k-steps
    static constexpr int B_BYTES = B_WORDS + M_SCALES + M_ZEROS;  // 4736 (WN = 4), 9472 (WN = 8)
    static constexpr int B_ROWS = 1024 / B_PITCH;         // k-rows per 1 KB word copy (16 or 8)
    static constexpr int M_TILE = 16 * MT;                // workgroup tile rows
    static constexpr int A_BYTES = M_TILE * GA_PITCH;     // one X buffer
    // (16, 2, 3, 4): 79744, two workgroups per CU; (16, 2, 3, 8): 93952, one
    static constexpr int LDS = AB * A_BYTES + BB * B_BYTES;
    static constexpr int A_COPIES = M_TILE / (8 * WN);    // 8-row X copies per wave and stage
    static_assert(B_ROWS * WN == GB_K && A_COPIES * 8 * WN == M_TILE, "whole copies, one word copy per wave");
};

// X rows: 16-byte segment s of row r is stored at position s ^ (r & 7), so the
// 8 rows read by a lane octet cover all banks.
__device__ __forceinline__ int aseg(int r, int s) { return s ^ (r & 7); }
// Packed words: segment s (4 words) of k-row r is stored at s ^ ((r>>3)&3):
// one word read serves rows 8 apart (lane groups gq = 0..3), which then sit
// in four different 16-byte segments, i.e. on disjoint banks (a k-row has 4
// or 8 segments; the XOR stays inside them).
__device__ __forceinline__ int bseg(int r, int s) { return s ^ ((r >> 3) & 3); }

// Output columns of MFMA u relative to the lane's word-column (before + 2h).
__host__ __device__ constexpr int gemm_col(int u) { return (u & 1) + ((u >> 1) << 2); }

// WN = 4: 128-column tiles, two workgroups per CU; WN = 8: 256-column tiles
// (one workgroup of 8 waves per CU), which halve the X bytes copied per
// multiply-add.
// KS = 2 (WN = 4 only): the workgroup holds two groups of 4 waves that share
// the output tile and split its K range (each with its own LDS ring); the
// groups trade partial sums through LDS at the end.  This doubles the waves
// per SIMD for layers with no more tiles than CUs.
template <int DT, bool SYM, int KS, int MT, int AB, int BB, int WN>
__global__ __launch_bounds__(64 * WN * KS, WN == 8 ? 1 : KS == 2 ? 1 : MT == 8 ? 3 : 2) void w4a16_gemm(const uint16_t *__restrict__ x,
                                                                const uint32_t *__restrict__ qw,
                                                                const uint16_t *__restrict__ sc,
                                                                const uint32_t *__restrict__ qz,
                                                                uint16_t *__restrict__ y, uint64_t *__restrict__ acc64,
                                                                int M, int N, int K, int G, int S, int sep) {
    using R = GRing<MT, AB, BB, WN>;
    static_assert(KS == 1 || (WN == 4 && KS * R::LDS >= 2 * 4 * MT * 64 * 16), "the K-split handover fits in the rings");
    static_assert(AB >= 2 && BB >= 3 && MT > kPrefA, "ring depths and prefetch distance");
    constexpr int GB_M = R::M_TILE, GA_BYTES = R::A_BYTES, G_LDS = R::LDS;
    constexpr int GB_N = R::N_TILE, GB_PITCH = R::B_PITCH, GB_WORDS = R::B_WORDS, GM_SCALES = R::M_SCALES;
    constexpr int GB_BYTES = R::B_BYTES, WC = R::WC;
    __shared__ __attribute__((aligned(16))) unsigned char lds_all[KS * G_LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = KS == 1 ? 0 : wv / WN, wave = wv % WN;
    unsigned char *const lds = lds_all + grp * G_LDS;
    unsigned char *const Abase = lds;
    unsigned char *const Bbase = lds + AB * GA_BYTES;
    const int j = lane & 15, gq = lane >> 4;
    const int nw = N >> 3;
    // logical tile of this workgroup (XCD-aware order over the tiles_n x tiles_m grid)
    const int tile = tile_of_xcd_order(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
    const int tn = tile % gridDim.x, tm = tile / gridDim.x, split = blockIdx.z;
    const int m0 = tm * GB_M, wc0 = tn * WC;
    const int T = K / GB_K;
    // stages of this workgroup, then of this group: group 0 takes the first
    // ceil(n/2), group 1 the rest; both pass `iters` loop barriers (group 1
    // adds an idle one when n is odd), so their barriers pair up
    const int w_lo = (int)((int64_t)T * split / S), w_hi = (int)((int64_t)T * (split + 1) / S);
    const int iters = (w_hi - w_lo + KS - 1) / KS;
    const int s_lo = w_lo + grp * iters, s_hi = min(w_hi, s_lo + iters);

    // Copy assignment (byte offsets from the workgroup's corner; all fit in
    // 32 bits: at most 256 X rows and 64 k-rows of words are addressed).
    // X: wave w copies rows (GB_M/WN) w + 8i + lane/8 (i < A_COPIES), lane%8
    // being the stored segment position; rows past M repeat row M-1 (their
    // outputs are never stored).  Words: wave w copies k-rows B_ROWS w +
    // lane/(WC/4), lane%(WC/4) being the stored segment; word-columns past
    // the end repeat the last 4.
    const char *const xg = (const char *)(x + (size_t)m0 * K);
    const char *const wg = (const char *)(qw + wc0);
    // descriptors over the rest of X from row m0 and of the packed words from
    // word-column wc0 (the planner keeps both under 2^31 bytes)
    const __amdgpu_buffer_rsrc_t xrs = buf_rsrc(xg, (int64_t)(M - m0) * K * 2);
    const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(wg, (int64_t)K * nw * 4 - (int64_t)wc0 * 4);
    const int lg = __builtin_ctz(G);  // G is 32, 64 or 128
    uint32_t xoff[R::A_COPIES];
#pragma unroll
    for (int i = 0; i < R::A_COPIES; ++i) {
        const int r = (GB_M / WN) * wave + 8 * i + (lane >> 3);
        const int m = min(m0 + r, M - 1);
        xoff[i] = (uint32_t)(((m - m0) * K + 8 * aseg(r, lane & 7)) * 2);
    }
    uint32_t woff;
    {
        const int r = R::B_ROWS * wave + lane / (WC / 4);
        const int wc = min(wc0 + 4 * bseg(r, lane % (WC / 4)), nw - 4);
        woff = (uint32_t)((r * nw + wc - wc0) * 4);
    }
    // Metadata: 2 WC lanes copy 8 scales each (k-step lane/WC, word-column
    // wc0 + lane%WC), WC/2 lanes 4 zero words each (k-step l/(WC/4), word-
    // columns wc0 + 4 (l%(WC/4)) on), through descriptors over the scale and
    // zero-point arrays: the group of k-step 0 of the stage is a scalar offset,
    // the k-step's step past it (one group when G = 32) part of the lane's
    // fixed offset.  WN = 4: wave 0, lanes 0..31 and 32..39 (the zero copy's
    // LDS position follows from the lane number); WN = 8: wave 0 all lanes
    // (scales), wave 1 lanes 0..15 (zero points).
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(sc, (int64_t)(K / G) * N * 2);
    const __amdgpu_buffer_rsrc_t zrs = buf_rsrc(SYM ? (const void *)sc : (const void *)qz, SYM ? 0 : (int64_t)(K / G) * nw * 4);
    const bool zero_wave = WN == 8 ? wave == 1 : wave == 0;
    const int zl = WN == 8 ? lane : lane - 2 * WC;  // zero-copy lane number
    const bool scale_lane = wave == 0 && lane < 2 * WC;
    const bool zero_lane = !SYM && zero_wave && zl >= 0 && zl < WC / 2;
    uint32_t m_voff = 0;
    if (scale_lane) {
        const int meta_ks = lane / WC, meta_col = min(wc0 + lane % WC, nw - 1);
        m_voff = (uint32_t)((((32 * meta_ks) >> lg) * N + 8 * meta_col) * 2);
    } else if (zero_lane) {
        const int meta_ks = zl / (WC / 4), meta_col = min(wc0 + 4 * (zl % (WC / 4)), nw - 4);
        m_voff = (uint32_t)((((32 * meta_ks) >> lg) * nw + meta_col) * 4);
    }

    // copies of stage st into X buffer / word buffer `buf`
    auto copyA = [&](int st, int buf) {
        unsigned char *dst = Abase + buf * GA_BYTES + (GB_M / WN) * wave * GA_PITCH;
#pragma unroll
        for (int i = 0; i < R::A_COPIES; ++i)
            dma16_buf(xrs, xoff[i], (uint32_t)st * (GB_K * 2), dst + 8 * i * GA_PITCH);
    };
    auto copyB = [&](int st, int buf) {
        unsigned char *dst = Bbase + buf * GB_BYTES;
        dma16_buf(wrs, woff, (uint32_t)st * (GB_K * 4) * (uint32_t)nw, dst + R::B_ROWS * wave * GB_PITCH);
        const uint32_t g0 = (uint32_t)((st * GB_K) >> lg);
        if (scale_lane) dma16_buf(srs, m_voff, g0 * (uint32_t)N * 2, dst + GB_WORDS);
        else if (zero_lane) dma16_buf(zrs, m_voff, g0 * (uint32_t)nw * 4, dst + (WN == 8 ? GB_WORDS + GM_SCALES : GB_WORDS));
    };

    f32x4 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[mt][u] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Lane j takes columns 2*pi and 2*pi + 1 (pi = j % 4) of word-column
    // 4 * wave + j / 4: the first comes from pair_x, the second from pair_y,
    // both at nibble position pi (byte pi / 2 of each half, low or high
    // nibble).  The byte shift is folded into the per-lane v_perm selectors
    // (selector 0x0C gives a zero byte; the mask below drops that byte
    // anyway).
    const int c4 = j >> 2, pi = j & 3;
    const int hi = pi & 1;
    const uint32_t shift_sel = (pi & 2) ? 0x00010001u : 0u;
    const uint32_t selx = 0x0C040C00u + shift_sel, sely = 0x0C060C02u + shift_sel;
    const uint32_t nmask = hi ? 0x00F000F0u : 0x000F000Fu;
    const uint32_t mul2 = hi ? 0x2C002C00u : 0x3C003C00u;  // fp16 (1/16, 1/16) or (1, 1)
    const uint32_t zbase = hi ? 0xD400u : 0xE400u;         // -(64 + z) or -(1024 + z)
    const int zsh = hi ? 4 : 0;
    const int wcl = 4 * wave + c4;  // word-column within the workgroup tile
    const int wcol = wc0 + wcl;
    const bool col_ok = wcol < nw;
    uint32_t zc[2], sc2[2];
    float zf[2], sf[2];
    int gcur = -1;

    // dequantisation constants of this lane's 2 columns for k-step (st, ks)
    auto load_consts = [&](int st, int ks) {
        const int g = (st * GB_K + 32 * ks) >> lg;
        if (g == gcur) return;
        gcur = g;
        const unsigned char *Mt = Bbase + ((st - s_lo) % BB) * GB_BYTES + GB_WORDS;
        const uint32_t s2 = *(const uint32_t *)(Mt + ks * (GB_N * 2) + wcl * 16 + 4 * pi);
        const uint32_t zw = SYM ? 0x88888888u : *(const uint32_t *)(Mt + GM_SCALES + ks * (GB_N / 2) + wcl * 4);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t z = (zw >> (4 * pi + 16 * u)) & 0xFu;  // nibble of column 2 pi + u
            const uint32_t sb = (s2 >> (16 * u)) & 0xFFFFu;
            if (DT == DT_F16) {
                const uint32_t h = zbase | (z << zsh);
                zc[u] = h | (h << 16);
                sc2[u] = sb | (sb << 16);
            } else {
                const float sv = bf16_bits_to_f32(sb);
                sf[u] = hi ? sv * 0.0625f : sv;
                zf[u] = (float)z * sv;
            }
        }
    };
    // packed words of k-step (st, ks): 8 consecutive k-rows of this lane's word-column
    auto load_words = [&](int st, int ks, uint32_t (&w)[8]) {
        const unsigned char *B = Bbase + ((st - s_lo) % BB) * GB_BYTES;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r = 32 * ks + 8 * gq + e;
            w[e] = *(const uint32_t *)(B + r * GB_PITCH + bseg(r, wave) * 16 + c4 * 4);
        }
    };
    // B operand of MFMA u (4 registers = 8 k of one column) from paired words
    auto dequant = [&](const uint32_t (&pr)[4], int u) {
        u32x4 bop;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t v = pr[p];
            if (DT == DT_F16) {
                // exact (q - z): lo nibble h16 - (1024+z); hi nibble h16/16 - (64+z)
                const f16x2 q16 = bit_as<f16x2>((v & nmask) | 0x64006400u);
                const f16x2 d = q16 * bit_as<f16x2>(mul2) + bit_as<f16x2>(zc[u]);
                bop[p] = bit_as<uint32_t>(d * bit_as<f16x2>(sc2[u]));
            } else {
                const uint32_t m = v & nmask;
                const float w0 = __builtin_fmaf((float)(m & 0xFFu), sf[u], -zf[u]);
                const float w1 = __builtin_fmaf((float)((m >> 16) & 0xFFu), sf[u], -zf[u]);
                bop[p] = (uint32_t)bit_as<uint16_t>((__bf16)w0) | ((uint32_t)bit_as<uint16_t>((__bf16)w1) << 16);
            }
        }
        return bop;
    };
    auto pair_words = [&](const uint32_t (&w)[8], uint32_t (&px)[4], uint32_t (&py)[4]) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            px[p] = perm_b32(w[2 * p + 1], w[2 * p], selx);
            py[p] = perm_b32(w[2 * p + 1], w[2 * p], sely);
        }
    };
    auto load_a = [&](const unsigned char *A, int ks, int mt) {
        const int r = 16 * mt + j;
        return *(const u32x4 *)(A + r * GA_PITCH + aseg(r, 4 * ks + gq) * 16);
    };

    // Every wave issues its copies at the top of each stage (X AB - 1 and
    // words BB - 1 stages ahead).  (Measured alternatives, for 8 waves per
    // CU: a vector-memory instruction waiting to issue also holds up the
    // matrix-core issue of its SIMD, so the burst costs about 10 cycles per
    // 1 KB copy on the CU; copies spread between the matrix-core instructions
    // stalled them longer -- gate/up at M = 2048 1017 -> 915 TFLOP/s --
    // and copies issued by half the waves after their last matrix-core
    // instruction, with rings one stage deeper, gained nothing: the other
    // half cannot keep the matrix cores busy alone.)
    // Copies a stage leaves in flight at its end: those issued after the
    // latest copy the next stage reads -- X of st + 1, issued at st + 2 - AB,
    // or the words of st + 2 (read by its second k-step), issued at
    // st + 3 - BB; within a stage X is issued first.  The metadata waves
    // (wave 0; WN = 8 with zero points: waves 0 and 1) issue one more copy
    // per stage (wave 0 with WN = 4 and zero points: two).
    constexpr int kA = R::A_COPIES, kB0 = WN == 8 ? 2 : (SYM ? 2 : 3);
    const bool meta_wave = wave == 0 || (WN == 8 && !SYM && wave == 1);
    constexpr int kSa = 2 - AB, kSb = 3 - BB;            // issue stages relative to st
    constexpr int kFlight0 = kSa > kSb ? kB0 + (-kSa) * (kA + kB0) : (-kSb) * (kA + kB0);
    constexpr int kFlight1 = kSa > kSb ? 1 + (-kSa) * (kA + 1) : (-kSb) * (kA + 1);
    static_assert(kFlight0 < 64 && kFlight1 < 64, "vmcnt holds 6 bits");

    u32x4 bc[2];  // B operands of the current k-step
    if (s_lo < s_hi) {
#pragma unroll
        for (int d = 0; d < BB - 1; ++d) copyB(min(s_lo + d, s_hi - 1), d);
#pragma unroll
        for (int d = 0; d < AB - 1; ++d) copyA(min(s_lo + d, s_hi - 1), d);
    }
    wait_vm_all();
    __syncthreads();
    if (s_lo < s_hi) {
        uint32_t w[8], px[4], py[4];
        load_words(s_lo, 0, w);
        load_consts(s_lo, 0);
        pair_words(w, px, py);
        bc[0] = dequant(px, 0);
        bc[1] = dequant(py, 1);
    }
    for (int st = s_lo; st < s_hi; ++st) {
        const int rel = st - s_lo;
        const int ast = min(st + AB - 1, s_hi - 1), abuf = (rel + AB - 1) % AB;
        const int bst = min(st + BB - 1, s_hi - 1), bbuf = (rel + BB - 1) % BB;
        copyA(ast, abuf);
        copyB(bst, bbuf);
        const unsigned char *A = Abase + (rel % AB) * GA_BYTES;
        u32x4 a[MT];
#pragma unroll
        for (int mt = 0; mt < kPrefA; ++mt) a[mt] = load_a(A, 0, mt);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // the next k-step: (st, 1) or (st + 1, 0).  After the last stage
            // this dequantises stale (in-bounds) LDS data that is never used,
            // which keeps the loop body free of branches.
            const int nst = st + ks, nks = ks ^ 1;
            uint32_t w[8], px[4], py[4];
            u32x4 bn[2];
            load_words(nst, nks, w);
            load_consts(nst, nks);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
                for (int u = 0; u < 2; ++u) acc[mt][u] = mma<DT>(a[mt], bc[u], acc[mt][u]);
                // X operands kPrefA row tiles ahead (within this stage only)
                if (mt + kPrefA < MT) a[mt + kPrefA] = load_a(A, ks, mt + kPrefA);
                else if (ks == 0) a[mt + kPrefA - MT] = load_a(A, 1, mt + kPrefA - MT);
                if (mt == 1) pair_words(w, px, py);
                if (mt == 1 + MT / 4) bn[0] = dequant(px, 0);
                if (mt == 1 + MT / 2) bn[1] = dequant(py, 1);
                // keep each row tile's operand read where it is written: the
                // scheduler would otherwise sink the reads next to their
                // MFMAs and lose the prefetch distance
                __builtin_amdgcn_sched_barrier(0);
            }
            bc[0] = bn[0];
            bc[1] = bn[1];
        }
        if (meta_wave)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (kFlight0 & 15) | ((kFlight0 >> 4) << 14));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70 | (kFlight1 & 15) | ((kFlight1 >> 4) << 14));
        // no memory fence (it would wait for every copy); the clobber keeps
        // LDS accesses from moving across the barrier
        asm volatile("s_barrier" ::: "memory");
    }
    wait_vm_all();  // the copies re-issued near the end land before the LDS is reused

    // Epilogue: lane holds rows m0 + 16mt + 4gq + r and columns 8*wcol + 2pi
    // (MFMA 0) and 8*wcol + 2pi + 1 (MFMA 1).  Without a K split it writes the
    // output.  With one, each split stores its partial tile and the tile's
    // last split sums them in split order (split_tile_last_atomic: no cache
    // write-back fences, which cost more than the split saved).
    //
    // KS = 2: group 1's idle iteration (odd stage count), its barrier only;
    // then both groups hold partial sums of the whole tile.  Group 0 takes
    // row tiles 0..H-1 and group 1 row tiles H..MT-1 (H = MT/2): each parks
    // the other half in LDS (both rings are free once the last barrier has
    // passed) and adds the half parked by the other group to its own, as
    // group 0 + group 1.  res = the NTL row tiles this lane finishes, from
    // row tile lo.  (Picked by value, not by indexing the accumulators with
    // the group: such an index puts them in scratch.)
    constexpr int NTL = MT / KS;
    const int lo = KS == 1 ? 0 : grp * NTL;
    f32x4 res[NTL][2];
    if constexpr (KS == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int u = 0; u < 2; ++u) res[mt][u] = acc[mt][u];
    } else {
        for (int k = s_hi - s_lo; k < iters; ++k) __syncthreads();
        __syncthreads();  // every wave's copies have landed before the rings are reused
        f32x4 *xfer = (f32x4 *)lds_all + (size_t)wave * MT * 64 + lane;
        f32x4 *const mine = xfer + grp * 4 * MT * 64, *const theirs = xfer + (grp ^ 1) * 4 * MT * 64;
#pragma unroll
        for (int mt = 0; mt < NTL; ++mt)
#pragma unroll
            for (int u = 0; u < 2; ++u) mine[(mt * 2 + u) * 64] = grp == 0 ? acc[NTL + mt][u] : acc[mt][u];
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < NTL; ++mt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                res[mt][u] = theirs[(mt * 2 + u) * 64] + (grp == 0 ? acc[mt][u] : acc[NTL + mt][u]);
    }
    const int n0 = 8 * wcol + 2 * pi;
    uint32_t *const cnt = (uint32_t *)acc64 + (tn + gridDim.x * tm);
    if (S == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int i = 0; i < NTL; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * (lo + i) + 4 * gq + r;
                if (m < M)
                    *(uint32_t *)(y + (size_t)m * N + n0) = (uint32_t)f32_to_out_bits(res[i][0][r], DT) |
                                                            ((uint32_t)f32_to_out_bits(res[i][1][r], DT) << 16);
            }
        return;
    }
    // (256-column tiles never split K: the launcher refuses such a plan, and
    // the split path below would only add to their register count)
    if constexpr (WN == 8) {
        return;
    } else {
    // K split.  The partials move as column quads, 16 bytes each, with the
    // cache policy of agent-scope atomics (sc1: through to the device-wide
    // coherence point): lanes 2k and 2k+1 (pi even, odd) hold columns n0, n0+1
    // and n0+2, n0+3 of the same rows, and one swap between them (DPP) gives
    // the even lane rows 2h and the odd lane rows 2h+1 of all four columns.
    // Quad (i, h) of a lane: row m0 + 16 (LO + i) + 4 gq + 2h + odd, columns
    // qc .. qc+3.  Split s's partials are an [M, N] fp32 array after the tile
    // counters (under 2^31 bytes: the planner sees to it).
    const bool odd = pi & 1;
    const int qc = n0 - (odd ? 2 : 0);
    constexpr int NQ = 2 * NTL;
    // the last split keeps its own quads in registers where they fit beside
    // the loads (8 quads), else reads them back like the others
    constexpr bool kKeepOwn = NQ <= 8;
    // byte offset of quad q in an [M, N] fp32 array, and whether it is stored
    auto quad_at = [&](int q, bool &ok) {
        const int m = m0 + 16 * (lo + q / 2) + 4 * gq + 2 * (q % 2) + (odd ? 1 : 0);
        ok = col_ok && m < M;
        return ok ? ((uint32_t)m * (uint32_t)N + (uint32_t)qc) * 4u : 0u;
    };
    char *const part = (char *)acc64 + split_counters_bytes((int64_t)gridDim.x * gridDim.y);
    const uint32_t slot_bytes = (uint32_t)M * (uint32_t)N * 4u;
    auto split_rsrc = [&](int s) { return buf_rsrc(part + (size_t)s * slot_bytes, slot_bytes); };
    f32x4 own[kKeepOwn ? NQ : 1];
    // sep: the reduction kernel launched next adds the splits (plain stores,
    // made visible by the kernel boundary); else the tile's last split adds
    // them below.
    {
        const __amdgpu_buffer_rsrc_t rs = split_rsrc(split);
#pragma unroll
        for (int i = 0; i < NTL; ++i) {
            const f32x4 c0 = res[i][0], c1 = res[i][1];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float k0 = odd ? c0[2 * h + 1] : c0[2 * h], k1 = odd ? c1[2 * h + 1] : c1[2 * h];
                const float g0 = odd ? c0[2 * h] : c0[2 * h + 1], g1 = odd ? c1[2 * h] : c1[2 * h + 1];
                const float r0 = lane_pair_swap(g0), r1 = lane_pair_swap(g1);
                const f32x4 v = odd ? (f32x4){r0, r1, k0, k1} : (f32x4){k0, k1, r0, r1};
                bool ok;
                const uint32_t off = quad_at(2 * i + h, ok);
                if (ok) {
                    if (sep) __builtin_amdgcn_raw_buffer_store_b128(bit_as<u32x4>(v), rs, off, 0, 0);
                    else __builtin_amdgcn_raw_buffer_store_b128(bit_as<u32x4>(v), rs, off, 0, kPartCoherent);
                }
                if constexpr (kKeepOwn) own[2 * i + h] = v;
            }
        }
    }
    if (sep || !split_tile_last_atomic(cnt, S)) return;
    // The tile's last split: for 8 quads (four row tiles) at a time, the
    // splits' partials, kB splits per batch with every load of the batch in
    // flight before the first add (one memory round trip per batch), added in
    // split order (its own from registers where kept); then the output is
    // written and every partial of the tile cleared.
    constexpr int QC = NQ <= 8 ? NQ : 4;
    constexpr int kB = 4;
    static_assert(NQ % QC == 0, "whole quad chunks");
#pragma unroll
    for (int q0 = 0; q0 < NQ; q0 += QC) {
        bool ok[QC];
        uint32_t off[QC];
#pragma unroll
        for (int q = 0; q < QC; ++q) off[q] = quad_at(q0 + q, ok[q]);
        f32x4 sum[QC];
#pragma unroll
        for (int q = 0; q < QC; ++q) sum[q] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < S; s0 += kB) {
            u32x4 b[QC][kB];
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const int sp = s0 + i;
#pragma unroll
                for (int q = 0; q < QC; ++q) b[q][i] = (u32x4){0u, 0u, 0u, 0u};
                if (sp < S && !(kKeepOwn && sp == split)) {
                    const __amdgpu_buffer_rsrc_t rs = split_rsrc(sp);
#pragma unroll
                    for (int q = 0; q < QC; ++q)
                        if (ok[q]) b[q][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[q], 0, kPartCoherent);
                }
            }
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const int sp = s0 + i;
                if (sp >= S) break;
#pragma unroll
                for (int q = 0; q < QC; ++q) {
                    f32x4 add = bit_as<f32x4>(b[q][i]);
                    if constexpr (kKeepOwn) add = sp == split ? own[q0 + q] : add;
                    sum[q] += add;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < QC; ++q)
            if (ok[q]) *(uint2 *)((char *)y + off[q] / 2) = quad_out_bits<DT>(sum[q]);
        for (int sp = 0; sp < S; ++sp) {
            const __amdgpu_buffer_rsrc_t rs = split_rsrc(sp);
#pragma unroll
            for (int q = 0; q < QC; ++q)
                if (ok[q]) __builtin_amdgcn_raw_buffer_store_b128((u32x4){0u, 0u, 0u, 0u}, rs, off[q], 0, kPartCoherent);
        }
    }
    }
}

// K-split reduction of the W4A16 GEMM kernels (this one and the streaming
// kernel) where the partial tiles are large: y = the S fp32 partial [M, N]
// arrays added in split order from +0 and rounded once to the activation
// type -- the same sums as the in-kernel exchange -- and the partials then
// zeroed (the workspace is zero again after the call).  A launch of its own:
// the kernel boundary makes the partials visible to plain loads, and the
// reduction is spread over the whole GPU instead of the few CUs that finish
// the tiles, which move device-coherent data at about 50 GB/s each.  One
// thread per quad of 4 outputs; the loads of 8 splits in flight together.
template <int DT>
__global__ __launch_bounds__(256) void w4a16_split_reduce(f32x4 *__restrict__ part, uint16_t *__restrict__ y,
                                                          int64_t quads, int S) {
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
    *(uint2 *)(y + 4 * q) = quad_out_bits<DT>(v);
    for (int s = 0; s < S; ++s) p[s * quads] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_w4a16_split_reduce(const W4A16Args &a, const W4A16Plan &p, int64_t tiles, hipStream_t st) {
    if (p.acc == nullptr || p.splits < 2 || (a.M * a.N) % 4) return hipErrorInvalidValue;
    f32x4 *const part = (f32x4 *)((char *)p.acc + split_counters_bytes(tiles));
    const int64_t quads = a.M * a.N / 4;
    const dim3 grid((unsigned)((quads + 255) / 256));
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL(w4a16_split_reduce<DT_F16>, grid, dim3(256), 0, st, part, (uint16_t *)a.y, quads, p.splits);
    else
        hipLaunchKernelGGL(w4a16_split_reduce<DT_BF16>, grid, dim3(256), 0, st, part, (uint16_t *)a.y, quads, p.splits);
    return hipGetLastError();
}

template <int DT, bool SYM, int KS, int MT, int AB, int BB, int WN>
static hipError_t launch_gemm_t(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    dim3 grid(p.tiles_n, p.tiles_m, p.splits);
    const int sep = split_reduce_apart(p.splits, 16 * MT);
    hipLaunchKernelGGL((w4a16_gemm<DT, SYM, KS, MT, AB, BB, WN>), grid, dim3(64 * WN * KS), 0, st, (const uint16_t *)a.x,
                       (const uint32_t *)a.qweight, (const uint16_t *)a.scales, (const uint32_t *)a.qzeros,
                       (uint16_t *)a.y, p.acc, (int)a.M, (int)a.N, (int)a.K, a.G, p.splits, sep);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !sep) return e;
    return launch_w4a16_split_reduce(a, p, (int64_t)p.tiles_n * p.tiles_m, st);
}

template <int KS, int MT, int AB, int BB, int WN>
static hipError_t launch_gemm_ks(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    const bool sym = a.qzeros == nullptr;
    if (a.dtype == DT_F16)
        return sym ? launch_gemm_t<DT_F16, true, KS, MT, AB, BB, WN>(a, p, st)
                   : launch_gemm_t<DT_F16, false, KS, MT, AB, BB, WN>(a, p, st);
    return sym ? launch_gemm_t<DT_BF16, true, KS, MT, AB, BB, WN>(a, p, st)
               : launch_gemm_t<DT_BF16, false, KS, MT, AB, BB, WN>(a, p, st);
}

// 256-row (p.mt = 16) or 128-row (p.mt = 8) tiles, 128 columns wide
// (p.wn = 4) or, for 256-row tiles without a K-split group, 256 (p.wn = 8);
// rings of 2 X and 3 word buffers
hipError_t launch_w4a16_gemm(const W4A16Args &a, const W4A16Plan &p, hipStream_t st) {
    // a K split reduces through the workspace
    if (p.splits > 1 && p.acc == nullptr) return hipErrorInvalidValue;
    if (p.wn == 8) {
        if (p.mt != 16 || p.ksplit != 1 || p.splits != 1) return hipErrorInvalidValue;
        return launch_gemm_ks<1, 16, 2, 3, 8>(a, p, st);
    }
    if (p.mt == 8) return p.ksplit == 2 ? launch_gemm_ks<2, 8, 2, 3, 4>(a, p, st) : launch_gemm_ks<1, 8, 2, 3, 4>(a, p, st);
    return p.ksplit == 2 ? launch_gemm_ks<2, 16, 2, 3, 4>(a, p, st) : launch_gemm_ks<1, 16, 2, 3, 4>(a, p, st);
}

}  // namespace awq4
