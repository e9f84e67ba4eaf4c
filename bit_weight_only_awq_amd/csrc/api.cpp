// api.cpp -- the extern "C" entry points declared in include/awq4.h.
//
// Every entry point validates its arguments with pure host code first (no HIP
// call, so validation works without a GPU and a rejected call writes
// nothing), then plans the launch as a pure function of the shape, and only
// then enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/awq4.h"
#include "launch.hpp"

namespace awq4 {

static constexpr int64_t kMaxDim = int64_t(1) << 20;
// The planners below size grids from the device's compute-unit count (cus):
// two workgroups of 4 waves per CU is the target fill of the tiled kernels.
static int64_t target_workgroups(const DeviceProps &d) { return 2 * (int64_t)d.cus; }

// K splits of the skinny W4A8 kernels (counting atomics, M <= 64): every
// split adds one atomic per output element, all S of an element landing on
// one address at about the same time, so their cost grows faster than S * M *
// N, while long K needs the splits to spread its stream.  The split count
// that fills the CUs (s) is capped at 2^20 sqrt(K / 4096) / (M N), rounded
// down.  Measured (int8 GEMM, rotated weights): 4096 x 14336 at M = 64, 3
// splits 42.5 us, 2 28.5, 1 21.4 (INT4-FP8 39.3 -> 18.4 with 1); at M = 32
// 19.1 / 18.0 / 16.7; 4096 x 4096 at M = 64, 8 splits 22.5, 4 20.7; the QQQ
// shape (K = 21760) best at the 4 to 8 that fill the CUs.
static int64_t skinny_splits(int64_t s, int64_t M, int64_t N, int64_t K) {
    const double cap = 1048576.0 * std::sqrt((double)K / 4096.0) / ((double)M * (double)N);
    return std::max<int64_t>(1, std::min<int64_t>(s, (int64_t)cap));
}
// The W4A8 LDS GEMMs take M above 64, and M above 32 where the skinny
// kernel's plan (p, made first) splits K.
static bool lds_rows(int64_t M, const W4A8Plan &p) { return M > 64 || (M > 32 && p.kind == 0 && p.splits > 1); }
// The W4A16 LDS GEMM takes M above 64 (the decode kernel takes M <= 8, the
// streaming kernel 8 < M <= 64).
static constexpr int64_t kW16LdsMinM = 64;
// Largest W4A8 K: the kernels multiply int8 activations (down to -128) by
// int8 weight bytes 16 q (down to -128), so |acc| <= 2^14 K must stay below
// 2^31: K < 2^17, and K % 64 == 0 makes that K <= 131008.
static constexpr int64_t kW8MaxK = 131072 - 64;

// Once-per-device property cache.  The first call on a device asks HIP for
// its compute-unit count; later calls read the cached value (lock-free: a
// racing first call stores the same number).  With no device visible (the
// validation-only case) the planners assume a whole MI355X.
static constexpr int kMaxDevices = 64;
static std::atomic<int> g_device_cus[kMaxDevices];

static DeviceProps props_of_device(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return DeviceProps{kDefaultCUs};
    int cus = g_device_cus[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = kDefaultCUs;
        g_device_cus[dev].store(v, std::memory_order_relaxed);
        cus = v;
    }
    return DeviceProps{cus};
}

// the device that `stream` belongs to (the current device for the null
// stream), or -1 when none can be found
static int stream_device(void *stream) {
    int dev = -1;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &d) == hipSuccess) dev = (int)d;
    }
    if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return -1;
    return dev;
}

// properties of the device that `stream` belongs to
static DeviceProps stream_props(void *stream) {
    const int dev = stream_device(stream);
    return dev < 0 ? DeviceProps{kDefaultCUs} : props_of_device(dev);
}

// ---------------------------------------------------------------------------
// Static split-K scratch of the no-allocation decode entry point
// (awq_gemv_w4a16_static).  Each device that loads the library holds its own
// copy until the process ends.  In host code `scratch` only names the array:
// its device address comes from hipGetSymbolAddress, taken once per device
// with that device current and kept in g_scratch; kernels and clears use that
// address, never the name.
constexpr size_t kScratchBytes = AWQ_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
    std::atomic<void *> ptr{nullptr};
    std::atomic<int> cleared{0};  // a clear has been enqueued outside graph capture
};
static ScratchSlot g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// fills n 16-byte words with zero (a kernel rather than a memset, so that a
// clear recorded into a graph replays correctly)
__global__ void scratch_zero(uint4 *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

static int scratch_of_device(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return AWQ_EHIP;
    void *p = g_scratch[dev].ptr.load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].ptr.load(std::memory_order_acquire);
        if (!p) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess) return AWQ_EHIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess) return AWQ_EHIP;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev) (void)hipSetDevice(cur);
            if (e != hipSuccess || !p) return AWQ_EHIP;
            g_scratch[dev].ptr.store(p, std::memory_order_release);
        }
    }
    *out = p;
    return AWQ_OK;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

W4A16Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int G, int split_k, int dtype, const DeviceProps &d) {
    const int64_t cus = d.cus;
    // workgroups of the CS <= 2 decode kernel resident at once (4 per CU)
    const int64_t decode_resident_wgs = 4 * cus, decode_small_chunk_wgs = 2 * cus;
    W4A16Plan p{};
    const int64_t nw = N / 8;
    const int64_t T = K / 32;
    int64_t tiles;
    if (M <= 8) {
        // decode kernel: one 32*cs-wide K chunk per wave, 4 chunks per
        // workgroup; the K split is fixed by the chunking (split_k is ignored)
        p.kind = 0;
        p.blk = nw % 2 == 0 ? 2 : 1;  // 128 B per k-row per wave: whole cache lines
        p.cs = G >= 64 ? 2 : 1;
        p.waves = 4;
        p.tiles_n = (int)cdiv(nw, 16 * p.blk);
        // 32-k chunks when that still gives at most two workgroups per CU:
        // twice the waves per SIMD on narrow layers (measured at M = 1 on
        // 4096 x 4096: 5.14 -> 4.88 us; layers past that bound were slower,
        // and each extra split adds an atomic per output element and row)
        if (M <= 2 && (int64_t)p.tiles_n * cdiv(K / 32, p.waves) <= decode_small_chunk_wgs) p.cs = 1;
        // M >= 4: one 128-k group per wave when that still gives three
        // quarters of the CUs a workgroup -- half the K splits, so half the
        // per-element atomics, which grow with M (measured at M = 16: down
        // 11008 x 4096 35.2 -> 21.0 us, qkv 4096 x 6144 16.2 -> 14.7 us;
        // 4096 x 4096, with 128 such workgroups, was slower)
        if (M >= 4 && G % 128 == 0 && (int64_t)p.tiles_n * cdiv(K / 128, p.waves) >= 3 * cus / 4) p.cs = 4;
        p.tiles_m = 1;
        p.splits = (int)cdiv(K / (32 * p.cs), p.waves);
        // more workgroups than stay resident (4 per CU): one 128-k group per
        // wave instead, so that the layer still runs in a single round
        if (G % 128 == 0 && (int64_t)p.tiles_n * p.splits > decode_resident_wgs) {
            p.cs = 4;
            p.splits = (int)cdiv(K / 128, p.waves);
        }
        // bf16 reduces its splits through per-tile fp32 partials (several
        // memory round trips per workgroup, against one for the fp16
        // counting atomics), so at M <= 2 it takes the fewest splits: one
        // 128-k group per wave, or with smaller groups 8-wave workgroups of
        // group-sized chunks.  Measured at M = 1: Llama-2-7B o 12.0 -> 8.2
        // us, down 16.3 -> 12.4, qkv 11.4 -> 11.1, gate/up level (g128);
        // 4096 x 4096 and 11008 x 4096 12.0 -> 8.4 and 16.5 -> 12.5 us (g64),
        // 12.0 -> 9.4 and 25.8 -> 17.1 us (g32), even where the grid then
        // takes two rounds
        if (dtype == AWQ_DTYPE_BF16 && M <= 2) {
            if (G % 128 == 0) {
                p.cs = 4;
            } else {
                p.waves = 8;
                p.cs = G >= 64 ? 2 : 1;
            }
            p.splits = (int)cdiv(K / (32 * p.cs), p.waves);
        }
        // M >= 4: workgroups of 8 waves (chunks chosen by the same rules)
        // wherever their grid still runs in one round (two per CU, one at
        // CS = 4): half the K splits, so half the per-element atomics.
        // Measured on the Llama-2-7B layers: M = 8 qkv 14.9 -> 12.7 us, o
        // 10.9 -> 8.9, down 14.5 -> 12.9; M = 4 qkv 12.0 -> 10.3, o 8.2 ->
        // 7.4, down 11.7 -> 10.7; slower at M = 1 (qkv 8.4 -> 9.3) and where
        // the grid takes two rounds (gate/up at M = 4: 15.1 -> 18.4)
        if (M >= 4) {
            int cs8 = G >= 64 ? 2 : 1;
            if (G % 128 == 0 && (int64_t)p.tiles_n * cdiv(K / 128, 8) >= 3 * cus / 4) cs8 = 4;
            const int64_t splits8 = cdiv(K / (32 * cs8), 8);
            if ((int64_t)p.tiles_n * splits8 <= (cs8 >= 4 ? 1 : 2) * cus) {
                p.waves = 8;
                p.cs = cs8;
                p.splits = (int)splits8;
            }
        }
        tiles = p.tiles_n;
    }
    if (M > 8 || p.splits > kMaxSplitK) {
        p.kind = 1;
        p.blk = 1;
        p.cs = 1;
        p.mt = M >= 128 ? 4 : (M >= 64 ? 2 : 1);
        const int64_t bm = 32 * p.mt;
        p.tiles_n = (int)cdiv(N, 256);
        p.tiles_m = (int)cdiv(M, bm);
        tiles = (int64_t)p.tiles_n * p.tiles_m;
        int64_t s = 1;
        if (tiles < cus) {
            // at most 4 K splits: each adds an M x N partial tile to write,
            // read and clear, which costs more than it saves beyond that
            // (measured on the Llama-3-8B layers at M = 64)
            s = cdiv(target_workgroups(d), tiles);
            s = std::min<int64_t>(s, std::max<int64_t>(1, T / 2));
            s = std::min<int64_t>(s, 4);
        }
        p.splits = (int)std::max<int64_t>(1, s);
        if (split_k > 0) p.splits = (int)std::min<int64_t>(split_k, T);
        p.splits = (int)std::min<int64_t>(p.splits, kMaxSplitK);
    }
    // 8 < M <= 64: the streaming kernel (measured against the decode kernel
    // at M = 8 and 16 on the Llama-2-7B layers: level at 8, 1.3-1.6x faster at
    // 16, where the decode kernel's per-element atomics dominate).
    // The K split S trades the per-CU stream (weights plus the X rows every
    // column tile reads again, divided over S workgroups; a CU sustains about
    // 25 GB/s with all CUs busy) against the partial tiles the last workgroup
    // of a column tile sums (S x rows x 128 fp32 at about 40 GB/s): the S
    // in [1, CUs / tiles] (every workgroup resident at once, every wave with a
    // chunk) with the least estimated time.
    // (Its split partials are addressed as one buffer of M x N floats per
    // split, hence M x N x 4 under 2^31 bytes.)
    if (M > 8 && M <= 64 && M * N * 4 < (int64_t(1) << 31)) {
        const int cs = G >= 64 ? 2 : 1;
        const int mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
        const int wv = kStreamWaves(mt);
        const int64_t tiles_n = cdiv(N, 128);
        const int64_t chunks = K / (32 * cs);
        const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(cus / tiles_n, chunks / wv));
        const double rows = 16.0 * mt;
        const double stream_bytes = (double)K * (64 + 2 * rows), tail_bytes = rows * 128 * 4;
        int64_t s = 1;
        double best = 0;
        for (int64_t c = 1; c <= smax; ++c) {
            const double t = stream_bytes / c / 25.0 + c * tail_bytes / 40.0;
            if (c == 1 || t < best) best = t, s = c;
        }
        if (split_k > 0) s = std::min<int64_t>(split_k, chunks);
        p.kind = 5;
        p.blk = 1;
        p.cs = cs;
        p.waves = wv;
        p.mt = mt;
        p.ksplit = 1;
        p.tiles_n = (int)tiles_n;
        p.tiles_m = 1;
        p.splits = (int)std::min<int64_t>(s, kMaxSplitK);
        p.workspace_bytes = p.splits > 1 ? (size_t)split_tiles_bytes(p.tiles_n, p.splits, M, N) : 0;
        return p;
    }
    // buffer-descriptor copies address X and the packed words with 32-bit offsets
    const bool fits_rsrc = M * K * 2 < (int64_t(1) << 31) && K * (N / 2) < (int64_t(1) << 31);
    if (M > kW16LdsMinM && K % 64 == 0 && N % 32 == 0 && fits_rsrc) {
        // LDS-pipelined GEMM: 256- or 128-row x 128 workgroup tiles, K in
        // stages of 64
        p.kind = 3;
        // (below 128 rows: the 128-row tiles with two wave groups splitting
        // K; copy rings 8 word slots deep at one workgroup per CU measured
        // slower on every Llama-3-8B layer -- M = 64: gate/up 69.3 vs
        // 45.6 us, down 83.7 vs 61.8; M = 96: qkv 55.3 vs 36.6, o 40.5 vs 30.5)
        // 128-row tiles at M <= 128 (256-row ones would be half padding) and
        // where there would be at most 128 tiles of 256 rows (half the CUs
        // idle).  Measured on the Llama-3-8B layers at M = 128..2048: o at
        // M = 256, 56 -> 37 us; down at M = 128, 90 -> 57 us; with more
        // 256-row tiles than that (qkv at M = 1024, gate/up at M = 256) the
        // 256-row tiles' better operand reuse wins.
        p.mt = (M <= 128 || cdiv(N, 128) * cdiv(M, 256) <= cus / 2) ? 8 : 16;
        p.tiles_n = (int)cdiv(N, 128);
        p.tiles_m = (int)cdiv(M, 16 * p.mt);
        tiles = (int64_t)p.tiles_n * p.tiles_m;
        const int64_t stages = K / 64;
        // K splits fill the CUs: about one workgroup (two wave groups) per CU,
        // at most one split per 16 stages and 8 in all; where that leaves
        // one split, long K (>= 128 stages) on 128-row tiles, at most one
        // tile per CU, still takes 3-4 splits of single-group workgroups.
        // Measured on the Llama-3-8B layers at M = 96..4096 (explicit splits
        // 1..8): M = 256 qkv 40 -> 32 us (2 splits), o 38 -> 27 us (4),
        // M = 96 down 115 -> 39 us (8), M = 768 down 136 -> 107 us and
        // M = 1024 down 145 -> 136 us (4 and 3, single group); 256-row tiles
        // at M = 2048 gain nothing from them (down 239 vs 245 us).
        const int64_t smax = std::min<int64_t>(8, std::max<int64_t>(1, stages / 16));
        int64_t s = std::min<int64_t>(smax, std::max<int64_t>(1, cus / tiles));
        if (s == 1 && p.mt == 8 && stages >= 128 && tiles <= cus)
            s = std::min<int64_t>(4, std::max<int64_t>(1, 3 * cus / tiles));
        // and where the two-group workgroups would leave more than an eighth
        // of the CUs idle, single-group splits that give each CU three: down
        // at M = 384, 96 tiles (192 two-group workgroups), 80.7 -> 68.0 us
        // with 8 splits (768 workgroups)
        else if (p.mt == 8 && stages >= 128 && 8 * tiles * s < 7 * cus)
            s = std::max<int64_t>(s, std::min<int64_t>(smax, 3 * cus / tiles));
        if (split_k > 0) s = std::min<int64_t>(split_k, stages);
        p.splits = (int)std::min<int64_t>(s, kMaxSplitK);
        // a split's partials are addressed as one buffer of M x N floats
        if (M * N * 4 >= (int64_t(1) << 31)) p.splits = 1;
        // no more workgroups than CUs: two wave groups per workgroup split K
        // inside it (twice the waves per SIMD, no extra atomics)
        p.ksplit = tiles * p.splits <= cus && stages / p.splits >= 4 ? 2 : 1;
        // 256-column tiles (8 waves, one workgroup per CU) wherever they
        // still give more than half the CUs a tile and the plan has neither
        // a K split nor a split group: the X bytes copied per multiply-add
        // halve.  Measured at M = 2048: (4096, 14336) 266 -> 252 us, the
        // Llama-3-8B qkv layer 137 -> 125 us, its gate/up layer unchanged.
        // Not where the 128-column tiles spread over the CUs at least 1.25x
        // more evenly (tiles / (CUs x tiles on the busiest CU)): the Llama-3-8B
        // qkv layer at M = 4096, 384 wide tiles (0.75) against 768 (1.0),
        // 209 -> 195 us; at 1.14x (gate/up at M = 2048, 896 against 1792)
        // the two are level.
        p.wn = 4;
        const int64_t wide_tiles = cdiv(N, 256) * p.tiles_m;
        const int64_t wide_rounds = cdiv(wide_tiles, cus), narrow_rounds = cdiv(tiles, cus);
        const bool wide_even = 5 * wide_tiles * narrow_rounds >= 4 * tiles * wide_rounds;
        if (p.mt == 16 && p.ksplit == 1 && p.splits == 1 && N >= 256 && wide_tiles > cus / 2 && wide_even) {
            p.wn = 8;
            p.tiles_n = (int)cdiv(N, 256);
        }
    }
    if (p.splits <= 1) {
        p.workspace_bytes = 0;
    } else if (p.kind == 0) {
        // decode: counting accumulators (fp16) or per-tile partials (bf16)
        const size_t atomics = (size_t)M * N * sizeof(uint64_t);
        const size_t tiles_ws = (size_t)split_tiles_bytes(p.tiles_n, p.splits, M, N);
        p.workspace_bytes = dtype == AWQ_DTYPE_F16 ? atomics
                            : dtype == AWQ_DTYPE_BF16 ? tiles_ws : std::max(atomics, tiles_ws);
    } else {
        p.workspace_bytes = (size_t)split_tiles_bytes((int64_t)p.tiles_n * p.tiles_m, p.splits, M, N);
    }
    return p;
}

// The fused-quantisation path of w4a8_linear: one activation row (measured:
// the fused form saves the quantisation launch at M = 1 but is slower from
// M = 4 on, where every workgroup re-reads and re-quantises several rows),
// K <= 32768, and the int8 row of each wave's K range in LDS.
bool w4a8_fuses_quant(int64_t M, int64_t K, const W4A8Plan &p) {
    return p.kind == 0 && p.mt == 1 && M == 1 && K <= 32768 && w4a8_fused_lds_bytes(M, K, p.blk, p.splits) <= 64 * 1024;
}

W4A8Plan plan_w4a8(int64_t M, int64_t N, int64_t K, int G, const DeviceProps &d) {
    const int64_t cus = d.cus;
    W4A8Plan p{};
    const int64_t T = K / 64;
    int64_t tiles;
    // M <= 64: the split-K skinny kernel (up to four 16-row tiles per
    // workgroup; measured against the tiled kernel on the QQQ shape:
    // M = 33 62 -> 34 us, M = 64 66 -> 48 us)
    if (M <= 64) {
        p.kind = 0;
        p.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
        p.blk = (M <= 16 && N % 128 == 0) ? 2 : 1;
        p.tiles_n = (int)cdiv(N, 64 * p.blk);
        p.tiles_m = 1;
        tiles = p.tiles_n;
        int64_t s = cdiv(target_workgroups(d), tiles);
        s = std::min<int64_t>(s, std::max<int64_t>(1, T / 4));
        s = skinny_splits(s, M, N, K);
        p.splits = (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
    } else {
        p.kind = 1;
        p.blk = 1;
        p.mt = M >= 128 ? 4 : (M >= 64 ? 2 : 1);
        p.tiles_n = (int)cdiv(N, 128);
        p.tiles_m = (int)cdiv(M, 32 * p.mt);
        tiles = (int64_t)p.tiles_n * p.tiles_m;
        int64_t s = 1;
        if (tiles < cus) {
            s = cdiv(target_workgroups(d), tiles);
            s = std::min<int64_t>(s, std::max<int64_t>(1, T / 2));
            s = std::min<int64_t>(s, 4);  // partial tiles: see the W4A16 tiled kernel
        }
        p.splits = (int)std::max<int64_t>(1, s);
    }
    // buffer-descriptor copies address a8, the packed words and s3 with
    // 32-bit offsets
    const bool fits_rsrc = M * K < (int64_t(1) << 31) && (K / 8) * N * 4 < (int64_t(1) << 31) &&
                           (G <= 0 || (K / G) * N * 2 < (int64_t(1) << 31));
    // From 65 rows the LDS-pipelined GEMM (its last row tile padded): the
    // register-tiled kernel above keeps only shapes past its 32-bit offsets.
    // Measured at M = 65..127 against it: (4096, 14336) 45-50 -> 22-23 us,
    // the QQQ shape 67-71 -> 37-38 us (the INT4-FP8 GEMM the same).  From 33
    // rows also wherever the skinny kernel would split K (its per-element
    // atomics grow with S M N); cache-cold at M = 48 / 64: (4096, 4096)
    // 17.5 / 20.7 -> 13.3 / 14.2 us, the QQQ shape 41.2 / 49.4 -> 35.6 /
    // 36.0, (14336, 4096) 24.0 / 29.8 -> 24.1 / 24.8; with one split
    // ((4096, 14336)) the two are level (19.3 / 21.2 against 19.6 / 20.7).
    if (lds_rows(M, p) && fits_rsrc) {
        // LDS-pipelined int8 GEMM, K in stages of 64: 128 x 256 workgroup
        // tiles (8 waves) where more than half the CUs get one, else 128 x 128
        // (4 waves).  Measured at M = 384..768: (4096, 14336) at M = 384, 168
        // wide tiles, 34.7 -> 30.6 us; the QQQ shape at M = 768, 192 of them,
        // 145 -> 128 us; with 128 (the QQQ shape at M = 512) the narrow tiles
        // win, 97.6 against 107.7.
        p.kind = 2;
        const int64_t wide = cdiv(N, 256) * cdiv(M, 128);
        p.blk = 2 * wide > cus ? 2 : 1;
        // no more wide tiles than CUs: two groups of 8 waves per workgroup
        // split K inside it (four waves per SIMD instead of two)
        p.ksplit = p.blk == 2 && wide <= cus && T >= 8 ? 2 : 1;
        p.mt = 4;
        p.tiles_n = (int)cdiv(N, 128 * p.blk);
        p.tiles_m = (int)cdiv(M, 128);
        tiles = (int64_t)p.tiles_n * p.tiles_m;
        // K splits for the narrow tiles where they leave CUs idle: every split
        // adds an M x N int32 partial tile written, read back and cleared, so
        // short K (under 256 stages) takes only whole multiples of the tiles
        // that fit (CUs / tiles, rounded down) and long K rounds up; at most
        // 4.  Measured (separate reduction): (4096, 4096) at M = 128 21.0 ->
        // 16.2 us (4 splits; 8: 20.9), at M = 768 1 split 24.3 against 2 30.5;
        // (4096, 14336) at M = 256 25.4 against 2 splits 32.6; the QQQ shape
        // (K = 21760) at M = 128 84 -> 36 us (4), at M = 384 89.3 -> 84.9 (2).
        int64_t s = 1;
        if (p.blk == 1 && tiles < cus) {
            s = T >= 256 ? cdiv(cus, tiles) : cus / tiles;
            s = std::min<int64_t>({s, 4, std::max<int64_t>(1, T / 16)});
        }
        p.splits = (int)std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplitK));
    }
    (void)tiles;
    // the small-M kernel (M <= 64) keeps one counting atomic per output
    // element: a single round trip at the end, measured faster there than
    // partial tiles up to M = 32; the larger kernels reduce by partial tiles
    p.tilered = p.kind != 0;
    if (p.splits <= 1)
        p.workspace_bytes = 0;
    else if (!p.tilered)
        p.workspace_bytes = (size_t)M * N * sizeof(uint64_t);
    else
        p.workspace_bytes = (size_t)split_tiles_bytes((int64_t)p.tiles_n * p.tiles_m, p.splits, M, N);
    return p;
}

W4A8Plan plan_w4a8_fp8(int64_t M, int64_t N, int64_t K, const DeviceProps &d) {
    const int64_t cus = d.cus;
    W4A8Plan p{};
    const int64_t T = K / 128;  // 128-k steps
    int64_t tiles;
    if (M <= 64) {
        // split-K skinny kernel, counting fixed-point accumulators
        p.kind = 0;
        p.mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
        p.blk = (M <= 16 && N % 128 == 0) ? 2 : 1;
        p.tiles_n = (int)cdiv(N, 64 * p.blk);
        p.tiles_m = 1;
        tiles = p.tiles_n;
        int64_t s = cdiv(target_workgroups(d), tiles);
        s = std::min<int64_t>(s, std::max<int64_t>(1, T / 2));
        s = skinny_splits(s, M, N, K);
        p.splits = (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
        p.workspace_bytes = p.splits > 1 ? (size_t)M * N * sizeof(uint64_t) : 0;
    } else {
        // register-tiled kernel, K split through per-tile fp32 partials
        p.kind = 1;
        p.blk = 1;
        p.mt = M >= 128 ? 4 : 2;
        p.tiles_n = (int)cdiv(N, 128);
        p.tiles_m = (int)cdiv(M, 32 * p.mt);
        tiles = (int64_t)p.tiles_n * p.tiles_m;
        int64_t s = 1;
        if (tiles < cus) s = std::min<int64_t>({cdiv(target_workgroups(d), tiles), std::max<int64_t>(1, T / 2), 4});
        p.splits = (int)std::max<int64_t>(1, s);
        p.tilered = 1;
        p.workspace_bytes = p.splits > 1 ? (size_t)split_tiles_bytes(tiles, p.splits, M, N) : 0;
    }
    // LDS-pipelined GEMM from 65 rows (as in the int8 planner): 128 x 256 tiles (one workgroup per
    // CU), 128-k stages; a K split through per-tile fp32 partials where tiles
    // are fewer than CUs.  Every split adds an M x N partial tile written,
    // read back and cleared, so the splits are those that fit in one round
    // (CUs / tiles), at most K / 1024, K / (4 M) and 8.  Measured (separate
    // reduction) at M = 128..1024: (4096, 4096) at M = 128 64.2 -> 18.8 us (4
    // splits), at M = 512 28.2 (2) against 31.3 (4), at M = 1024 33.4 (1)
    // against 36.7 (2); (14336, 4096) at M = 128 120.7 -> 25.7 (8); the QQQ
    // shape at M = 256 87.3 -> 57.1 (4), at M = 768 181 -> 134 (1).
    // (Buffer-descriptor copies address the codes and the packed words with
    // 32-bit offsets.)
    const bool fits_rsrc = M * K < (int64_t(1) << 31) && (K / 8) * N * 4 < (int64_t(1) << 31);
    if (lds_rows(M, p) && fits_rsrc) {
        p.kind = 2;
        p.blk = 2;
        p.mt = 4;
        p.tiles_n = (int)cdiv(N, 256);
        p.tiles_m = (int)cdiv(M, 128);
        tiles = (int64_t)p.tiles_n * p.tiles_m;
        int64_t s = 1;
        if (tiles < cus) s = std::min<int64_t>({cus / tiles, K / 1024, K / (4 * M), 8});
        p.splits = (int)std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplitK));
        p.tilered = 1;
        p.workspace_bytes = p.splits > 1 ? (size_t)split_tiles_bytes(tiles, p.splits, M, N) : 0;
    }
    return p;
}

// INT4-FP8 shapes: K in 128-k matrix-core steps; the skinny kernel's
// fixed-point split-K sum holds |sum a u 2^-9| <= 13.2 K below 2^27
static int check_fp8_shape(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 8 || K < 1 || M > kMaxDim || N > kMaxDim) return AWQ_EINVAL;
    if (N % 8) return AWQ_EINVAL;
    if (K % 128 || K > kW8MaxK) return AWQ_EUNSUPPORTED;
    return AWQ_OK;
}

static int check_w4a16(const void *x, const int32_t *qweight, const void *scales, const int32_t *qzeros, void *y,
                       int64_t M, int64_t N, int64_t K, int G, int dtype, int split_k) {
    if (!x || !qweight || !scales || !y) return AWQ_EINVAL;
    if (M < 1 || N < 8 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return AWQ_EINVAL;
    if (N % 8 != 0) return AWQ_EINVAL;
    if (G != 32 && G != 64 && G != 128) return AWQ_EINVAL;
    if (K % G != 0) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    if (split_k < 0 || split_k > K / 32 || split_k > kMaxSplitK) return AWQ_EINVAL;
    if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y)) return AWQ_EALIGN;
    if (qzeros && !aligned16(qzeros)) return AWQ_EALIGN;
    return AWQ_OK;
}

static int check_workspace(void *ws, size_t have, size_t need) {
    if (need == 0) return AWQ_OK;
    if (!ws || have < need) return AWQ_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return AWQ_EALIGN;
    return AWQ_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_EHIP; }

static int run_w4a16(const void *x, const int32_t *qweight, const void *scales, const int32_t *qzeros, void *y,
                     int64_t M, int64_t N, int64_t K, int G, int dtype, int split_k, void *workspace,
                     size_t workspace_bytes, void *stream, bool gemv) {
    int rc = check_w4a16(x, qweight, scales, qzeros, y, M, N, K, G, dtype, split_k);
    if (rc != AWQ_OK) return rc;
    if (gemv && M > 8) return AWQ_EUNSUPPORTED;
    W4A16Plan p = plan_w4a16(M, N, K, G, split_k, dtype, stream_props(stream));
    rc = check_workspace(workspace, workspace_bytes, p.workspace_bytes);
    if (rc != AWQ_OK) return rc;
    // every plan that needs a workspace (split-K or stream-K) gets it
    if (p.workspace_bytes > 0) p.acc = static_cast<uint64_t *>(workspace);
    W4A16Args a{x, qweight, scales, qzeros, y, M, N, K, G, dtype};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (p.kind) {
        case 0: e = launch_w4a16_decode(a, p, st); break;
        case 3: e = launch_w4a16_gemm(a, p, st); break;
        case 5: e = launch_w4a16_stream(a, p, st); break;
        default: e = launch_w4a16_tiled(a, p, st); break;
    }
    return hip_status(e);
}

}  // namespace awq4

using namespace awq4;

extern "C" {

const char *awq_status_str(int status) {
    switch (status) {
        case AWQ_OK: return "AWQ_OK";
        case AWQ_EINVAL: return "AWQ_EINVAL: invalid argument";
        case AWQ_EUNSUPPORTED: return "AWQ_EUNSUPPORTED: unsupported shape or mode";
        case AWQ_EWORKSPACE: return "AWQ_EWORKSPACE: workspace missing or too small";
        case AWQ_EALIGN: return "AWQ_EALIGN: pointer not 16-byte aligned";
        case AWQ_EHIP: return "AWQ_EHIP: HIP launch error";
        default: return "AWQ_UNKNOWN";
    }
}

int awq_version(void) { return 102; }

static int check_pack_shape(int64_t rows, int64_t cols, int layout) {
    if (rows < 0 || cols < 0 || rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return AWQ_EINVAL;
    if (layout == AWQ_LAYOUT_V2) return AWQ_OK;
    if (layout == AWQ_LAYOUT_N8) return cols % 8 ? AWQ_EINVAL : AWQ_OK;
    if (layout == W4A8_LAYOUT_K8) return rows % 8 ? AWQ_EINVAL : AWQ_OK;
    return AWQ_EINVAL;
}

int awq_pack(const void *vals, int32_t *packed, int64_t rows, int64_t cols, int layout, int32_t *clamp_count,
             void *stream) {
    int rc = check_pack_shape(rows, cols, layout);
    if (rc != AWQ_OK) return rc;
    if (rows == 0 || cols == 0) return AWQ_OK;  // nothing to do (empty tensors may have null data)
    if (!vals || !packed) return AWQ_EINVAL;
    if (!aligned16(vals) || !aligned16(packed)) return AWQ_EALIGN;
    return hip_status(launch_pack(vals, packed, rows, cols, layout, clamp_count, static_cast<hipStream_t>(stream)));
}

int awq_unpack(const int32_t *packed, void *vals, int64_t rows, int64_t cols, int layout, void *stream) {
    int rc = check_pack_shape(rows, cols, layout);
    if (rc != AWQ_OK) return rc;
    if (rows == 0 || cols == 0) return AWQ_OK;
    if (!vals || !packed) return AWQ_EINVAL;
    if (!aligned16(vals) || !aligned16(packed)) return AWQ_EALIGN;
    return hip_status(launch_unpack(packed, vals, rows, cols, layout, static_cast<hipStream_t>(stream)));
}

int awq_repack_v2(const int32_t *qweight_v2, const int32_t *qzeros_v2, int32_t *qweight, int32_t *qzeros, int64_t N,
                  int64_t K, int group_size, void *stream) {
    if (!qweight_v2 || !qweight || (qzeros_v2 && !qzeros)) return AWQ_EINVAL;
    if (N < 8 || K < 1 || N > kMaxDim || K > kMaxDim || N % 8) return AWQ_EINVAL;
    if (group_size != 32 && group_size != 64 && group_size != 128) return AWQ_EINVAL;
    if (K % group_size) return AWQ_EINVAL;
    if (!aligned16(qweight_v2) || !aligned16(qweight)) return AWQ_EALIGN;
    if (qzeros_v2 && (!aligned16(qzeros_v2) || !aligned16(qzeros))) return AWQ_EALIGN;
    return hip_status(launch_repack_v2(qweight_v2, qzeros_v2, qweight, qzeros, N, K, group_size,
                                       static_cast<hipStream_t>(stream)));
}

int awq_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0) return AWQ_EINVAL;
    if (!aligned16(src) || !aligned16(sink)) return AWQ_EALIGN;
    return hip_status(launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

size_t awq_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int group_size, int split_k) {
    if (op == AWQ_OP_GEMM_W4A16 || op == AWQ_OP_GEMV_W4A16) {
        int64_t dummy = 16;  // any aligned non-null value: only shapes are checked here
        if (check_w4a16(&dummy, (const int32_t *)&dummy, &dummy, nullptr, &dummy, M, N, K, group_size,
                        AWQ_DTYPE_F16, split_k) == AWQ_EINVAL)
            return 0;
        if (op == AWQ_OP_GEMV_W4A16 && M > 8) return 0;
        return plan_w4a16(M, N, K, group_size, split_k, -1, stream_props(nullptr)).workspace_bytes;
    }
    if (op == AWQ_OP_W4A8_FP8_GEMM) {
        if (check_fp8_shape(M, N, K) != AWQ_OK) return 0;
        return plan_w4a8_fp8(M, N, K, stream_props(nullptr)).workspace_bytes;
    }
    if (op == AWQ_OP_W4A8_GEMM) {
        if (M < 1 || N < 8 || N % 8 || K < 64 || K % 64 || M > kMaxDim || N > kMaxDim || K > kW8MaxK) return 0;
        if (group_size != -1 && ((group_size != 32 && group_size != 64 && group_size != 128) || K % group_size))
            return 0;
        return plan_w4a8(M, N, K, group_size, stream_props(nullptr)).workspace_bytes;
    }
    return 0;
}

int awq_plan_info(int op, int64_t M, int64_t N, int64_t K, int group_size, int split_k, int cu_count,
                  awq_plan_t *out) {
    if (!out || cu_count < 0) return AWQ_EINVAL;
    const DeviceProps d = cu_count > 0 ? DeviceProps{cu_count} : stream_props(nullptr);
    if (op == AWQ_OP_GEMM_W4A16 || op == AWQ_OP_GEMV_W4A16) {
        int64_t dummy = 16;
        int rc = check_w4a16(&dummy, (const int32_t *)&dummy, &dummy, nullptr, &dummy, M, N, K, group_size,
                             AWQ_DTYPE_F16, split_k);
        if (rc != AWQ_OK) return rc;
        if (op == AWQ_OP_GEMV_W4A16 && M > 8) return AWQ_EUNSUPPORTED;
        const W4A16Plan p = plan_w4a16(M, N, K, group_size, split_k, -1, d);
        *out = awq_plan_t{p.kind, p.tiles_n, p.tiles_m, p.splits, p.mt, std::max(1, p.ksplit), d.cus,
                          (int64_t)p.workspace_bytes, p.kind == 3 ? 32 * p.wn : 0};
        return AWQ_OK;
    }
    if (op == AWQ_OP_W4A8_FP8_GEMM) {
        const int rc = check_fp8_shape(M, N, K);
        if (rc != AWQ_OK) return rc;
        const W4A8Plan p = plan_w4a8_fp8(M, N, K, d);
        *out = awq_plan_t{p.kind, p.tiles_n, p.tiles_m, p.splits, p.mt, 1, d.cus, (int64_t)p.workspace_bytes,
                          p.kind == 2 ? 256 : 0};
        return AWQ_OK;
    }
    if (op == AWQ_OP_W4A8_GEMM) {
        if (M < 1 || N < 8 || N % 8 || M > kMaxDim || N > kMaxDim) return AWQ_EINVAL;
        if (group_size != -1 && ((group_size != 32 && group_size != 64 && group_size != 128) || K % group_size))
            return AWQ_EINVAL;
        if (K < 64 || K % 64 || K > kW8MaxK) return AWQ_EUNSUPPORTED;
        const W4A8Plan p = plan_w4a8(M, N, K, group_size, d);
        *out = awq_plan_t{p.kind, p.tiles_n, p.tiles_m, p.splits, p.mt, std::max(1, p.ksplit), d.cus,
                          (int64_t)p.workspace_bytes, p.kind == 2 ? 128 * p.blk : 0};
        return AWQ_OK;
    }
    return AWQ_EINVAL;
}

int awq_gemm_w4a16(const void *x, const int32_t *qweight, const void *scales, const int32_t *qzeros, void *y,
                   int64_t M, int64_t N, int64_t K, int group_size, int dtype, int split_k, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return run_w4a16(x, qweight, scales, qzeros, y, M, N, K, group_size, dtype, split_k, workspace,
                     workspace_bytes, stream, false);
}

int awq_gemv_w4a16(const void *x, const int32_t *qweight, const void *scales, const int32_t *qzeros, void *y,
                   int64_t M, int64_t N, int64_t K, int group_size, int dtype, int split_k, void *workspace,
                   size_t workspace_bytes, void *stream) {
    return run_w4a16(x, qweight, scales, qzeros, y, M, N, K, group_size, dtype, split_k, workspace,
                     workspace_bytes, stream, true);
}

int awq_gemv_w4a16_static(const void *x, const int32_t *qweight, const void *scales, const int32_t *qzeros,
                          void *y, int64_t M, int64_t N, int64_t K, int group_size, int dtype, void *stream) {
    int rc = check_w4a16(x, qweight, scales, qzeros, y, M, N, K, group_size, dtype, 0);
    if (rc != AWQ_OK) return rc;
    if (M > 8) return AWQ_EUNSUPPORTED;
    const int dev = stream_device(stream);
    if (dev < 0) return AWQ_EHIP;
    W4A16Plan p = plan_w4a16(M, N, K, group_size, 0, dtype, props_of_device(dev));
    if (p.workspace_bytes > kScratchBytes) return AWQ_EWORKSPACE;
    void *ws = nullptr;
    rc = scratch_of_device(dev, &ws);
    if (rc != AWQ_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The split-K kernels need the scratch zero (they leave it zero after
    // every call).  Until a clear has been enqueued on this device outside
    // graph capture, clear it first; a clear recorded into a graph runs only
    // when the graph does, so it does not count.
    if (!g_scratch[dev].cleared.load(std::memory_order_acquire)) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) != hipSuccess) return AWQ_EHIP;
        hipLaunchKernelGGL(scratch_zero, dim3(256), dim3(256), 0, st, static_cast<uint4 *>(ws),
                           kScratchBytes / sizeof(uint4));
        if (hipGetLastError() != hipSuccess) return AWQ_EHIP;
        if (cs == hipStreamCaptureStatusNone) g_scratch[dev].cleared.store(1, std::memory_order_release);
    }
    if (p.workspace_bytes > 0) p.acc = static_cast<uint64_t *>(ws);
    W4A16Args a{x, qweight, scales, qzeros, y, M, N, K, group_size, dtype};
    return hip_status(p.kind == 0 ? launch_w4a16_decode(a, p, st) : launch_w4a16_tiled(a, p, st));
}

int awq_dequant_w4a16(const int32_t *qweight, const void *scales, const int32_t *qzeros, void *w, int64_t N,
                      int64_t K, int group_size, int dtype, void *stream) {
    int64_t dummy = 16;  // stands in for x and y, which this call does not have
    int rc = check_w4a16(&dummy, qweight, scales, qzeros, w ? w : nullptr, 1, N, K, group_size, dtype, 0);
    if (rc != AWQ_OK) return rc;
    if ((K / 8) * ((N / 8 + 255) / 256) >= (int64_t(1) << 31)) return AWQ_EUNSUPPORTED;
    return hip_status(launch_w4a16_dequant(qweight, scales, qzeros, w, N, K, group_size, dtype,
                                           static_cast<hipStream_t>(stream)));
}

int w4a8_quant_act(const void *x, int8_t *a8, float *s1, int64_t M, int64_t K, int dtype, void *stream) {
    if (!x || !a8 || !s1) return AWQ_EINVAL;
    if (M < 1 || K < 1 || M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 30)) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    if (!aligned16(x) || !aligned16(a8) || !aligned16(s1)) return AWQ_EALIGN;
    return hip_status(launch_w4a8_quant(x, a8, s1, M, K, dtype, static_cast<hipStream_t>(stream)));
}

int w4a8_gemm(const int8_t *a8, const int32_t *b_packed, const float *s1, const void *s2_f16, const void *s3_f16,
              void *y_f16, int32_t *acc_out, int64_t M, int64_t N, int64_t K, int group_size, int dtype,
              void *workspace, size_t workspace_bytes, void *stream) {
    if (!a8 || !b_packed || !s1 || !s2_f16 || !y_f16) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    if (M < 1 || N < 8 || K < 1 || M > kMaxDim || N > kMaxDim) return AWQ_EINVAL;
    if (N % 8) return AWQ_EINVAL;
    if (group_size == -1) {
        if (s3_f16) return AWQ_EINVAL;
    } else {
        if (group_size != 32 && group_size != 64 && group_size != 128) return AWQ_EINVAL;
        if (!s3_f16 || K % group_size) return AWQ_EINVAL;
    }
    // 64 k per matrix-core step; |acc| <= 128 * 128 * K must stay below 2^31
    if (K % 64 || K > kW8MaxK) return AWQ_EUNSUPPORTED;
    if (!aligned16(a8) || !aligned16(b_packed) || !aligned16(s1) || !aligned16(s2_f16) || !aligned16(y_f16))
        return AWQ_EALIGN;
    if ((s3_f16 && !aligned16(s3_f16)) || (acc_out && !aligned16(acc_out))) return AWQ_EALIGN;
    W4A8Plan p = plan_w4a8(M, N, K, group_size, stream_props(stream));
    int rc = check_workspace(workspace, workspace_bytes, p.workspace_bytes);
    if (rc != AWQ_OK) return rc;
    if (p.splits > 1) {
        p.acc = static_cast<uint64_t *>(workspace);
    }
    W4A8Args a{a8, b_packed, s1, s2_f16, s3_f16, y_f16, acc_out, M, N, K, group_size};
    a.dtype = dtype;
    return hip_status(launch_w4a8(a, p, static_cast<hipStream_t>(stream)));
}

int w4a8_fp8_quant_act(const void *x, uint8_t *a, float *s1, float *asum, int64_t M, int64_t K, int dtype,
                       void *stream) {
    if (!x || !a || !s1 || !asum) return AWQ_EINVAL;
    if (M < 1 || K < 1 || M > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 30)) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    if (!aligned16(x) || !aligned16(a) || !aligned16(s1) || !aligned16(asum)) return AWQ_EALIGN;
    return hip_status(launch_w4a8_fp8_quant(x, a, s1, asum, M, K, dtype, static_cast<hipStream_t>(stream)));
}

int w4a8_fp8_gemm(const uint8_t *a, const int32_t *b_packed, const float *s1, const float *asum, const void *s2,
                  void *y, float *acc_out, int64_t M, int64_t N, int64_t K, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream) {
    if (!a || !b_packed || !s1 || !asum || !s2 || !y) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    int rc = check_fp8_shape(M, N, K);
    if (rc != AWQ_OK) return rc;
    if (!aligned16(a) || !aligned16(b_packed) || !aligned16(s1) || !aligned16(asum) || !aligned16(s2) ||
        !aligned16(y) || (acc_out && !aligned16(acc_out)))
        return AWQ_EALIGN;
    W4A8Plan p = plan_w4a8_fp8(M, N, K, stream_props(stream));
    rc = check_workspace(workspace, workspace_bytes, p.workspace_bytes);
    if (rc != AWQ_OK) return rc;
    if (p.splits > 1) p.acc = static_cast<uint64_t *>(workspace);
    W4A8Fp8Args g{a, b_packed, s1, asum, s2, y, acc_out, M, N, K, dtype};
    return hip_status(launch_w4a8_fp8(g, p, static_cast<hipStream_t>(stream)));
}

int w4a8_fp8_linear(const void *x, uint8_t *a, float *s1, float *asum, const int32_t *b_packed, const void *s2,
                    void *y, float *acc_out, int64_t M, int64_t N, int64_t K, int dtype, void *workspace,
                    size_t workspace_bytes, void *stream) {
    if (!x || !a || !s1 || !asum || !b_packed || !s2 || !y) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    int rc = check_fp8_shape(M, N, K);
    if (rc != AWQ_OK) return rc;
    if (!aligned16(x) || !aligned16(a) || !aligned16(s1) || !aligned16(asum) || !aligned16(b_packed) ||
        !aligned16(s2) || !aligned16(y) || (acc_out && !aligned16(acc_out)))
        return AWQ_EALIGN;
    W4A8Plan p = plan_w4a8_fp8(M, N, K, stream_props(stream));
    rc = check_workspace(workspace, workspace_bytes, p.workspace_bytes);
    if (rc != AWQ_OK) return rc;
    if (p.splits > 1) p.acc = static_cast<uint64_t *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    W4A8Fp8Args g{a, b_packed, s1, asum, s2, y, acc_out, M, N, K, dtype};
    if (w4a8_fp8_fuses_quant(M, K, p)) return hip_status(launch_w4a8_fp8_fused(g, x, s1, p, st));
    rc = hip_status(launch_w4a8_fp8_quant(x, a, s1, asum, M, K, dtype, st));
    if (rc != AWQ_OK) return rc;
    return hip_status(launch_w4a8_fp8(g, p, st));
}

int w4a8_linear(const void *x_f16, int8_t *a8, float *s1, const int32_t *b_packed, const void *s2_f16,
                const void *s3_f16, void *y_f16, int32_t *acc_out, int64_t M, int64_t N, int64_t K, int group_size,
                int dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (!x_f16 || !a8 || !s1 || !b_packed || !s2_f16 || !y_f16) return AWQ_EINVAL;
    if (dtype != AWQ_DTYPE_F16 && dtype != AWQ_DTYPE_BF16) return AWQ_EINVAL;
    if (M < 1 || N < 8 || K < 1 || M > kMaxDim || N > kMaxDim) return AWQ_EINVAL;
    if (N % 8) return AWQ_EINVAL;
    if (group_size == -1) {
        if (s3_f16) return AWQ_EINVAL;
    } else {
        if (group_size != 32 && group_size != 64 && group_size != 128) return AWQ_EINVAL;
        if (!s3_f16 || K % group_size) return AWQ_EINVAL;
    }
    if (K % 64 || K > kW8MaxK) return AWQ_EUNSUPPORTED;
    if (!aligned16(x_f16) || !aligned16(a8) || !aligned16(s1) || !aligned16(b_packed) || !aligned16(s2_f16) ||
        !aligned16(y_f16))
        return AWQ_EALIGN;
    if ((s3_f16 && !aligned16(s3_f16)) || (acc_out && !aligned16(acc_out))) return AWQ_EALIGN;
    W4A8Plan p = plan_w4a8(M, N, K, group_size, stream_props(stream));
    int rc = check_workspace(workspace, workspace_bytes, p.workspace_bytes);
    if (rc != AWQ_OK) return rc;
    if (p.splits > 1) p.acc = static_cast<uint64_t *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    W4A8Args a{a8, b_packed, s1, s2_f16, s3_f16, y_f16, acc_out, M, N, K, group_size};
    a.dtype = dtype;
    if (w4a8_fuses_quant(M, K, p)) {
        a.x = x_f16;
        a.s1_out = s1;
        return hip_status(launch_w4a8_fused(a, p, st));
    }
    rc = hip_status(launch_w4a8_quant(x_f16, a8, s1, M, K, dtype, st));
    if (rc != AWQ_OK) return rc;
    return hip_status(launch_w4a8(a, p, st));
}

}  // extern "C"
