// launch.hpp -- internal interface between the C-ABI layer (api.cpp) and the
// kernel launchers (*.hip).  Arguments are validated by api.cpp before any
// launcher is called; launchers only enqueue work on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq4 {

struct W4A16Args {
    const void *x;
    const int32_t *qweight;
    const void *scales;
    const int32_t *qzeros;  // nullptr = symmetric (z = 8)
    void *y;
    int64_t M, N, K;
    int G;
    int dtype;
};

// Kernel choice and grid for one W4A16 call (pure function of the shape).
struct W4A16Plan {
    int kind;     // 0 = decode (chunk) kernel, 1 = tiled kernel,
                  // 3 = LDS-pipelined GEMM (large M), 5 = streaming kernel (8 < M <= 64)
    int blk;      // decode: word-columns per lane (1, 2)
    int cs;       // decode: 32-k steps per wave chunk (1, 2, 4)
    int waves;    // decode: waves per workgroup (4)
    int mt;       // tiled: row tiles per wave (1, 2, 4); LDS GEMM: 16 or 8
    int ksplit;   // LDS GEMM: groups of 4 waves per workgroup splitting K (1, 2)
    int wn;       // LDS GEMM: waves along N, 32 columns each (4: 128-column tiles, 8: 256)
    int tiles_n;  // grid x
    int tiles_m;  // tiled: grid y
    int splits;   // workgroups along K (1 = none); decode: grid y
    size_t workspace_bytes;
    // filled in by the caller from the workspace pointer
    uint64_t *acc;
};

struct W4A8Args {
    const int8_t *a8;  // int8 activations (unused by the fused kernel)
    const int32_t *b;
    const float *s1;
    const void *s2;
    const void *s3;  // nullptr = per-channel
    void *y;
    int32_t *acc_out;  // may be nullptr
    int64_t M, N, K;
    int G;  // -1 = per-channel
    // fused quantisation (w4a8_linear): fp16 or bf16 activations and the s1 output
    const void *x = nullptr;
    float *s1_out = nullptr;
    int dtype = 0;  // DT_F16 / DT_BF16: activations, s2, s3 and y
};

// INT4-FP8 W4A8 (E4M3 activation codes, per-channel int4 weights)
struct W4A8Fp8Args {
    const uint8_t *a;     // E4M3 codes [M, K]
    const int32_t *b;     // K8-packed int4 [K/8, N]
    const float *s1;      // [M]
    const float *asum;    // [M], row sums of the codes' values
    const void *s2;       // [N], activation type
    void *y;              // [M, N], activation type
    float *acc_out;       // [M, N] fp32 sum_k a q, or nullptr
    int64_t M, N, K;
    int dtype;
};

struct W4A8Plan {
    int kind;  // 0 = skinny, 1 = tiled, 2 = LDS-pipelined GEMM (large M)
    int blk;   // skinny: 64-column sets per lane-row (1, 2)
    int mt;    // row tiles (skinny: M <= 16*mt; tiled and LDS GEMM: per wave)
    int tiles_n, tiles_m, splits;
    int tilered;  // split-K through partial tiles (tiled and LDS kernels), else per-element atomics (skinny)
    int ksplit;   // LDS GEMM: groups of waves splitting K inside a workgroup (1, 2)
    size_t workspace_bytes;
    uint64_t *acc;
};

// Workspace of a split-K launch, zero between calls (device.hpp): for the
// decode GEMV and small W4A8 outputs one 64-bit counting accumulator per
// output element (M x N); for the GEMM kernels per-tile arrival counters and
// fp32 / int32 partial tiles.  Splits are capped at 255.
constexpr int kMaxSplitK = 255;

// Partial-tile split-K workspace: uint32 arrival counters, one per output
// tile, padded to 256 bytes, then S partial [M, N] tiles of 4-byte values.
constexpr int64_t kSplitCounterAlign = 256;
__host__ __device__ constexpr int64_t split_counters_bytes(int64_t tiles) {
    return (tiles * 4 + kSplitCounterAlign - 1) / kSplitCounterAlign * kSplitCounterAlign;
}
__host__ __device__ constexpr int64_t split_tiles_bytes(int64_t tiles, int64_t S, int64_t M, int64_t N) {
    return split_counters_bytes(tiles) + S * M * N * 4;
}

// What the launch planners need to know about the device a call runs on,
// queried once per device (api.cpp) and passed to the pure planners.
struct DeviceProps {
    int cus;  // compute units (256 on a whole MI355X; fewer on a partition)
};
constexpr int kDefaultCUs = 256;

// dtype: DT_F16 / DT_BF16 (the decode kernel's split-K workspace depends on
// it), or -1 for a workspace large enough for either
W4A16Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int G, int split_k, int dtype, const DeviceProps &d);
W4A8Plan plan_w4a8(int64_t M, int64_t N, int64_t K, int G, const DeviceProps &d);
// INT4-FP8: kind 0 = skinny split-K (M <= 64), 1 = register-tiled
W4A8Plan plan_w4a8_fp8(int64_t M, int64_t N, int64_t K, const DeviceProps &d);
bool w4a8_fuses_quant(int64_t M, int64_t K, const W4A8Plan &p);

hipError_t launch_w4a16_decode(const W4A16Args &a, const W4A16Plan &p, hipStream_t st);
hipError_t launch_w4a16_gemm(const W4A16Args &a, const W4A16Plan &p, hipStream_t st);
hipError_t launch_w4a16_tiled(const W4A16Args &a, const W4A16Plan &p, hipStream_t st);
// streaming kernel (plan kind 5): waves per workgroup for MT 16-row tiles --
// eight waves up to 32 rows, four 512-register waves at 64
constexpr int kStreamWaves(int mt) { return mt >= 4 ? 4 : 8; }
hipError_t launch_w4a16_stream(const W4A16Args &a, const W4A16Plan &p, hipStream_t st);
// K-split reduction of the LDS GEMM and the streaming kernel in a launch of
// its own (partials after the counters of `tiles` tiles), taken where a
// tile's partials are large: S splits of `rows`-row tiles, S x rows >= 384.
// Measured on the Llama-3-8B layers: down at M = 96 and 128 (eight splits of
// 128 rows) 37.2 -> 31.7 and 42.6 -> 34.8 us, o at M = 64 (six of 64) 18.7 ->
// 17.2 us; smaller volumes keep the in-kernel exchange, which saves the
// launch (qkv at M = 32, five splits of 32 rows: 11.9 against 12.2 us).
constexpr bool split_reduce_apart(int splits, int rows) { return splits > 1 && splits * rows >= 384; }
hipError_t launch_w4a16_split_reduce(const W4A16Args &a, const W4A16Plan &p, int64_t tiles, hipStream_t st);
hipError_t launch_w4a8_gemm_lds(const W4A8Args &a, const W4A8Plan &p, hipStream_t st);
hipError_t launch_w4a8_quant(const void *x, int8_t *a8, float *s1, int64_t M, int64_t K, int dtype, hipStream_t st);
hipError_t launch_w4a8(const W4A8Args &a, const W4A8Plan &p, hipStream_t st);
hipError_t launch_w4a8_fp8_quant(const void *x, uint8_t *a, float *s1, float *asum, int64_t M, int64_t K, int dt,
                                 hipStream_t st);
hipError_t launch_w4a8_fp8(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st);
// the INT4-FP8 skinny GEMM with the single token's quantisation fused in
// (x: the fp16/bf16 activation row; s1_out: its scale, written)
bool w4a8_fp8_fuses_quant(int64_t M, int64_t K, const W4A8Plan &p);
size_t w4a8_fp8_fused_lds_bytes(int64_t K, int blk, int splits);
hipError_t launch_w4a8_fp8_fused(const W4A8Fp8Args &g, const void *x, float *s1_out, const W4A8Plan &p,
                                 hipStream_t st);
// INT4-FP8 LDS-pipelined GEMM (plan kind 2, M >= 128)
hipError_t launch_w4a8_fp8_lds(const W4A8Fp8Args &g, const W4A8Plan &p, hipStream_t st);
// skinny W4A8 GEMM with the per-token quantisation fused in (plan kind 0,
// mt 1); its dynamic LDS and per-wave int8 row area
hipError_t launch_w4a8_fused(const W4A8Args &a, const W4A8Plan &p, hipStream_t st);
size_t w4a8_fused_lds_bytes(int64_t M, int64_t K, int blk, int splits);
// read-only bandwidth probe: at most kStreamMaxBlocks workgroups, one sink
// word per wave
constexpr int64_t kStreamMaxBlocks = 2048;
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st);
// dense [K, N] fp16/bf16 copy of the dequantised weights (a comparator's operand)
hipError_t launch_w4a16_dequant(const int32_t *qweight, const void *scales, const int32_t *qzeros, void *w, int64_t N,
                                int64_t K, int G, int dtype, hipStream_t st);
hipError_t launch_pack(const void *vals, int32_t *packed, int64_t rows, int64_t cols, int layout,
                       int32_t *clamp_count, hipStream_t st);
hipError_t launch_repack_v2(const int32_t *qweight_v2, const int32_t *qzeros_v2, int32_t *qweight, int32_t *qzeros,
                            int64_t N, int64_t K, int G, hipStream_t st);
hipError_t launch_unpack(const int32_t *packed, void *vals, int64_t rows, int64_t cols, int layout,
                         hipStream_t st);

}  // namespace awq4
