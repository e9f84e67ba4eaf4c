/*
 * awq4.h -- C ABI of the MI355X (gfx950) 4-bit-weight GEMM library.
 *
 * The library computes the group-quantised 4-bit-weight linear layer
 *     Y = X . dequant(Wq),   w[k,n] = (q[k,n] - z[k/G,n]) * s[k/G,n]
 * in the first-generation AWQ GEMM weight format, in a decode regime (GEMV,
 * M <= 8) and a prefill regime (GEMM, any M), plus the QQQ-style W4A8 variant
 * (per-token int8 activations x symmetric int4 weights, exact int32
 * accumulation, per-token and per-channel (optionally per-group) scales).
 *
 * Sources (web pages, cited by title and passage):
 *  [P1] vLLM pull request "Speed up AWQ 2.5x with updated kernel": the list of
 *       differences between the old and new AWQ packings (old GEMM order map
 *       [0,2,4,6,1,3,5,7]), and the dispatch snippet (M > 8 -> GEMM, else GEMV;
 *       kernels take inputs, qweight, scales, qzeros, group_size, and the GEMM
 *       a split_k_iters count).
 *  [P2] AutoAWQ pull request "Marlin symmetric quantization and inference":
 *       the symmetric variant without zero points; one workspace per device
 *       rather than per layer.
 *  [P5] vLLM pull request "Support W4A8 quantization for vllm" (QQQ): dynamic
 *       per-token activation quantisation; int4 -> int8 by placing the nibble
 *       in the upper four bits; int32 global reduce through a temporary
 *       buffer; s1 (per token) and s2 (per channel) applied to the output,
 *       with per-group scales in addition for grouped weights; the GEMM
 *       signature (a, b_q_weight, s1, s2, s3, workspace, size_m, size_n,
 *       size_k) with const operands; a missing clamp in packing as a real bug.
 *
 * Conventions for every entry point:
 *  - All tensors are dense, row-major and contiguous, in device memory owned
 *    by the caller.  Device pointers must be 16-byte aligned (AWQ_EALIGN).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued on it; no entry point synchronises or allocates device
 *    memory, so all of them are asynchronous and safe to call from several
 *    host threads on different streams.  Faults inside a kernel surface at
 *    the caller's next synchronisation, as for any HIP launch.
 *  - Arguments are validated before anything is enqueued; a call that
 *    returns an error has written nothing.  Validation needs no GPU.
 *  - Return value: AWQ_OK or a negative AWQ_E* status.
 *  - Results are deterministic: the same inputs give the same bits on every
 *    run (split-K partials are summed in a fixed order).
 */
#ifndef AWQ4_H
#define AWQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define AWQ_OK 0
#define AWQ_EINVAL (-1)       /* bad shape, null pointer, unknown enum value */
#define AWQ_EUNSUPPORTED (-2) /* valid request this library does not implement (e.g. GEMV with M > 8) */
#define AWQ_EWORKSPACE (-3)   /* workspace missing or smaller than awq_workspace_bytes() */
#define AWQ_EALIGN (-4)       /* a device pointer is not 16-byte aligned */
#define AWQ_EHIP (-5)         /* the HIP runtime reported an error when launching */

/* Activation / scale / output dtypes. */
#define AWQ_DTYPE_F16 0
#define AWQ_DTYPE_BF16 1

/* Packed layouts for awq_pack / awq_unpack. */
#define AWQ_LAYOUT_N8 0  /* AWQ: uint8 vals [rows, cols] in 0..15 -> int32 [rows, cols/8];
                            nibble i of word [r][j] holds column 8j + {0,2,4,6,1,3,5,7}[i] ([P1]) */
#define W4A8_LAYOUT_K8 1 /* W4A8: int8 vals [K=rows, N=cols] in -8..7 -> int32 [K/8, N];
                            nibble i of word [kb][n] holds k = 8kb + {0,4,1,5,2,6,3,7}[i],
                            two's complement (this library's own layout) */

#define AWQ_LAYOUT_V2 2   /* the newer AWQ packing ([P1], list of differences; this library's reading):
                            uint8 vals [rows, cols] in 0..15 -> int32 [rows, ceil(cols/8)];
                            nibble i of word [r][j] holds column 8j + i (identity order map),
                            nibbles past the last column are left 0 (skipped); any cols */

/* Operation ids for awq_workspace_bytes. */
#define AWQ_OP_GEMM_W4A16 0
#define AWQ_OP_GEMV_W4A16 1
#define AWQ_OP_W4A8_GEMM 2
#define AWQ_OP_W4A8_FP8_GEMM 3

/* Human-readable name of a status code (static string, never NULL). */
const char *awq_status_str(int status);

/* Library ABI version (major * 100 + minor). */
int awq_version(void);

/*
 * awq_pack -- pack 4-bit values into 32-bit words ([P1] order map for
 * AWQ_LAYOUT_N8; K-packed two's complement for W4A8_LAYOUT_K8).  Used for
 * qweight and qzeros alike.
 *   vals:        device, uint8 [rows, cols] (N8) or int8 [rows, cols] (K8).
 *   packed:      device, int32 [rows, cols/8] (N8) or [rows/8, cols] (K8).
 *   clamp_count: device int32 or NULL.  Values outside 0..15 (N8) / -8..7 (K8)
 *                are clamped into range (the lesson of the missing clamp in
 *                [P5]) and their number is atomically added to *clamp_count,
 *                which the caller zeroes beforehand.
 * rows == 0 or cols == 0 is a no-op that returns AWQ_OK.
 * Errors: AWQ_EINVAL if a pointer is NULL, rows/cols < 0, cols % 8 (N8) or
 * rows % 8 (K8) is non-zero, or the layout is unknown.  AWQ_LAYOUT_V2 takes
 * any cols.
 */
int awq_pack(const void *vals, int32_t *packed, int64_t rows, int64_t cols, int layout,
             int32_t *clamp_count, void *stream);

/*
 * awq_unpack -- inverse of awq_pack: words -> uint8 (N8, 0..15) or int8
 * (K8, -8..7) values [rows, cols].  Same shape rules and errors as awq_pack.
 */
int awq_unpack(const int32_t *packed, void *vals, int64_t rows, int64_t cols, int layout,
               void *stream);

/*
 * awq_repack_v2 -- weights in the newer AWQ packing ([P1]: identity order
 * map, zero points packed per output channel along the groups with unused
 * nibbles skipped, a zeros width of ceil(groups / 8) words) rewritten into
 * the first-generation format that the GEMM and GEMV calls take, bit for bit
 * the same logical values.  A checkpoint in the newer format is repacked
 * once at load; the scales are the same [K/G, N] tensor in both.
 *   qweight_v2: device int32 [K, N/8], AWQ_LAYOUT_V2 along each row.
 *   qzeros_v2:  device int32 [N, ceil((K/G)/8)], AWQ_LAYOUT_V2 along each
 *               output channel's groups; NULL = symmetric (then qzeros is
 *               not written).
 *   qweight:    device int32 [K, N/8], AWQ_LAYOUT_N8 (written).
 *   qzeros:     device int32 [K/G, N/8], AWQ_LAYOUT_N8 (written).
 * Errors: AWQ_EINVAL (shapes, G, NULL qzeros with non-NULL qzeros_v2),
 * AWQ_EALIGN, AWQ_EHIP.
 */
int awq_repack_v2(const int32_t *qweight_v2, const int32_t *qzeros_v2, int32_t *qweight, int32_t *qzeros,
                  int64_t N, int64_t K, int group_size, void *stream);

/*
 * awq_workspace_bytes -- bytes of device workspace the given call needs
 * (0 if none) on the current device.  split_k as passed to the call
 * (0 = automatic).  For W4A8, group_size is the one passed to w4a8_gemm.
 * Workspace rules ([P2]: one workspace per device, reused by every layer):
 *  - it is caller-owned, 16-byte aligned, and may be shared by any number of
 *    calls that are ordered on one stream;
 *  - a split-K fp16 decode GEMV, or a split-K W4A8 call on the skinny
 *    kernel (M <= 32), uses one 64-bit counting accumulator per output
 *    element (M x N); the last contribution to an element writes the output
 *    and clears it (the size returned for the W4A16 calls covers both
 *    activation dtypes);
 *  - a split-K bf16 decode GEMV and the GEMM kernels (M > 8 for W4A16,
 *    M > 32 for W4A8) use one 32-bit
 *    arrival counter per output tile (padded to 256 bytes) followed by S
 *    partial [M, N] results of 4 bytes each (fp32 for W4A16, int32 for
 *    W4A8); the last workgroup of a tile to arrive adds the S partials in
 *    split order, writes the output, clears them and re-arms the counter --
 *    or, where the partials are large (always for the W4A8 GEMMs), a second
 *    kernel enqueued right after the first on the same stream adds them in
 *    split order, writes the output and clears them (counters untouched);
 *  - either way the workspace is zero again after every call;
 *  - it must be zero-filled once when allocated; no per-call clearing is
 *    needed;
 *  - calls that overlap in time (different streams) need separate workspaces.
 * Returns 0 for invalid arguments.
 */
size_t awq_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int group_size, int split_k);

/*
 * awq_plan_info -- how a call would be launched, without launching it: the
 * kernel, grid and workspace the library's planner picks for the given shape
 * on a device with `cu_count` compute units (0 = the current device, queried
 * once per device and cached; a whole MI355X, 256, when no device is
 * visible).  The planners size their grids from this count, so a partitioned
 * or smaller part gets grids of its own size.  Needs no GPU when cu_count > 0.
 *   op: AWQ_OP_*; other arguments as for the call (group_size -1 = W4A8
 *   per-channel).
 *   out: host pointer, written on success.
 * Errors: the validation status the call itself would return for the shape
 * (AWQ_EINVAL, AWQ_EUNSUPPORTED), or AWQ_EINVAL for a NULL out or a negative
 * cu_count.
 */
typedef struct {
    int kernel;    /* W4A16: 0 decode GEMV, 1 register-tiled GEMM, 3 LDS-pipelined GEMM;
                      W4A8: 0 skinny split-K, 1 register-tiled, 2 LDS-pipelined */
    int tiles_n;   /* workgroup tiles along N */
    int tiles_m;   /* workgroup tiles along M */
    int splits;    /* workgroups along K (1 = no split) */
    int row_tiles; /* 16-row matrix-core tiles per wave or workgroup column */
    int ksplit;    /* wave groups splitting K inside one workgroup (1 or 2) */
    int cu_count;  /* the compute-unit count the plan was made for */
    int64_t workspace_bytes;
    int tile_cols; /* LDS-pipelined GEMMs: output columns per workgroup tile (128 or 256);
                      0 for the other kernels */
} awq_plan_t;
int awq_plan_info(int op, int64_t M, int64_t N, int64_t K, int group_size, int split_k, int cu_count,
                  awq_plan_t *out);

/*
 * awq_gemm_w4a16 -- Y = X . dequant(qweight, qzeros, scales) for any M >= 1
 * (the prefill path of the [P1] dispatch; also correct for small M).
 *   x:       device, [M, K] fp16 or bf16 (dtype).
 *   qweight: device, int32 [K, N/8], AWQ_LAYOUT_N8.
 *   scales:  device, [K/G, N] in the activation dtype.
 *   qzeros:  device, int32 [K/G, N/8], AWQ_LAYOUT_N8; NULL = symmetric
 *            weights with z = 8 ([P2]).
 *   y:       device, [M, N] in the activation dtype (written, not accumulated).
 *   group_size G in {32, 64, 128}; K % G == 0; N % 8 == 0; M, N, K >= 1.
 *   split_k: number of K slices reduced through the workspace (0 = chosen by
 *            the library, 1 = none, at most min(K/32, 255)).  For M <= 8
 *            the library's decode kernel fixes the K split itself and
 *            ignores split_k.
 * Numerics: M <= 32, and bf16 up to M = 64 -- the exact (q - z) products
 * are summed in fp32 on the matrix cores and scaled by s in fp32 once per
 * chunk (32 to 128 consecutive k inside one group); fp16 at 32 < M <= 64
 * and M > 64 -- each weight is dequantised exactly to (q - z) and multiplied
 * by s with one rounding to the activation dtype, products accumulating in
 * fp32.  The
 * output is rounded to nearest even.
 * Errors: AWQ_EINVAL (shapes, pointers, dtype, G), AWQ_EALIGN, AWQ_EWORKSPACE,
 * AWQ_EHIP.
 */
int awq_gemm_w4a16(const void *x, const int32_t *qweight, const void *scales,
                   const int32_t *qzeros, void *y, int64_t M, int64_t N, int64_t K,
                   int group_size, int dtype, int split_k, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * awq_gemv_w4a16 -- the decode path of the [P1] dispatch: same tensors,
 * formats, numerics and errors as awq_gemm_w4a16, for 1 <= M <= 8
 * (AWQ_EUNSUPPORTED otherwise).  The weight stream is split over K across
 * the whole GPU and reduced through the workspace.
 */
int awq_gemv_w4a16(const void *x, const int32_t *qweight, const void *scales,
                   const int32_t *qzeros, void *y, int64_t M, int64_t N, int64_t K,
                   int group_size, int dtype, int split_k, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * awq_dequant_w4a16 -- the dense weight matrix W[k,n] = (q - z) * s rounded
 * once (to nearest even) to the activation dtype, [K, N] row-major: the
 * operand a dense vendor GEMM needs for the "dequantise, then call the dense
 * BLAS GEMM for long sequences" route of the [P1] TODO list.  Not used by the
 * 4-bit GEMM calls; provided for comparison and export.
 *   qweight, scales, qzeros, group_size, dtype: as awq_gemm_w4a16 (qzeros
 *   NULL = symmetric, z = 8).
 *   w: device, [K, N] fp16 or bf16, written.
 * Errors: AWQ_EINVAL, AWQ_EALIGN, AWQ_EHIP.
 */
int awq_dequant_w4a16(const int32_t *qweight, const void *scales, const int32_t *qzeros, void *w,
                      int64_t N, int64_t K, int group_size, int dtype, void *stream);

/*
 * awq_gemv_w4a16_static -- awq_gemv_w4a16 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same kernels, results and argument rules,
 * without a workspace argument.  The split-K reduction runs in a static
 * scratch array of 16 MiB (AWQ_STATIC_SCRATCH_BYTES) that each device holds
 * from the library's load until the process ends; the call itself allocates
 * and frees nothing.
 *   Its first call on a device looks up that device's copy of the array and
 *   enqueues a clear of it on `stream` ahead of the GEMV (again on each later
 *   call until one runs outside graph capture, since a clear recorded into a
 *   graph runs only with the graph).
 *   Every call on one device shares that device's array, which the kernels
 *   leave zero after each call: calls that overlap in time on one device
 *   (different streams, or a graph replayed beside an eager call) race and
 *   must be ordered by the caller.
 * Errors: as awq_gemv_w4a16 (AWQ_EUNSUPPORTED for M > 8), plus
 * AWQ_EWORKSPACE when the call's split-K reduction needs more than
 * AWQ_STATIC_SCRATCH_BYTES (awq_plan_info reports the need), and AWQ_EHIP if
 * the device or its copy of the array cannot be found.
 */
#define AWQ_STATIC_SCRATCH_BYTES (16u << 20)
int awq_gemv_w4a16_static(const void *x, const int32_t *qweight, const void *scales,
                          const int32_t *qzeros, void *y, int64_t M, int64_t N, int64_t K,
                          int group_size, int dtype, void *stream);

/*
 * w4a8_quant_act -- dynamic per-token int8 quantisation of activations
 * ([P5], the dynamic_quant helper):
 *   s1[m]   = float( act( max_k |x[m,k]| / 127 ) )
 *   a8[m,k] = clamp( round_half_even( float(x[m,k]) / s1[m] ), -128, 127 )
 * with a correctly rounded fp32 divide; act() rounds to the activation type
 * (nearest even); a row whose s1 is 0 gives a8 = 0.  [P5] defines the fp16
 * form and lists bf16 as not yet supported; for bf16 this library takes the
 * same recipe with the quotient rounded to bf16.
 *   x: device fp16 or bf16 [M, K] (dtype AWQ_DTYPE_F16 / AWQ_DTYPE_BF16);
 *   a8: device int8 [M, K]; s1: device fp32 [M].
 * Errors: AWQ_EINVAL (M, K < 1, pointers, dtype), AWQ_EALIGN, AWQ_EHIP.
 */
int w4a8_quant_act(const void *x, int8_t *a8, float *s1, int64_t M, int64_t K, int dtype, void *stream);

/*
 * w4a8_gemm -- QQQ-style W4A8 GEMM ([P5]):
 *   acc[m,n] = sum_k a8[m,k] * w8[k,n]   (exact, int32)
 *   y[m,n]   = act( acc[m,n] * s1[m] * s2[n] )   (fp32 arithmetic, RNE)
 * with w8 = q for per-channel weights (s3 == NULL, group_size == -1) and
 * w8 = q * s3[k/G, n] for per-group weights, where s3 holds small integers
 * 1..16 so that w8 stays an int8.  s2, s3 and y are in the activation type
 * `dtype` (AWQ_DTYPE_F16 or AWQ_DTYPE_BF16; acc does not depend on it).
 *   a8:       device int8 [M, K] (from w4a8_quant_act).
 *   b_packed: device int32 [K/8, N], W4A8_LAYOUT_K8 (q in -8..7).
 *   s1:       device fp32 [M];  s2: device [N];  s3: device [K/G, N] or NULL.
 *   y:        device [M, N].
 *   acc_out:  device int32 [M, N] or NULL: if given, the exact accumulators
 *             are written too (for checking).
 *   K % 64 == 0 and K <= 131008 (so that the int32 accumulator, which
 *   holds up to 2^14 * K, cannot wrap); N % 8 == 0; group_size -1
 *   (per-channel) or one of 32, 64, 128.
 * Errors: AWQ_EINVAL (also an unknown dtype), AWQ_EALIGN, AWQ_EWORKSPACE,
 * AWQ_EUNSUPPORTED (K % 64 != 0 or K > 131008), AWQ_EHIP.
 */
int w4a8_gemm(const int8_t *a8, const int32_t *b_packed, const float *s1, const void *s2,
              const void *s3, void *y, int32_t *acc_out, int64_t M, int64_t N,
              int64_t K, int group_size, int dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a8_linear -- the whole W4A8 layer in one call: w4a8_quant_act of x
 * followed by w4a8_gemm, with identical results (y, s1 and acc_out bit for
 * bit).  The pages note that quantising activations in a separate kernel
 * costs performance ([P5]); for a single token (M == 1, K <= 32768, fp16 or
 * bf16) the quantisation runs inside the GEMM kernel: every workgroup reads
 * the activation row, derives s1 and quantises its own K range into LDS, so
 * the int8 activations never travel through device memory and there is one
 * launch.  Otherwise the two steps run back to back.
 *   x:   device fp16 or bf16 [M, K] (dtype).
 *   a8:  device int8 [M, K], scratch: holds the quantised activations when
 *        the two-step path runs, left untouched by the fused path.
 *   s1:  device fp32 [M], written (the per-token scales).
 *   other arguments, layouts, workspace and errors: as w4a8_gemm.
 */
int w4a8_linear(const void *x, int8_t *a8, float *s1, const int32_t *b_packed,
                const void *s2, const void *s3, void *y, int32_t *acc_out,
                int64_t M, int64_t N, int64_t K, int group_size, int dtype, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * INT4-FP8 W4A8.  [P5] names "INT4-FP8 QQQ (W4A8)" as its authors' next step
 * and gives nothing more; this library takes the int8 recipe above with OCP
 * FP8 E4M3 activation codes (sign, 4 exponent bits biased by 7, 3 mantissa
 * bits; largest finite value 448; 0x7f and 0xff are NaN and never produced)
 * and 448 in place of the int8 codes and 127, per-channel scales only.
 *
 * w4a8_fp8_quant_act -- per-token E4M3 quantisation:
 *   s1[m]   = float( act( max_k |x[m,k]| / 448 ) )   (correctly rounded fp32
 *             divide, then rounded to the activation type)
 *   a[m,k]  = e4m3( clamp( float(x[m,k]) / s1[m], -448, 448 ) )  (fp32
 *             divide, round to nearest even); a row whose s1 is 0 gives codes 0
 *   asum[m] = float( sum_k value(a[m,k]) )  (the exact sum, rounded once; the
 *             GEMM needs it)
 *   x: device fp16/bf16 [M, K] (dtype); a: device uint8 [M, K];
 *   s1, asum: device fp32 [M].
 * Errors: AWQ_EINVAL, AWQ_EALIGN, AWQ_EHIP.
 */
int w4a8_fp8_quant_act(const void *x, uint8_t *a, float *s1, float *asum, int64_t M, int64_t K, int dtype,
                       void *stream);

/*
 * w4a8_fp8_gemm -- y[m,n] = act( acc[m,n] * s1[m] * s2[n] ) with
 * acc[m,n] = sum_k value(a[m,k]) * q[k,n], accumulated in fp32 on the fp8
 * matrix cores (not exact: compare within a tolerance).
 *   a, s1, asum: from w4a8_fp8_quant_act; b_packed: int32 [K/8, N],
 *   W4A8_LAYOUT_K8 (q in -8..7); s2: device [N] and y: device [M, N] in the
 *   activation type `dtype`; acc_out: device fp32 [M, N] or NULL (the fp32
 *   sums, for checking).
 *   K % 128 == 0 and K <= 131008; N % 8 == 0.  Workspace as for w4a8_gemm
 *   (op AWQ_OP_W4A8_FP8_GEMM in awq_workspace_bytes).
 * Errors: AWQ_EINVAL, AWQ_EALIGN, AWQ_EWORKSPACE, AWQ_EUNSUPPORTED (K), AWQ_EHIP.
 */
int w4a8_fp8_gemm(const uint8_t *a, const int32_t *b_packed, const float *s1, const float *asum,
                  const void *s2, void *y, float *acc_out, int64_t M, int64_t N, int64_t K, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * w4a8_fp8_linear -- the whole INT4-FP8 layer in one call:
 * w4a8_fp8_quant_act of x followed by w4a8_fp8_gemm.  As for w4a8_linear
 * ([P5]: quantising in a separate kernel costs performance), a single token
 * (M == 1) runs as one kernel: every workgroup reads the activation row,
 * derives s1 and quantises its own K range into LDS, and the GEMM's epilogue
 * takes each range's own sum of the codes' values, so no workgroup needs the
 * whole row's.  s1 and every code are those of w4a8_fp8_quant_act; the output
 * forms acc = 512 t - 8 asum once from the exact split-K sum, where the
 * two-launch path first rounds t to fp32 (at most one fp32 rounding of acc
 * apart; y then at most one rounding of the activation type).  Otherwise the
 * two steps run back to back.
 *   x: device fp16/bf16 [M, K] (dtype).
 *   a, asum: device uint8 [M, K] and fp32 [M], scratch: the codes and row
 *            sums when the two-step path runs, untouched by the fused path.
 *   s1: device fp32 [M], written.
 *   other arguments, layouts, workspace (op AWQ_OP_W4A8_FP8_GEMM) and errors:
 *   as w4a8_fp8_gemm.
 */
int w4a8_fp8_linear(const void *x, uint8_t *a, float *s1, float *asum, const int32_t *b_packed,
                    const void *s2, void *y, float *acc_out, int64_t M, int64_t N, int64_t K, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * awq_stream_read -- measurement helper, not a step of the method: reads
 * `bytes` bytes at `src` once (16-byte loads spread over up to 2048
 * workgroups) and writes an XOR checksum per wave to `sink`, so that the
 * achievable device-memory read rate at the size of a layer's weights can be
 * timed beside the GEMV that streams them.
 *   src:   device, 16-byte aligned, bytes > 0 and bytes % 16 == 0.
 *   sink:  device uint32 [AWQ_STREAM_SINK_WORDS], overwritten (contents are
 *          meaningless beyond keeping the loads alive).
 * Errors: AWQ_EINVAL, AWQ_EALIGN, AWQ_EHIP.
 */
#define AWQ_STREAM_SINK_WORDS 8192
int awq_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ4_H */
