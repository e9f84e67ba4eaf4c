// device.hpp -- gfx950 device helpers for the 4-bit-weight kernels.
//
// Packed-word facts used here (first-generation AWQ GEMM format, vLLM pull
// request "Speed up AWQ 2.5x with updated kernel", list of format
// differences): a 32-bit word packs eight output columns 8j..8j+7 of one
// k-row; nibble i holds column 8j + {0,2,4,6,1,3,5,7}[i].  Hence byte b of a
// word holds columns (0,2), (4,6), (1,3), (5,7) for b = 0..3 (low nibble
// first), and the zero-point word of a group uses the same map.
//
// Matrix-core operand model (v_mfma_*_16x16x32 / 16x16x64): lane l supplies
// row (A) or column (B) l % 16 and a chunk of the reduction index chosen by
// l / 16; C lane l holds rows 4*(l/16) + r, r = 0..3, of column l % 16.  The
// reduction index order inside a lane is free as long as A and B agree, so
// the kernels assign lane group g = l/16 the consecutive k range g*8..g*8+7
// (fp16/bf16) or g*16..g*16+15 (int8) of each step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace awq4 {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// f(std::integral_constant<int, 0>) ... f(std::integral_constant<int, N - 1>),
// in order: a loop whose index is a compile-time constant in every body
// (guaranteed unrolling, `if constexpr` on the index).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T, typename F>
__device__ __forceinline__ T bit_as(F v) {
    static_assert(sizeof(T) == sizeof(F), "size mismatch");
    return __builtin_bit_cast(T, v);
}

// v_perm_b32: result byte i = byte sel[i] of the 8-byte value {hi:lo}
// (selector 0..3 = bytes of lo, 4..7 = bytes of hi).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Interleave two words of the same 8 columns at consecutive k (lo = k even,
// hi = k odd) so that each 16-bit half holds one k:
//   pair_x -> halves hold nibbles of columns {0,2,4,6} (bytes 0,1 of each word)
//   pair_y -> halves hold nibbles of columns {1,3,5,7} (bytes 2,3 of each word)
__device__ __forceinline__ uint32_t pair_x(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_y(uint32_t lo, uint32_t hi) { return perm_b32(hi, lo, 0x07060302u); }

// Where column t (0..7) of a word sits after pair_x / pair_y:
//   source  = pair_y if t is odd, else pair_x
//   pos     = t >> 1 : nibble position inside each 16-bit half
//   shift   = 8 for pos 2,3 (upper byte of the half), else 0
//   hi      = pos is odd (upper nibble of that byte)
// and the nibble index of column t inside a (zero-point) word.
__host__ __device__ constexpr int col_src_y(int t) { return t & 1; }
__host__ __device__ constexpr int col_shift(int t) { return ((t >> 1) & 2) ? 8 : 0; }
__host__ __device__ constexpr int col_hi(int t) { return (t >> 1) & 1; }
__host__ __device__ constexpr int col_nibble(int t) { return (t >> 1) + 4 * (t & 1); }

// ---------------------------------------------------------------------------
// fp16 dequantisation of two k-values of one column, exact up to the final
// multiply by the scale (one rounding, to nearest even):
//   lo nibble: as_f16(0x6400 | q) = 1024 + q;     (1024 + q) - (1024 + z) = q - z
//   hi nibble: as_f16(0x6400 | 16q) = 1024 + 16q; (1024 + 16q)/16 - (64 + z) = q - z
// zc holds -(1024 + z) or -(64 + z) in both halves; sc holds s in both halves.
template <int HI>
__device__ __forceinline__ uint32_t dq_f16(uint32_t v, uint32_t zc, uint32_t sc) {
    const uint32_t mask = HI ? 0x00F000F0u : 0x000F000Fu;
    f16x2 h = bit_as<f16x2>((v & mask) | 0x64006400u);
    f16x2 z = bit_as<f16x2>(zc);
    f16x2 d;
    if (HI) {
        const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
        d = h * sixteenth + z;
    } else {
        d = h + z;
    }
    return bit_as<uint32_t>(d * bit_as<f16x2>(sc));
}

// fp16 zero-point constant for column t from the group's zero nibble z.
template <int HI>
__device__ __forceinline__ uint32_t zconst_f16(uint32_t z) {
    uint32_t h = HI ? (0xD400u | (z << 4)) : (0xE400u | z);  // -(64+z) or -(1024+z)
    return h | (h << 16);
}

// bf16 dequantisation of two k-values of one column, computed exactly in
// fp32 and rounded once:  q*s' - z*s  with s' = s (lo nibble) or s/16 (hi
// nibble, whose byte holds 16q).  Returns the bf16 pair (even k low half).
__device__ __forceinline__ uint32_t dq_bf16(uint32_t v, uint32_t mask, float s_eff, float zs) {
    uint32_t m = v & mask;
    float q0 = (float)(m & 0xFFu);          // v_cvt_f32_ubyte0
    float q1 = (float)((m >> 16) & 0xFFu);  // v_cvt_f32_ubyte2
    float w0 = __builtin_fmaf(q0, s_eff, -zs);
    float w1 = __builtin_fmaf(q1, s_eff, -zs);
    __bf16 b0 = (__bf16)w0;
    __bf16 b1 = (__bf16)w1;
    return (uint32_t)bit_as<uint16_t>(b0) | ((uint32_t)bit_as<uint16_t>(b1) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return bit_as<float>(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) { return (float)bit_as<f16>((uint16_t)b); }

template <int DT>
__device__ __forceinline__ float act_bits_to_f32(uint32_t b) {
    return DT == DT_F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

__device__ __forceinline__ uint16_t f32_to_out_bits(float v, int dt) {
    if (dt == DT_BF16) return bit_as<uint16_t>((__bf16)v);
    return bit_as<uint16_t>((f16)v);
}

// Two fp32 values as one 64-bit word (x in the low half), for 64-bit atomics.
__device__ __forceinline__ uint64_t pack_f32x2(float2 v) {
    return (uint64_t)bit_as<uint32_t>(v.x) | ((uint64_t)bit_as<uint32_t>(v.y) << 32);
}
__device__ __forceinline__ float2 unpack_f32x2(uint64_t w) {
    return make_float2(bit_as<float>((uint32_t)w), bit_as<float>((uint32_t)(w >> 32)));
}

// ---------------------------------------------------------------------------
// Direct global -> LDS copies of 16 bytes per lane: lane i of the wave writes
// bytes [16 i, 16 i + 16) after the LDS address `dst` of the first active
// lane (M0).
//
// They are issued from inline assembly on purpose.  The compiler's own form
// of these copies (the global_load_lds / buffer_load_lds builtins) cannot
// tell which LDS bytes a copy writes, so it waits for every copy in flight
// before any later LDS read: a copy issued for the next pipeline stage then
// stalls the reads of the current one for a whole memory latency.  The
// compiler does not see these copies at all, so the code that reads their
// data waits for them itself (wait_vm_all(), then a workgroup barrier).  Its
// own vector-memory waits stay correct: loads complete in issue order, and a
// wait computed without the hidden copies only waits for more of them.
// M0 takes the first active lane's address (as the compiler's own copies do)
__device__ __forceinline__ uint32_t lds_address(const void *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}
// from a global address (per lane)
__device__ __forceinline__ void dma16(const void *src, void *dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_address(dst)), "v"(src)
                 : "memory", "m0");
}
// through a buffer descriptor: address = base + voff (per lane) + soff
// (wave-uniform); offsets past the descriptor's size read as zero
constexpr int kBufDword3 = 0x00020000;  // raw 32-bit buffer, no format conversion
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, kBufDword3);
}
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void *dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_address(dst)), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}
// Wait until every vector-memory load of this wave has landed (the direct
// LDS copies included).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8
// XCDs (workgroup i of a launch runs on XCD i % 8), and each XCD has its own
// L2.  Tile `tile_of_xcd_order(i, T)` gives XCD x a contiguous run of the T
// tiles (in row-major tile order, so the workgroups of one XCD share X row
// blocks in that XCD's L2) instead of every eighth tile.  A bijection of
// 0..T-1 for any T.
constexpr int kXcds = 8;
__device__ __forceinline__ int tile_of_xcd_order(int i, int T) {
    const int x = i % kXcds, l = i / kXcds;
    const int q = T / kXcds, r = T % kXcds;
    return x * q + min(x, r) + l;
}

// ---------------------------------------------------------------------------
// int8 B operand (16 consecutive k of one column) from two consecutive K8
// words.  Nibble i of a K8 word holds k = [0,4,1,5,2,6,3,7][i], so the low
// nibbles of its four bytes are k 0..3 and the high nibbles k 4..7.
//  per-channel: bytes = 16*q (the x16 is divided out of the int32 result);
//               two instructions per word.
//  per-group:   bytes = q*s3 with s3 in 1..16.  With u = q + 8 in 0..15,
//               u*s3 + (128 - 8*s3) lies in 0..240 per byte, so a packed
//               16-bit multiply-add forms two bytes per half with no carry
//               between them (full-rate, unlike a 32-bit multiply); flipping
//               bit 7 then subtracts 128.
template <bool GROUP>
__device__ __forceinline__ u32x4 int8_b_operand(uint32_t w0, uint32_t w1, uint32_t s3) {
    u32x4 b;
    if (!GROUP) {
        b[0] = (w0 << 4) & 0xF0F0F0F0u;
        b[1] = w0 & 0xF0F0F0F0u;
        b[2] = (w1 << 4) & 0xF0F0F0F0u;
        b[3] = w1 & 0xF0F0F0F0u;
    } else {
        const u16x2 sv = {(uint16_t)s3, (uint16_t)s3};
        const u16x2 cv = (u16x2){0x8080, 0x8080} - sv * (u16x2){0x0808, 0x0808};
        auto bytes = [&](uint32_t u) { return bit_as<uint32_t>(bit_as<u16x2>(u) * sv + cv) ^ 0x80808080u; };
        const uint32_t u0 = w0 ^ 0x88888888u, u1 = w1 ^ 0x88888888u;
        b[0] = bytes(u0 & 0x0F0F0F0Fu);
        b[1] = bytes((u0 >> 4) & 0x0F0F0F0Fu);
        b[2] = bytes(u1 & 0x0F0F0F0Fu);
        b[3] = bytes((u1 >> 4) & 0x0F0F0F0Fu);
    }
    return b;
}

// ---------------------------------------------------------------------------
// Matrix-core wrappers.
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_as<f16x8>(a), bit_as<f16x8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_as<bf16x8>(a), bit_as<bf16x8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(bit_as<i32x4>(a), bit_as<i32x4>(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Split-K completion with one counting atomic per output element.
//
// Every output element of a split-K launch owns one 64-bit accumulator in the
// workspace (zero between calls):
//   bits 63..56  number of contributions received so far
//   bits 55..0   sum over the contributions of (value + kBias)
// A contribution adds (1 << 56) + value + kBias with 0 <= value + kBias < 2^48,
// so up to 255 contributions never carry into the count.  The add is a
// device-scope read-modify-write atomic returning the old word; the
// contribution that brings the count to S therefore holds the exact total
// (old + its own add), writes the output, and clears the accumulator for the
// next call.  Only single-location atomicity is relied on -- no fences, no
// separate counters -- and the integer sum does not depend on the order of
// arrival, so every run gives the same bits.  fp32 partials are converted to
// fixed point first; int32 partials are used as they are.

constexpr int kCountShift = 56;
constexpr uint64_t kValueMask = (uint64_t(1) << kCountShift) - 1;
constexpr int64_t kBias = int64_t(1) << 47;
constexpr int kMaxSplits = 255;

// Fixed-point resolution: fp16 outputs (|y| <= 65504) use 2^-28 with range
// 2^19; bf16 outputs use 2^-16 with range 2^31.
template <int DT>
struct FixedPoint {
    static constexpr double kScale = DT == DT_BF16 ? 65536.0 : 268435456.0;
};

template <int DT>
__device__ __forceinline__ int64_t to_fixed(float v) {
    const double lim = (double)(kBias - 1);
    double d = (double)v * FixedPoint<DT>::kScale;
    d = fmin(fmax(d, -lim), lim);
    return (int64_t)__builtin_rint(d);
}

template <int DT>
__device__ __forceinline__ float from_fixed(int64_t v) {
    return (float)((double)v * (1.0 / FixedPoint<DT>::kScale));
}

// Adds one contribution (value in -kBias+1 .. kBias-1) to *acc.  Returns true
// in the final contribution, with the exact total in *total.
__device__ __forceinline__ bool splitk_contribute(uint64_t *acc, int64_t value, int S, int64_t *total) {
    const uint64_t add = (uint64_t(1) << kCountShift) + (uint64_t)(value + kBias);
    const uint64_t old = __hip_atomic_fetch_add(acc, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t now = old + add;
    if ((int)(now >> kCountShift) != S) return false;
    *total = (int64_t)(now & kValueMask) - (int64_t)S * kBias;
    __hip_atomic_store(acc, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// ---------------------------------------------------------------------------
// Split-K by partial tiles, for the GEMM kernels: their outputs have far too
// many elements for one device-scope atomic each.  Workspace layout: one
// uint32 arrival counter per output tile (rounded up to 256 bytes), then fp32
// or int32 partials [S][M][N]; all zero between calls.
//
// Per workgroup: every thread stores its partial elements of the tile into
// slot `split` with agent-scope atomic stores, which go through to the
// device-wide coherence point themselves; split_tile_last_atomic() then waits
// until every store of the workgroup has completed and counts the tile's
// arrival with one atomic.  The workgroup that completes the count returns
// true: it reads the partials with agent-scope atomic loads (issued after it
// has seen the count, through the barrier), which do not read stale L2
// lines, sums them for each of its elements in split order (so the result
// does not depend on which split arrives last), writes the output and zeroes
// every partial of the tile; the counter is re-armed at once.  One atomic per
// workgroup, against one per output element and split, and no fence: an
// agent-scope release fence writes back the issuing XCD's whole L2 (the
// write-back plain stores would need before other XCDs could read them), and
// one per workgroup measured several times the kernels' own time -- 4-5x on
// a ~1000-workgroup decode launch, and more than a K split saves in the GEMMs.
// (The workspace sizes, split_counters_bytes / split_tiles_bytes, are in
// launch.hpp, shared with the host-side planner.)
__device__ __forceinline__ bool split_tile_last_atomic(uint32_t *cnt, int S) {
    __shared__ uint32_t last_flag;
    wait_vm_all();    // this thread's partial stores have completed
    __syncthreads();  // ... and every other thread's
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t last = old == (uint32_t)(S - 1) ? 1u : 0u;
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = last;
    }
    __syncthreads();
    return last_flag != 0;
}

// Buffer cache-policy operand for split partials: sc1, the policy of the
// agent-scope atomic loads and stores above (through to the device-wide
// coherence point), for 16-byte accesses that atomics do not offer.
constexpr int kPartCoherent = 16;

// The value of the same register in the other lane of the pair (lane ^ 1).
__device__ __forceinline__ float lane_pair_swap(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

// Four fp32 outputs as the activation type, packed for one 8-byte store.
template <int DT>
__device__ __forceinline__ uint2 quad_out_bits(f32x4 t) {
    return make_uint2((uint32_t)f32_to_out_bits(t[0], DT) | ((uint32_t)f32_to_out_bits(t[1], DT) << 16),
                      (uint32_t)f32_to_out_bits(t[2], DT) | ((uint32_t)f32_to_out_bits(t[3], DT) << 16));
}

// Partial tiles of 16-byte vectors (4 int32 or 4 fp32) for the exchange
// above: each vector moves as two 64-bit agent-scope atomics (p 8-byte
// aligned).  part_sum adds, in split order, the S partials of R vectors
// (addr(s, i) = the uint64_t address of vector i of split s; vectors with
// !valid(i) are skipped and left zero), with the loads of kB splits in
// flight together (four unless a kernel's register budget asks for fewer):
// one memory round trip per kB splits rather than one per split.  The +0 terms that pad the last batch change no sum: the running
// sums start at +0 and so are never -0.  part_clear_all then zeroes every
// partial read, which leaves the workspace as the next call expects it.
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
template <typename V>
__device__ __forceinline__ void part_put(uint64_t *p, V v) {
    const u64x2 w = bit_as<u64x2>(v);
    __hip_atomic_store(p, w[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, w[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V part_get(uint64_t *p) {
    u64x2 w;
    w[0] = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w[1] = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return bit_as<V>(w);
}
template <int R, int kB = 4, typename V, typename Addr, typename Valid>
__device__ __forceinline__ void part_sum(V (&v)[R], int S, Addr addr, Valid valid) {
#pragma unroll
    for (int i = 0; i < R; ++i) v[i] = V{};
    for (int s0 = 0; s0 < S; s0 += kB) {
        V b[kB][R];
#pragma unroll
        for (int k = 0; k < kB; ++k)
#pragma unroll
            for (int i = 0; i < R; ++i) b[k][i] = s0 + k < S && valid(i) ? part_get<V>(addr(s0 + k, i)) : V{};
#pragma unroll
        for (int k = 0; k < kB; ++k)
#pragma unroll
            for (int i = 0; i < R; ++i) v[i] += b[k][i];
    }
}
template <int R, typename Addr, typename Valid>
__device__ __forceinline__ void part_clear_all(int S, Addr addr, Valid valid) {
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < R; ++i)
            if (valid(i)) {
                uint64_t *p = addr(s, i);
                __hip_atomic_store(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(p + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
}

}  // namespace awq4
