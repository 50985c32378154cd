// Device-side helpers shared by the gfx950 kernels of libbfq: vector types, the e4m3fn and
// int8 element encoders, bf16/fp16 output conversion and the MFMA wrappers.
//
// Pages cited by title and section:
//   [BENCH]  "vLLM DeepGEMM FP8 Block GEMM 基准测试：DeepSeek DeepGEMM 对比 Triton 与 CUTLASS
//             的块量化 GEMM 内核解析"
//   [PR]     vLLM pull request 42153 (per_token_group_quant 2-D grid)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bfq_internal.h"

namespace bfq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr float kFp8Max = 448.0f;    // largest finite e4m3fn value
constexpr float kInt8Max = 127.0f;   // symmetric int8 range [-127, 127]

template <int QT> __device__ __forceinline__ constexpr float qmax() {
    return QT == Q_FP8 ? kFp8Max : kInt8Max;
}

// ---------------------------------------------------------------- encoders ----
// Two fp32 values -> two e4m3fn codes in the low 16 bits (a in bits 0..7, b in 8..15).
// gfx950's conversion rounds to nearest even into the OCP e4m3fn format. Callers pass only
// finite values of magnitude below 464 (the midpoint above 448), so saturation never
// matters; NaN/Inf groups are handled by the callers without this instruction.
__device__ __forceinline__ uint32_t enc_fp8x2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four fp32 values -> four e4m3fn codes packed little-endian in one word.
__device__ __forceinline__ uint32_t enc_fp8x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// fp32 -> int8 code: round half to even, clamp to [-127, 127]. Finite inputs only.
__device__ __forceinline__ uint32_t enc_i8(float y) {
    float r = __builtin_rintf(y);
    r = __builtin_fminf(__builtin_fmaxf(r, -kInt8Max), kInt8Max);
    return (uint32_t)((int)r) & 0xFFu;
}

__device__ __forceinline__ uint32_t enc_i8x4(float a, float b, float c, float d) {
    return enc_i8(a) | (enc_i8(b) << 8) | (enc_i8(c) << 16) | (enc_i8(d) << 24);
}

// ---------------------------------------------------------------- conversions ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (f != f) ? 0x7FC0u : r;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;   // RNE
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------- MFMA ----
// D(16x16, fp32) = A(16x128 e4m3) * B(128x16 e4m3). Lane l supplies row (l % 16) of A and
// column (l % 16) of B, each as 32 bytes of the 128-long K slice; both operands use the
// same K placement, so the product is the full 128-term dot product. Output: lane l holds
// D[4*(l/16) + i][l % 16], i = 0..3.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b) {
    v4f z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// The same product added to an accumulator: D = C + A * B (per-token x per-channel scales,
// where the MFMA accumulates over the whole K and the scales come after).
__device__ __forceinline__ v4f mfma_fp8_16x16x128_acc(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D(32x32, fp32) = A(32x64 e4m3) * B(64x32 e4m3) + C. Lane l supplies row (l % 32) of A and
// column (l % 32) of B, 32 bytes of the 64-long K slice each (same placement for both).
// Output: lane l holds D[8*j + 4*(l/32) + i][l % 32] in element 4*j + i (i, j = 0..3).
__device__ __forceinline__ v16f mfma_fp8_32x32x64(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same 16x16x128 product with block scales applied and accumulated by the MFMA:
// D = C + sum_k (A[i][k] * 2^(ea - 127)) * (B[k][j] * 2^(eb - 127)), where ea is the E8M0
// exponent of row i's scale and eb that of column j's (each lane passes the scale of the row
// / column it supplies; all of a row's 128 K share one scale here).
__device__ __forceinline__ v4f mfma_fp8_16x16x128_e8(const v8i& a, const v8i& b, const v4f& c,
                                                     int ea, int eb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// E8M0 exponent byte of a positive power-of-two fp32 value (its biased exponent field).
__device__ __forceinline__ uint32_t e8m0_of(float pow2) { return (__float_as_uint(pow2) >> 23) & 0xFFu; }

// Packed UE8M0 activation scales (BFQ_SCALES_PACKED_UE8M0): byte j of a 32-bit word is the
// E8M0 code of group 4w + j. Its fp32 value is 2^(code - 127): code 0 is 2^-127 (an fp32
// subnormal), 255 is NaN.
__device__ __forceinline__ uint32_t e8m0_byte(uint32_t word, int j) { return (word >> (8 * j)) & 0xFFu; }
__device__ __forceinline__ float e8m0_value(uint32_t code) {
    // branch-free: bit 22 is set exactly for code 0 (0x00400000) and code 255 (0x7FC00000)
    const uint32_t edge = ((code + 1u) >> 8) | (1u - ((code + 255u) >> 8));
    return __uint_as_float((code << 23) | (edge << 22));
}
// The activation scale of K block kb from the 32 bits loaded for it: an fp32 value, or (packed)
// the word holding the codes of blocks 4*(kb/4) .. +3.
__device__ __forceinline__ float act_scale(float bits, int packed, int64_t kb) {
    return packed ? e8m0_value(e8m0_byte(__float_as_uint(bits), (int)(kb & 3))) : bits;
}
__device__ __forceinline__ int act_scale_e8(float bits, int packed, int64_t kb) {
    return packed ? (int)e8m0_byte(__float_as_uint(bits), (int)(kb & 3)) : (int)e8m0_of(bits);
}

// int8: D(16x16, int32) += A(16x64) * B(64x16); 16 bytes of K per lane.
__device__ __forceinline__ v4i mfma_i8_16x16x64(const v4i& a, const v4i& b, const v4i& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- buffer access ----
// Raw buffer resource over [base, base + bytes): loads whose offset (per-lane voffset plus
// scalar soffset; on gfx950 both count) reaches `bytes` return zero, which the GEMM kernels
// use for rows beyond M or N. bytes < 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds_base + lds_off + 16 * l (lds_off wave-uniform). voff per lane, soff uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base,
                                      uint32_t lds_off, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(lds_base + lds_off), 16, voff, soff, 0, 0);
}

// 4 bytes per lane into LDS (lane l -> lds_base + lds_off + 4 l): used to touch lines ahead.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base,
                                     uint32_t lds_off, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(lds_base + lds_off), 4, voff, soff, 0, 0);
}

// Cache-policy operand of the buffer intrinsics: "nt" (non-temporal, streamed once).
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// 16 bytes per lane between registers and a buffer (loads past the end return zero).
__device__ __forceinline__ v4f buf_load_v4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store_v4f(__amdgpu_buffer_rsrc_t r, v4f v, uint32_t voff,
                                              uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, voff, soff, 0);
}

// ---------------------------------------------------------------- LDS DMA ----
// 16 bytes per lane from global memory straight into LDS: the wave writes 1 KB at
// lds_base + lane * 16 (lds_base must be wave-uniform).
__device__ __forceinline__ void load_lds_16(const void* gsrc, uint8_t* lds_base, uint32_t off) {
    const uint32_t u = __builtin_amdgcn_readfirstlane(off);
    __builtin_amdgcn_global_load_lds(gsrc, lds_base + u, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory operations remain outstanding (they complete in issue
// order, so everything but the N most recent has landed).
template <int N> __device__ __forceinline__ void wait_vmem_keep_n() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
#define wait_vmem_keep(N) wait_vmem_keep_n<(N)>()

// A workgroup-uniform 64-bit value, stated as such (kept in scalar registers).
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// MoE grouped GEMM: the grid's row-tile index t walks the per-expert tiles (ceil(rows_e / bm)
// per expert, experts in order). moe_tile maps t to expert e and grouped rows [p0, p1) by a
// wave-wide prefix sum over 64 experts at a time; every wave computes the same result
// (wave-uniform, held in scalar registers). False when t is past the last tile.
struct MoeSpan {
    int64_t e, p0, p1;
};
// The offsets are clamped to a non-decreasing sequence in [0, pairs], so rows [p0, p1) always
// index inside the pair list whatever the offsets hold.
__device__ __forceinline__ bool moe_tile(const int32_t* __restrict__ offsets, int E, int64_t pairs,
                                         int bm, int64_t t, MoeSpan& sp) {
    const int lane = threadIdx.x & 63;
    const int32_t P = (int32_t)pairs;
    int64_t before = 0;
    for (int c = 0; c < E; c += 64) {
        const int e = c + lane;
        int32_t a = 0, b = 0;
        if (e < E) {
            a = min(max(offsets[e], 0), P);
            b = min(max(offsets[e + 1], a), P);
        }
        const int32_t tiles = (b - a + bm - 1) / bm;
        int32_t inc = tiles;                       // inclusive prefix over the 64 lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t v = __shfl_up(inc, d, 64);
            if (lane >= d) inc += v;
        }
        const int32_t total = __shfl(inc, 63, 64);
        if (t < before + total) {
            const int32_t r = (int32_t)(t - before);
            const int L = __builtin_ctzll(__ballot(inc > r));
            const int32_t incL = __shfl(inc, L, 64), tilesL = __shfl(tiles, L, 64);
            const int32_t aL = __shfl(a, L, 64), bL = __shfl(b, L, 64);
            const int64_t p0 = (int64_t)aL + (int64_t)(r - (incL - tilesL)) * bm;
            sp.e = uniform_i64(c + L);
            sp.p0 = uniform_i64(p0);
            sp.p1 = uniform_i64(p0 + bm < bL ? p0 + bm : bL);
            return true;
        }
        before += total;
    }
    return false;
}


// ---------------------------------------------------------------- tile order, LDS swizzle ----
// Tile id -> (pid_m, pid_n). raster 0: workgroup ids are dealt round-robin to the 8 XCDs, so
// ids are first remapped to give each XCD a contiguous range of tiles; raster 1: no remap.
// Then the grouped order: GROUP_M tile rows at a time, column by column within the group.
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                            int group_m, int raster, int64_t& pid_m,
                                            int64_t& pid_n) {
    const int64_t T = tiles_m * tiles_n;
    int64_t j = bid;
    if (raster == 0) {
        const int64_t xcd = bid & 7, local = bid >> 3;
        const int64_t base = T >> 3, rem = T & 7;
        j = xcd * base + (xcd < rem ? xcd : rem) + local;
    }
    const int64_t per_group = (int64_t)group_m * tiles_n;
    const int64_t gid = j / per_group;
    const int64_t first_m = gid * group_m;
    const int64_t gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int64_t in_group = j - gid * per_group;
    pid_m = first_m + in_group % gsize;
    pid_n = in_group / gsize;
}

// LDS slot of 16-byte chunk c in region row r: c ^ swz(r). Fragment reads touch 16
// consecutive rows (a multiple of 16 apart) at one chunk index; with this swizzle those 16
// reads hit 16 distinct (row parity, slot) pairs, i.e. distinct banks whether the LDS serves
// 8 lanes x 16 B or 16 lanes x 16 B per cycle. It depends only on r & 15.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// ---------------------------------------------------------------- output store ----
// Store four consecutive output values of one row.
template <int OT> __device__ __forceinline__ void store4(void* out, int64_t idx, v4f v) {
    if constexpr (OT == O_FP32) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + idx) = v;
    } else {
        uint32_t b0, b1, b2, b3;
        if constexpr (OT == O_BF16) {
            b0 = f32_to_bf16_bits(v.x); b1 = f32_to_bf16_bits(v.y);
            b2 = f32_to_bf16_bits(v.z); b3 = f32_to_bf16_bits(v.w);
        } else {
            b0 = f32_to_f16_bits(v.x); b1 = f32_to_f16_bits(v.y);
            b2 = f32_to_f16_bits(v.z); b3 = f32_to_f16_bits(v.w);
        }
        uint2 p;
        p.x = b0 | (b1 << 16);
        p.y = b2 | (b3 << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + idx) = p;
    }
}

}  // namespace bfq
