// Quantization kernels for gfx950: per-token-group activation quantization (bf16 -> e4m3fn
// or int8 codes + one fp32 scale per 1x128 group, optionally rounded up to a power of two),
// per-128x128-block weight quantization
// (fp32 -> codes + one fp32 scale per block), one-scale-per-row quantization (per token or
// per output channel), the weight-code packing into the 16-row fragment layout, and the
// element-encoder probe used by tests.
//
// Pages cited by title and section:
//   [BENCH] "vLLM DeepGEMM FP8 Block GEMM 基准测试 ..." §4.1 (per_token_group_quant_fp8,
//           per_block_cast_to_fp8: scale = amax / fp8_max per group or block)
//   [PR]    vLLM pull request 42153 — what the group kernel is parameterised by (group size,
//           eps, min/max code) and its point that index arithmetic should be compile-time
//           constants rather than runtime divisions.
//   [HELION] "Building a High-Performance and Portable vLLM Linear Backend with Helion",
//           scope section (per-token activation and per-channel weight scales).
//
// Group kernel layout (wave64): 16 lanes own one 128-element group, 8 bf16 (16 bytes) per
// lane, so one wave covers 4 groups of one token row per pass and each 16-byte load is
// fully coalesced. The group's absolute maximum is formed on the raw bf16 bits
// (|x| = bits & 0x7FFF; as unsigned integers NaN > Inf > every finite magnitude), which
// makes a NaN anywhere in the group win the reduction, then reduced over the 16 lanes.
#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

constexpr int kQuantWaves = 4;        // waves per workgroup
constexpr int kQuantPasses = 2;       // 4-group passes per wave (loads issued together)
constexpr int kGroupsPerWave = 4 * kQuantPasses;
constexpr int kGroupsPerBlock = kQuantWaves * kGroupsPerWave;

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 x = __builtin_bit_cast(us2, a), y = __builtin_bit_cast(us2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Encode 8 values x[0..7] divided by scale s; finite-amax groups only (|x| <= amax of the
// group or row that s was formed from). The quotient is taken as q = x * r with r = 1 / s,
// one IEEE division per lane instead of one per value, then corrected once by the exact
// remainder e = x - q * s (a fused multiply-add): q + e * r, with the sign of x (the
// correction never changes the sign of a nonzero value; it restores -0, which q + e * r would
// turn into +0). For every finite bf16 amax and every bf16 x with |x| <= amax, with fp32 or
// power-of-two scales and either code type, the code of this value equals the code of the
// IEEE quotient x / s (checked exhaustively on the CPU: tests/native/quotient_codes.c); where
// the two fp32 values differ at all (subnormal x in a group whose amax is below eps) both
// encode to zero. (r names the return value below; rs is the reciprocal.)
template <int QT>
__device__ __forceinline__ uint2 encode8(const float* x, float s) {
    const float rs = 1.0f / s;                         // IEEE division, once per lane
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = x[i] * rs;
        const float e = __builtin_fmaf(-q, s, x[i]);   // exact
        y[i] = __builtin_copysignf(__builtin_fmaf(e, rs, q), x[i]);
    }
    uint2 r;
    if constexpr (QT == Q_FP8) {
        r.x = enc_fp8x4(y[0], y[1], y[2], y[3]);
        r.y = enc_fp8x4(y[4], y[5], y[6], y[7]);
    } else {
        r.x = enc_i8x4(y[0], y[1], y[2], y[3]);
        r.y = enc_i8x4(y[4], y[5], y[6], y[7]);
    }
    return r;
}

// Groups whose amax is Inf or NaN. NaN amax: every code is NaN (0x7F) / 0 (int8).
// Inf amax: the scale is Inf, finite values divide to a signed zero, +-Inf to NaN.
template <int QT>
__device__ __forceinline__ uint2 encode8_special(const float* x, bool nan_group) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t code;
        if (nan_group || __builtin_isinf(x[i])) code = (QT == Q_FP8) ? 0x7Fu : 0u;
        else code = (QT == Q_FP8) ? ((__float_as_uint(x[i]) >> 24) & 0x80u) : 0u;
        b[i] = code;
    }
    uint2 r;
    r.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    r.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return r;
}

// UE8M0 scale format ([BENCH] §4.1, use_ue8m0): the smallest power of two >= s, for a
// positive normal fp32 s (s >= eps / Qmax keeps it normal; s <= FLT_MAX / 127 keeps the
// next power finite). A power of two stays; otherwise the mantissa is cleared and the
// exponent stepped up by one.
__device__ __forceinline__ float pow2_ceil(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x007FFFFFu) ? __uint_as_float((u & 0xFF800000u) + 0x00800000u) : s;
}

// packed != 0 (BFQ_SCALES_PACKED_UE8M0, UE8M0 scales): instead of one fp32 per group, the
// E8M0 codes of groups 4w .. 4w+3 go to one 32-bit word at words[w * s_stride_g + m]. A
// wave's pass covers exactly such a quartet (groups g0 + 4u, g0 a multiple of 4 in lane 0),
// so the word is assembled with two cross-lane ORs. The grid then also covers the padding
// rows M .. round_up(M, 4) - 1, which read nothing and write zero words.
template <int QT>
__global__ __launch_bounds__(64 * kQuantWaves) void quant_tokens_kernel(
    const uint4* __restrict__ x, uint2* __restrict__ q, float* __restrict__ scales,
    int64_t M, int64_t K, int64_t G, int64_t s_stride_m, int64_t s_stride_g, float eps,
    int ue8m0, int packed) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m = blockIdx.x;
    const bool row_live = m < M;                        // false only for packed padding rows
    const int part = lane & 15;                         // 16-byte slice within the group
    const int64_t g0 = (int64_t)blockIdx.y * kGroupsPerBlock + wave * kGroupsPerWave + (lane >> 4);

    uint4 raw[kQuantPasses];
#pragma unroll
    for (int u = 0; u < kQuantPasses; ++u) {
        int64_t g = g0 + 4 * u;
        if (g < G && row_live) raw[u] = x[(m * K + g * 128) / 8 + part];
        else raw[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kQuantPasses; ++u) {
        int64_t g = g0 + 4 * u;
        uint32_t mx = max_u16x2(max_u16x2(raw[u].x & 0x7FFF7FFFu, raw[u].y & 0x7FFF7FFFu),
                                max_u16x2(raw[u].z & 0x7FFF7FFFu, raw[u].w & 0x7FFF7FFFu));
        mx = max(mx & 0xFFFFu, mx >> 16);
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 8, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 4, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, 16));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, 16));
        if (packed) {
            // every lane of the wave takes part in the ORs; lane 0 stores the quartet's word
            uint32_t code = 0;
            if (g < G && row_live) {
                float sp;
                if (mx < 0x7F800000u >> 16) {
                    const float amax = __uint_as_float(mx << 16);
                    sp = pow2_ceil((amax > eps ? amax : eps) / qmax<QT>());
                } else {
                    sp = __uint_as_float(0x7FC00000u);   // NaN or Inf group: E8M0 has no Inf
                }
                code = e8m0_of(sp);
            }
            uint32_t word = code << (8 * (lane >> 4));
            word |= (uint32_t)__shfl_xor((int)word, 16, 64);
            word |= (uint32_t)__shfl_xor((int)word, 32, 64);
            if (lane == 0 && g < G) scales[(g >> 2) * s_stride_g + m] = __uint_as_float(word);
        }
        if (g >= G || !row_live) continue;

        float xv[8] = {bf16_lo(raw[u].x), bf16_hi(raw[u].x), bf16_lo(raw[u].y), bf16_hi(raw[u].y),
                       bf16_lo(raw[u].z), bf16_hi(raw[u].z), bf16_lo(raw[u].w), bf16_hi(raw[u].w)};
        float s;
        uint2 codes;
        if (mx < 0x7F80u) {                              // finite amax
            float amax = __uint_as_float(mx << 16);
            s = (amax > eps ? amax : eps) / qmax<QT>();
            if (ue8m0) s = pow2_ceil(s);
            codes = encode8<QT>(xv, s);
        } else {
            bool nan_group = mx > 0x7F80u;
            s = nan_group ? __uint_as_float(0x7FC00000u) : __uint_as_float(0x7F800000u);
            codes = encode8_special<QT>(xv, nan_group);
        }
        q[(m * K + g * 128) / 8 + part] = codes;
        if (part == 0 && !packed) scales[m * s_stride_m + g * s_stride_g] = s;
    }
}

// One workgroup per 128x128 weight block; 256 threads, 64 values each.
template <int QT>
__global__ __launch_bounds__(256) void quant_weight_blocks_kernel(
    const float* __restrict__ w, uint8_t* __restrict__ q, float* __restrict__ scales,
    int64_t N, int64_t K, float eps, int ue8m0) {
    const int64_t nb = blockIdx.y, kb = blockIdx.x, KB = K / 128;
    const int t = threadIdx.x;
    const int col4 = t & 31;          // float4 column within the 128-wide block row
    const int row0 = t >> 5;          // 8 rows per pass, 16 passes
    (void)N;
    __shared__ uint32_t red[4];

    float4 v[16];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int64_t r = nb * 128 + row0 + 8 * i;
        v[i] = *reinterpret_cast<const float4*>(w + r * K + kb * 128 + col4 * 4);
        mx = max(mx, __float_as_uint(v[i].x) & 0x7FFFFFFFu);
        mx = max(mx, __float_as_uint(v[i].y) & 0x7FFFFFFFu);
        mx = max(mx, __float_as_uint(v[i].z) & 0x7FFFFFFFu);
        mx = max(mx, __float_as_uint(v[i].w) & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));

    float s;
    const bool finite = mx < 0x7F800000u;
    const bool nan_block = mx > 0x7F800000u;
    if (finite) {
        float amax = __uint_as_float(mx);
        s = (amax > eps ? amax : eps) / qmax<QT>();
        if (ue8m0) s = pow2_ceil(s);
    } else {
        s = nan_block ? __uint_as_float(0x7FC00000u) : __uint_as_float(0x7F800000u);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int64_t r = nb * 128 + row0 + 8 * i;
        float e[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t word;
        if (finite) {
            float y0 = e[0] / s, y1 = e[1] / s, y2 = e[2] / s, y3 = e[3] / s;
            word = (QT == Q_FP8) ? enc_fp8x4(y0, y1, y2, y3) : enc_i8x4(y0, y1, y2, y3);
        } else {
            word = 0;
            for (int j = 0; j < 4; ++j) {
                uint32_t c;
                if (nan_block || __builtin_isinf(e[j])) c = (QT == Q_FP8) ? 0x7Fu : 0u;
                else c = (QT == Q_FP8) ? ((__float_as_uint(e[j]) >> 24) & 0x80u) : 0u;
                word |= c << (8 * j);
            }
        }
        *reinterpret_cast<uint32_t*>(q + r * K + kb * 128 + col4 * 4) = word;
    }
    if (t == 0) scales[nb * KB + kb] = s;
}

template <int QT>
__global__ __launch_bounds__(256) void debug_encode_kernel(const float* __restrict__ x,
                                                           uint8_t* __restrict__ out, int64_t n) {
    int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= n) {
        float4 v = *reinterpret_cast<const float4*>(x + i);
        uint32_t w = (QT == Q_FP8) ? enc_fp8x4(v.x, v.y, v.z, v.w) : enc_i8x4(v.x, v.y, v.z, v.w);
        *reinterpret_cast<uint32_t*>(out + i) = w;
    } else {
        for (int64_t j = i; j < n; ++j)
            out[j] = (uint8_t)((QT == Q_FP8) ? enc_fp8x2(x[j], 0.0f) : enc_i8(x[j]));
    }
}

// One scale per row ([HELION] scope section: FP8_Dynamic / W8A8_INT8 quantize activations per
// token and weights per output channel): one 256-thread workgroup per row, which it reads
// once into registers as 16-byte chunks (8 bf16 or 4 fp32 values; chunk c of the row is
// held by thread c % 256 in slot c / 256), reduces the row's absolute maximum on the raw
// bits (NaN > Inf > finite, as in the group kernel) over the workgroup, and encodes from
// registers. P slots per thread bound K: P * 256 * (8 or 4) elements.
template <int IS_F32, int QT, int P>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint4* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scales, int64_t K,
    int64_t s_stride, float eps, int ue8m0) {
    constexpr int E = IS_F32 ? 4 : 8;                  // values per 16-byte chunk
    const int t = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int64_t chunks = K / E;
    __shared__ uint32_t red[4];

    uint4 raw[P];
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int64_t c = (int64_t)u * 256 + t;
        raw[u] = c < chunks ? x[r * chunks + c] : make_uint4(0, 0, 0, 0);
        if constexpr (IS_F32) {
            mx = max(mx, max(max(raw[u].x & 0x7FFFFFFFu, raw[u].y & 0x7FFFFFFFu),
                             max(raw[u].z & 0x7FFFFFFFu, raw[u].w & 0x7FFFFFFFu)));
        } else {
            const uint32_t m2 = max_u16x2(max_u16x2(raw[u].x & 0x7FFF7FFFu, raw[u].y & 0x7FFF7FFFu),
                                          max_u16x2(raw[u].z & 0x7FFF7FFFu, raw[u].w & 0x7FFF7FFFu));
            mx = max(mx, max(m2 & 0xFFFFu, m2 >> 16));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));

    // bf16 magnitudes widen to fp32 bit patterns by a 16-bit shift
    const uint32_t mxf = IS_F32 ? mx : mx << 16;
    const bool finite = mxf < 0x7F800000u, nan_row = mxf > 0x7F800000u;
    float s;
    if (finite) {
        const float amax = __uint_as_float(mxf);
        s = (amax > eps ? amax : eps) / qmax<QT>();
        if (ue8m0) s = pow2_ceil(s);
    } else {
        s = nan_row ? __uint_as_float(0x7FC00000u) : __uint_as_float(0x7F800000u);
    }
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int64_t c = (int64_t)u * 256 + t;
        if (c >= chunks) continue;
        if constexpr (IS_F32) {
            const float e[4] = {__uint_as_float(raw[u].x), __uint_as_float(raw[u].y),
                                __uint_as_float(raw[u].z), __uint_as_float(raw[u].w)};
            uint32_t word = 0;
            if (finite) {
                const float y0 = e[0] / s, y1 = e[1] / s, y2 = e[2] / s, y3 = e[3] / s;
                word = (QT == Q_FP8) ? enc_fp8x4(y0, y1, y2, y3) : enc_i8x4(y0, y1, y2, y3);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t code;
                    if (nan_row || __builtin_isinf(e[j])) code = (QT == Q_FP8) ? 0x7Fu : 0u;
                    else code = (QT == Q_FP8) ? ((__float_as_uint(e[j]) >> 24) & 0x80u) : 0u;
                    word |= code << (8 * j);
                }
            }
            *reinterpret_cast<uint32_t*>(q + r * K + c * 4) = word;
        } else {
            const float xv[8] = {bf16_lo(raw[u].x), bf16_hi(raw[u].x), bf16_lo(raw[u].y),
                                 bf16_hi(raw[u].y), bf16_lo(raw[u].z), bf16_hi(raw[u].z),
                                 bf16_lo(raw[u].w), bf16_hi(raw[u].w)};
            const uint2 codes = finite ? encode8<QT>(xv, s) : encode8_special<QT>(xv, nan_row);
            *reinterpret_cast<uint2*>(q + r * K + c * 8) = codes;
        }
    }
    if (t == 0) scales[r * s_stride] = s;
}

// ---------------------------------------------------------------- launchers ----

template <int IS_F32, int QT>
static hipError_t launch_rows_p(const void* x, void* q, float* scales, int64_t rows, int64_t K,
                                int64_t s_stride, float eps, int ue, hipStream_t stream) {
    constexpr int E = IS_F32 ? 4 : 8;
    const int64_t slots = (K / E + 255) / 256;
    const dim3 grid((unsigned)rows);
    const uint4* xp = static_cast<const uint4*>(x);
    uint8_t* qp = static_cast<uint8_t*>(q);
#define BFQ_ROWS_CASE(PP)                                                                   \
    if (slots <= PP) {                                                                      \
        hipLaunchKernelGGL((quant_rows_kernel<IS_F32, QT, PP>), grid, dim3(256), 0, stream,  \
                           xp, qp, scales, K, s_stride, eps, ue);                           \
        return hipGetLastError();                                                           \
    }
    BFQ_ROWS_CASE(1)
    BFQ_ROWS_CASE(2)
    BFQ_ROWS_CASE(4)
    BFQ_ROWS_CASE(8)
    BFQ_ROWS_CASE(16)
    BFQ_ROWS_CASE(32)
#undef BFQ_ROWS_CASE
    return hipErrorInvalidValue;   // K beyond kChannelMaxK (rejected by the caller)
}

hipError_t launch_quant_rows(const void* x, int is_f32, void* q, float* scales, int64_t rows,
                             int64_t K, int qtype, int64_t s_stride, float eps, int sfmt,
                             hipStream_t stream) {
    const int ue = sfmt == S_UE8M0;
    if (is_f32)
        return qtype == Q_FP8
                   ? launch_rows_p<1, Q_FP8>(x, q, scales, rows, K, s_stride, eps, ue, stream)
                   : launch_rows_p<1, Q_INT8>(x, q, scales, rows, K, s_stride, eps, ue, stream);
    return qtype == Q_FP8
               ? launch_rows_p<0, Q_FP8>(x, q, scales, rows, K, s_stride, eps, ue, stream)
               : launch_rows_p<0, Q_INT8>(x, q, scales, rows, K, s_stride, eps, ue, stream);
}

// Row-major [N][K] codes -> BFQ_W_PACKED16. Thread c writes 16-byte chunk c of the packed
// matrix (coalesced): fragment F = c / 128 = f*KB + kb, half h, lane l; it reads the 16 bytes
// of row 16f + l%16 at column 128kb + 64h + 16*(l/16).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ w,
                                                           uint8_t* __restrict__ packed,
                                                           int64_t chunks, int64_t K) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t KB = K / 128;
    const int64_t F = c >> 7, f = F / KB, kb = F - f * KB;
    const int h = (int)(c >> 6) & 1, l = (int)c & 63;
    const int64_t row = 16 * f + (l & 15), col = 128 * kb + 64 * h + 16 * (l >> 4);
    *reinterpret_cast<v4u*>(packed + c * 16) = *reinterpret_cast<const v4u*>(w + row * K + col);
}

hipError_t launch_quant_tokens(const void* x, void* q, float* scales, int64_t M, int64_t K,
                               int qtype, int64_t s_stride_m, int64_t s_stride_g, float eps,
                               int sfmt, int packed, hipStream_t stream) {
    const int64_t G = K / 128;
    const int64_t rows = packed ? (M + 3) / 4 * 4 : M;    // packed: zero words up to 4 | rows
    dim3 grid((unsigned)rows, (unsigned)((G + kGroupsPerBlock - 1) / kGroupsPerBlock));
    dim3 block(64 * kQuantWaves);
    const int ue = sfmt == S_UE8M0;
    if (qtype == Q_FP8)
        hipLaunchKernelGGL(quant_tokens_kernel<Q_FP8>, grid, block, 0, stream,
                           (const uint4*)x, (uint2*)q, scales, M, K, G, s_stride_m, s_stride_g, eps,
                           ue, packed);
    else
        hipLaunchKernelGGL(quant_tokens_kernel<Q_INT8>, grid, block, 0, stream,
                           (const uint4*)x, (uint2*)q, scales, M, K, G, s_stride_m, s_stride_g, eps,
                           ue, packed);
    return hipGetLastError();
}

hipError_t launch_quant_weight_blocks(const float* w, void* q, float* scales, int64_t N,
                                      int64_t K, int qtype, float eps, int sfmt,
                                      hipStream_t stream) {
    dim3 grid((unsigned)(K / 128), (unsigned)(N / 128));
    const int ue = sfmt == S_UE8M0;
    if (qtype == Q_FP8)
        hipLaunchKernelGGL(quant_weight_blocks_kernel<Q_FP8>, grid, dim3(256), 0, stream, w,
                           (uint8_t*)q, scales, N, K, eps, ue);
    else
        hipLaunchKernelGGL(quant_weight_blocks_kernel<Q_INT8>, grid, dim3(256), 0, stream, w,
                           (uint8_t*)q, scales, N, K, eps, ue);
    return hipGetLastError();
}

hipError_t launch_debug_encode(const float* x, int64_t n, int qtype, void* out,
                               hipStream_t stream) {
    int64_t threads = (n + 3) / 4;
    dim3 grid((unsigned)((threads + 255) / 256));
    if (qtype == Q_FP8)
        hipLaunchKernelGGL(debug_encode_kernel<Q_FP8>, grid, dim3(256), 0, stream, x,
                           (uint8_t*)out, n);
    else
        hipLaunchKernelGGL(debug_encode_kernel<Q_INT8>, grid, dim3(256), 0, stream, x,
                           (uint8_t*)out, n);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const void* w, void* packed, int64_t N, int64_t K,
                               hipStream_t stream) {
    const int64_t chunks = N * K / 16;
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const uint8_t*>(w), static_cast<uint8_t*>(packed),
                       chunks, K);
    return hipGetLastError();
}

}  // namespace bfq
