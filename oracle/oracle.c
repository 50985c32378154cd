/*
 * CPU oracle for the block-scaled W8A8 linear layer — TEST INFRASTRUCTURE ONLY.
 * Plain C, no intrinsics, no BLAS; built with -ffp-contract=off so every fp32 operation
 * is a separately rounded IEEE operation. See oracle.h for the pages cited.
 *
 * What it computes (restated from the pages, in the pages' order):
 *  - activations are quantized per token and per 128-wide K group; the scale is the group's
 *    absolute maximum divided by the largest code, and the code is the value divided by
 *    that scale, stored as float8_e4m3fn ([BENCH] §4.1; [PR] kernel parameters eps,
 *    min_8bit, max_8bit);
 *  - weights are quantized per 128x128 block the same way ([BENCH] §4.1);
 *  - the GEMM walks K one 128-wide block at a time, forms the block's dot product and
 *    immediately multiplies it by the activation scale and then the weight scale before
 *    adding it to an fp32 accumulator ([BENCH] §4.2, the Triton kernel's inner step);
 *  - the output is written as bf16 ([BENCH] §4.2, output_dtype=bfloat16).
 * Readings of points the pages leave open (eps value, division vs reciprocal, NaN/Inf
 * handling, int8 range) are listed in the project design notes; each is marked here too.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- codecs ---- */

/* OCP FP8 E4M3 ("fn": no infinities, one NaN pattern per sign): 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits. Exponent field 0 holds the subnormals m * 2^-9;
 * exponent 15 with mantissa 7 is NaN, so the largest finite value is 1.75 * 2^8 = 448. */
double orc_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Round |x| to the nearest e4m3 value, ties to the even mantissa, then encode.
 * Reading: out-of-range magnitudes (and +-Inf) saturate to 448; NaN -> 0x7F; the sign of
 * zero is kept; e4m3 subnormals are produced, never flushed. */
uint8_t orc_e4m3_encode(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);                 /* exact */
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                              /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                             /* floor(log2 a) */
    if (e < -6) e = -6;                         /* subnormals share the lowest binade's spacing */
    double step = ldexp(1.0, e - 3);            /* spacing of e4m3 values in this binade */
    double n = nearbyint(a / step);             /* a / step is exact; nearbyint rounds to even */
    double v = n * step;                        /* exact; v <= 448 because a < 448 */
    if (v == 0.0) return sign;
    int ev;
    frexp(v, &ev);
    int E = ev - 1;
    if (E < -6) return sign | (uint8_t)(v * 512.0);           /* subnormal: v = m * 2^-9 */
    int mant = (int)(v / ldexp(1.0, E - 3)) - 8;               /* 0..7 */
    return sign | (uint8_t)(((E + 7) << 3) | mant);
}

/* Reading: symmetric int8 codes in [-127, 127] (never -128), round half to even;
 * NaN has no integer code and maps to 0. */
int8_t orc_int8_encode(float x) {
    if (isnan(x)) return 0;
    double r = nearbyint((double)x);
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (int8_t)r;
}

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

void orc_int8_encode_array(const float* x, int64_t n, int8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_int8_encode(x[i]);
}

void orc_f32_to_bf16_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------ quantizers ---- */

static float qmax_of(int qtype) { return qtype == ORC_FP8 ? 448.0f : 127.0f; }

/* scale = max(amax, eps) / Qmax as one correctly rounded fp32 division.
 * UE8M0 format ([BENCH] §4.1, use_ue8m0=True): that quotient is rounded up to a power of
 * two. Reading: "rounded up" is the smallest power of two that is >= the fp32 quotient (a
 * quotient that already is a power of two stays); the codes are then encode(x / scale).
 * Reading: a NaN amax propagates into the scale, an infinite one stays infinite. */
static float scale_of(float amax, float eps, int qtype, int scale_fmt) {
    if (isnan(amax)) return NAN;
    float a = amax > eps ? amax : eps;
    float t = a / qmax_of(qtype);
    if (scale_fmt != ORC_SCALE_UE8M0 || isinf(t)) return t;
    int e;
    double f = frexp((double)t, &e);            /* t = f * 2^e, f in [0.5, 1) */
    return f == 0.5 ? t : (float)ldexp(1.0, e);  /* 2^(e-1) < t < 2^e otherwise */
}

static void store_code(void* q, int64_t i, float y, int qtype) {
    if (qtype == ORC_FP8) ((uint8_t*)q)[i] = orc_e4m3_encode(y);
    else                  ((int8_t*)q)[i] = orc_int8_encode(y);
}

void orc_quant_groups(const uint16_t* x, int64_t M, int64_t K, int64_t group,
                      int qtype, void* q, float* s, float eps, int scale_fmt) {
    int64_t G = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < G; ++g) {
            const uint16_t* row = x + m * K + g * group;
            float amax = 0.0f;
            int nan_seen = 0;
            for (int64_t k = 0; k < group; ++k) {
                float v = orc_bf16_to_f32(row[k]);
                if (isnan(v)) nan_seen = 1;
                else if (fabsf(v) > amax) amax = fabsf(v);
            }
            if (nan_seen) amax = NAN;
            float sc = scale_of(amax, eps, qtype, scale_fmt);
            s[m * G + g] = sc;
            for (int64_t k = 0; k < group; ++k) {
                float y = orc_bf16_to_f32(row[k]) / sc;     /* IEEE division (reading) */
                store_code(q, m * K + g * group + k, y, qtype);
            }
        }
    }
}

void orc_quant_blocks(const float* w, int64_t N, int64_t K, int64_t bn, int64_t bk,
                      int qtype, void* q, float* s, float eps, int scale_fmt) {
    int64_t NB = N / bn, KB = K / bk;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t nb = 0; nb < NB; ++nb) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            float amax = 0.0f;
            int nan_seen = 0;
            for (int64_t i = 0; i < bn; ++i)
                for (int64_t j = 0; j < bk; ++j) {
                    float v = w[(nb * bn + i) * K + kb * bk + j];
                    if (isnan(v)) nan_seen = 1;
                    else if (fabsf(v) > amax) amax = fabsf(v);
                }
            if (nan_seen) amax = NAN;
            float sc = scale_of(amax, eps, qtype, scale_fmt);
            s[nb * KB + kb] = sc;
            for (int64_t i = 0; i < bn; ++i)
                for (int64_t j = 0; j < bk; ++j) {
                    int64_t idx = (nb * bn + i) * K + kb * bk + j;
                    store_code(q, idx, w[idx] / sc, qtype);
                }
        }
    }
}

/* --------------------------------------------------- packed UE8M0 scale words ---- */

/* [PR] page, per_token_group_quant_8bit_packed: the scales of a token's groups leave the
 * quantizer as UE8M0 bytes, four consecutive groups to one 32-bit word (output_s_packed),
 * the words stored token-major with the token count padded for TMA (tma_aligned_mn).
 * Reading: word (w, m) at words[w * ld + m]; its byte j (bits 8j..8j+7) is the E8M0 code of
 * the scale of group 4w + j of token m, 0 past the last group; the rows M .. round_up(M, 4)
 * - 1 hold zero words. The E8M0 code of a power of two 2^e is e + 127; NaN (and, since E8M0
 * has no infinity, Inf) is 255. */
static uint32_t e8m0_code(float s) {
    if (isnan(s) || isinf(s)) return 255u;
    int e;
    double f = frexp((double)s, &e);       /* s = f * 2^e, f = 0.5 for a power of two */
    (void)f;
    return (uint32_t)(e - 1 + 127);
}

void orc_pack_scales_ue8m0(const float* s, int64_t M, int64_t G, uint32_t* words, int64_t ld) {
    int64_t W = (G + 3) / 4, Mp = (M + 3) / 4 * 4;
    for (int64_t w = 0; w < W; ++w)
        for (int64_t m = 0; m < Mp; ++m) {
            uint32_t word = 0;
            for (int64_t j = 0; j < 4; ++j) {
                int64_t g = 4 * w + j;
                if (m < M && g < G) word |= e8m0_code(s[m * G + g]) << (8 * j);
            }
            words[w * ld + m] = word;
        }
}

/* ------------------------------------------------------------------ GEMM ---- */

static double g_dec[256];
static int g_dec_ready = 0;

static void init_decode_table(void) {
    if (g_dec_ready) return;
    for (int c = 0; c < 256; ++c) g_dec[c] = orc_e4m3_decode((uint8_t)c);
    g_dec_ready = 1;
}

/* One output element. The 128-term block sum is exact: in fp64 for e4m3 (every product is
 * a multiple of 2^-18 below 2^18 in magnitude, so every partial sum of at most 128 terms
 * needs fewer than 53 bits) and in int32 for int8 (|sum| <= 128 * 127^2). */
static float gemm_element(const void* qa, const float* sa, const void* qw, const float* sw,
                          int64_t m, int64_t n, int64_t K, int qtype) {
    int64_t KB = K / 128;
    float acc = 0.0f;
    for (int64_t kb = 0; kb < KB; ++kb) {
        float p;
        if (qtype == ORC_FP8) {
            const uint8_t* a = (const uint8_t*)qa + m * K + kb * 128;
            const uint8_t* w = (const uint8_t*)qw + n * K + kb * 128;
            double sum = 0.0;
            for (int k = 0; k < 128; ++k) sum += g_dec[a[k]] * g_dec[w[k]];
            p = (float)sum;
        } else {
            const int8_t* a = (const int8_t*)qa + m * K + kb * 128;
            const int8_t* w = (const int8_t*)qw + n * K + kb * 128;
            int32_t sum = 0;
            for (int k = 0; k < 128; ++k) sum += (int32_t)a[k] * (int32_t)w[k];
            p = (float)sum;                       /* exact: |sum| < 2^24 */
        }
        /* the block product times the activation scale, then times the weight scale,
         * then added to the running fp32 accumulator */
        float t = p * sa[m * KB + kb];
        t = t * sw[(n / 128) * KB + kb];
        acc = acc + t;
    }
    return acc;
}

void orc_block_gemm(const void* qa, const float* sa, const void* qw, const float* sw,
                    int64_t M, int64_t N, int64_t K, int qtype, float* c32, uint16_t* c16) {
    init_decode_table();
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float acc = gemm_element(qa, sa, qw, sw, m, n, K, qtype);
            if (c32) c32[m * N + n] = acc;
            if (c16) c16[m * N + n] = orc_f32_to_bf16(acc);
        }
}

void orc_block_gemm_sampled(const void* qa, const float* sa, const void* qw, const float* sw,
                            int64_t M, int64_t N, int64_t K, int qtype,
                            const int64_t* ms, const int64_t* ns, int64_t count, float* c32) {
    (void)M; (void)N;
    init_decode_table();
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        c32[i] = gemm_element(qa, sa, qw, sw, ms[i], ns[i], K, qtype);
}

/* ----------------------------------------------- per-token x per-channel GEMM ---- */

/* [HELION] scope section: in the FP8_Dynamic and W8A8_INT8 formats every token row of the
 * activations has one scale and every output channel (weight row) has one. Reading: the dot
 * product of the codes over the whole of K is taken exactly, rounded once to fp32, then
 * multiplied by the token scale and then by the channel scale (the left-to-right order the
 * block path uses within a block). Exactness: e4m3 products are multiples of 2^-18 below
 * 2^18 in magnitude, so a sum of K of them needs fewer than 53 bits while K < 2^17; int8
 * sums are exact in int64. */
static float channel_element(const void* qa, const float* sa, const void* qw, const float* sw,
                             int64_t m, int64_t n, int64_t K, int qtype) {
    float p;
    if (qtype == ORC_FP8) {
        const uint8_t* a = (const uint8_t*)qa + m * K;
        const uint8_t* w = (const uint8_t*)qw + n * K;
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) sum += g_dec[a[k]] * g_dec[w[k]];
        p = (float)sum;
    } else {
        const int8_t* a = (const int8_t*)qa + m * K;
        const int8_t* w = (const int8_t*)qw + n * K;
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k) sum += (int64_t)a[k] * (int64_t)w[k];
        p = (float)sum;
    }
    float t = p * sa[m];
    t = t * sw[n];
    return t;
}

void orc_channel_gemm(const void* qa, const float* sa, const void* qw, const float* sw,
                      int64_t M, int64_t N, int64_t K, int qtype, float* c32, uint16_t* c16) {
    init_decode_table();
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float v = channel_element(qa, sa, qw, sw, m, n, K, qtype);
            if (c32) c32[m * N + n] = v;
            if (c16) c16[m * N + n] = orc_f32_to_bf16(v);
        }
}

void orc_channel_gemm_sampled(const void* qa, const float* sa, const void* qw, const float* sw,
                              int64_t M, int64_t N, int64_t K, int qtype,
                              const int64_t* ms, const int64_t* ns, int64_t count, float* c32) {
    (void)M; (void)N;
    init_decode_table();
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        c32[i] = channel_element(qa, sa, qw, sw, ms[i], ns[i], K, qtype);
}

/* ------------------------------------------------------ MoE grouped GEMM ---- */

/* [CONFIG] §5: the MoE kernels reuse the per-shape, per-batch-size config scheme with an
 * expert count E in the key. Reading of the grouped GEMM the tables serve: token t routed
 * to experts topk_ids[t][0..topk-1] forms pairs q = t*topk + j; the pairs are grouped by
 * expert (a stable counting sort: ascending pair id within an expert), and each pair's
 * output row is the block-scaled GEMM of its token's quantized row with its expert's
 * weights, written at row q (pair order). */
void orc_moe_align(const int32_t* topk_ids, int64_t pairs, int64_t E, int32_t* offsets,
                   int32_t* sorted) {
    for (int64_t e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t q = 0; q < pairs; ++q) offsets[topk_ids[q] + 1] += 1;   /* counts */
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];         /* prefix */
    int64_t* cursor = (int64_t*)malloc((size_t)E * sizeof(int64_t));
    for (int64_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t q = 0; q < pairs; ++q) sorted[cursor[topk_ids[q]]++] = (int32_t)q;
    free(cursor);
}

/* out[q][n] for pair q = t*topk + j routed to expert e: the block GEMM element of token row t
 * of qa against row n of expert e's weights (qw + e*N*K, sw + e*(N/128)*(K/128)). */
static float moe_element(const void* qa, const float* sa, const void* qw, const float* sw,
                         const int32_t* topk_ids, int64_t topk, int64_t q, int64_t n, int64_t N,
                         int64_t K, int qtype) {
    int64_t t = q / topk, e = topk_ids[q];
    int64_t KB = K / 128;
    const uint8_t* we = (const uint8_t*)qw + e * N * K;
    const float* swe = sw + e * (N / 128) * KB;
    return gemm_element(qa, sa, we, swe, t, n, K, qtype);
}

void orc_moe_gemm(const void* qa, const float* sa, const int32_t* topk_ids, int64_t T,
                  int64_t topk, const void* qw, const float* sw, int64_t E, int64_t N,
                  int64_t K, int qtype, float* c32) {
    (void)E;
    init_decode_table();
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t q = 0; q < T * topk; ++q)
        for (int64_t n = 0; n < N; ++n)
            c32[q * N + n] = moe_element(qa, sa, qw, sw, topk_ids, topk, q, n, N, K, qtype);
}

void orc_moe_gemm_sampled(const void* qa, const float* sa, const int32_t* topk_ids,
                          int64_t topk, const void* qw, const float* sw, int64_t N, int64_t K,
                          int qtype, const int64_t* qs, const int64_t* ns, int64_t count,
                          float* c32) {
    init_decode_table();
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        c32[i] = moe_element(qa, sa, qw, sw, topk_ids, topk, qs[i], ns[i], N, K, qtype);
}

void orc_block_partials_i32(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N,
                            int64_t K, int32_t* out) {
    int64_t KB = K / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t kb = 0; kb < KB; ++kb) {
                int32_t sum = 0;
                for (int k = 0; k < 128; ++k)
                    sum += (int32_t)qa[m * K + kb * 128 + k] * (int32_t)qw[n * K + kb * 128 + k];
                out[(kb * M + m) * N + n] = sum;
            }
}

void orc_dequant_gemm_f64(const void* qa, const float* sa, const void* qw, const float* sw,
                          int64_t M, int64_t N, int64_t K, int qtype, double* d) {
    init_decode_table();
    int64_t KB = K / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a, w;
                if (qtype == ORC_FP8) {
                    a = g_dec[((const uint8_t*)qa)[m * K + k]];
                    w = g_dec[((const uint8_t*)qw)[n * K + k]];
                } else {
                    a = (double)((const int8_t*)qa)[m * K + k];
                    w = (double)((const int8_t*)qw)[n * K + k];
                }
                a *= (double)sa[m * KB + k / 128];
                w *= (double)sw[(n / 128) * KB + k / 128];
                sum += a * w;
            }
            d[m * N + n] = sum;
        }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
