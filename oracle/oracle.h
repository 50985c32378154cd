/*
 * CPU oracle for the block-scaled W8A8 linear layer — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may load
 * this library. It shares no source with the HIP library (block_scaled_w8a8_amd/csrc)
 * and includes none of its headers.
 *
 * Pages cited (by title and section):
 *   [BENCH]  "vLLM DeepGEMM FP8 Block GEMM 基准测试：DeepSeek DeepGEMM 对比 Triton 与 CUTLASS
 *             的块量化 GEMM 内核解析" (blog.gitcode.com)
 *   [CONFIG] "vLLM 量化 Kernel 配置机制：W8A8 Block FP8 Triton 内核的调优、选择与回退原理"
 *             (blog.gitcode.com)
 *   [PR]     vLLM pull request 42153, per_token_group_quant 2-D grid (prhub.com.cn)
 *   [HELION] "Building a High-Performance and Portable vLLM Linear Backend with Helion"
 *             (PyTorch blog, translated)
 *
 * Every function here is pinned by a "not gpu" test against something other than itself
 * (format definition, library codecs, brute force, exact special cases, printed figures).
 */
#ifndef BFQ_ORACLE_H
#define BFQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FP8 = 0, ORC_INT8 = 1 };
/* Scale formats: fp32 quotient, or that quotient rounded up to a power of two (UE8M0). */
enum { ORC_SCALE_FP32 = 0, ORC_SCALE_UE8M0 = 1 };

/* OCP FP8 e4m3fn codec. decode: 0x7F/0xFF -> NaN; exact value otherwise (as double). */
double  orc_e4m3_decode(uint8_t code);
/* fp32 -> e4m3fn code: round to nearest, ties to even, saturating to +-448; NaN -> 0x7F;
 * sign of zero kept; no flush of the e4m3 subnormals. */
uint8_t orc_e4m3_encode(float x);
/* fp32 -> int8 code: round to nearest, ties to even, clamp to [-127, 127]; NaN -> 0. */
int8_t  orc_int8_encode(float x);

/* Elementwise array forms of the encoders (OpenMP). */
void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out);
void orc_int8_encode_array(const float* x, int64_t n, int8_t* out);
void orc_f32_to_bf16_array(const float* x, int64_t n, uint16_t* out);

float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);   /* RNE; NaN -> 0x7FC0 */

/* Per-token-group quantization of bf16 activations x[M][K] (row-major).
 * q[M][K] codes (1 byte each); s[M][K/group] row-major fp32 scales.
 * scale = max(amax, eps) / Qmax with Qmax = 448 (fp8) or 127 (int8); code = enc(x / scale).
 * scale_fmt ORC_SCALE_UE8M0 rounds the scale up to a power of two first.
 * A group containing NaN gets a NaN scale. */
void orc_quant_groups(const uint16_t* x, int64_t M, int64_t K, int64_t group,
                      int qtype, void* q, float* s, float eps, int scale_fmt);

/* Per-block quantization of fp32 weights W[N][K] over bn x bk blocks.
 * q[N][K] codes; s[N/bn][K/bk] row-major fp32 scales. Same rule as the groups. */
void orc_quant_blocks(const float* w, int64_t N, int64_t K, int64_t bn, int64_t bk,
                      int qtype, void* q, float* s, float eps, int scale_fmt);

/* UE8M0 scales s[M][G] (powers of two) -> packed words: word (w, m) at words[w*ld + m],
 * byte j = E8M0 code (exponent + 127; NaN/Inf -> 255) of group 4w+j, 0 past G; rows
 * M .. round_up(M,4)-1 zero. ld >= round_up(M, 4). */
void orc_pack_scales_ue8m0(const float* s, int64_t M, int64_t G, uint32_t* words, int64_t ld);

/* Block-scaled GEMM C[M][N] = sum_kb (sum_{k in kb} A[m,k] W[n,k]) * sa[m,kb] * sw[n/128,kb].
 * qa[M][K], qw[N][K] codes; sa[M][K/128]; sw[N/128][K/128]. Per-block sums are exact
 * (fp64 for fp8, int32 for int8); the running accumulator is fp32 in ascending kb order.
 * c32 (may be NULL) gets the fp32 accumulator, c16 (may be NULL) its bf16 RNE rounding. */
void orc_block_gemm(const void* qa, const float* sa, const void* qw, const float* sw,
                    int64_t M, int64_t N, int64_t K, int qtype, float* c32, uint16_t* c16);

/* The same accumulator at `count` sampled output coordinates (ms[i], ns[i]). */
void orc_block_gemm_sampled(const void* qa, const float* sa, const void* qw, const float* sw,
                            int64_t M, int64_t N, int64_t K, int qtype,
                            const int64_t* ms, const int64_t* ns, int64_t count, float* c32);

/* Per-token x per-channel GEMM (FP8_Dynamic / W8A8_INT8):
 * C[m][n] = ((float)(sum_k A[m,k] W[n,k]) * sa[m]) * sw[n], the code dot product over the
 * whole K exact (fp64 for fp8 while K < 2^17, int64 for int8). sa[M], sw[N]. */
void orc_channel_gemm(const void* qa, const float* sa, const void* qw, const float* sw,
                      int64_t M, int64_t N, int64_t K, int qtype, float* c32, uint16_t* c16);
void orc_channel_gemm_sampled(const void* qa, const float* sa, const void* qw, const float* sw,
                              int64_t M, int64_t N, int64_t K, int qtype,
                              const int64_t* ms, const int64_t* ns, int64_t count, float* c32);

/* MoE routing: pairs q = t*topk + j with expert topk_ids[q] (flat [T*topk]) grouped by
 * expert, ascending q within an expert (stable counting sort). offsets[E+1] = prefix sums
 * of the per-expert counts; sorted[pairs] = pair ids in expert order. */
void orc_moe_align(const int32_t* topk_ids, int64_t pairs, int64_t E, int32_t* offsets,
                   int32_t* sorted);

/* MoE grouped block GEMM: out[q][n] (pair order, [T*topk][N]) = the block-scaled GEMM
 * element of token row q / topk of qa ([T][K], scales sa [T][K/128]) against row n of expert
 * topk_ids[q]'s weights (qw [E][N][K], sw [E][N/128][K/128]); same arithmetic as
 * orc_block_gemm. */
void orc_moe_gemm(const void* qa, const float* sa, const int32_t* topk_ids, int64_t T,
                  int64_t topk, const void* qw, const float* sw, int64_t E, int64_t N,
                  int64_t K, int qtype, float* c32);
void orc_moe_gemm_sampled(const void* qa, const float* sa, const int32_t* topk_ids,
                          int64_t topk, const void* qw, const float* sw, int64_t N, int64_t K,
                          int qtype, const int64_t* qs, const int64_t* ns, int64_t count,
                          float* c32);

/* int8 only: exact per-128-K-block integer partials, layout [K/128][M][N]. */
void orc_block_partials_i32(const int8_t* qa, const int8_t* qw, int64_t M, int64_t N,
                            int64_t K, int32_t* out);

/* fp64 dequantize-then-matmul: D[m][n] = sum_k (dec(qa)*sa) * (dec(qw)*sw). */
void orc_dequant_gemm_f64(const void* qa, const float* sa, const void* qw, const float* sw,
                          int64_t M, int64_t N, int64_t K, int qtype, double* d);

/* Number of OpenMP threads the oracle runs with. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
