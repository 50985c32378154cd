/*
 * bfq.h — C-ABI of libbfq: block-scaled W8A8 (e4m3fn / int8) linear layer on MI355X (gfx950).
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
 * Conventions for every entry point:
 *  - Device pointers unless marked "host". Every buffer is allocated and freed by the
 *    caller; the library never allocates, frees or synchronizes device memory. It owns only
 *    its host-side tile table and the static device buffer of bfq_block_gemm_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is enqueued
 *    asynchronously; the call returns once the launches are enqueued.
 *  - All arguments are validated before anything is enqueued. On a negative status nothing
 *    was launched and no output was touched; bfq_last_error() holds a detail string
 *    (thread-local). A positive status is success with a warning.
 *  - M = 0 is valid and launches nothing.
 *  - Shapes are int64; K and N must be multiples of 128 (GEMM: M, N < 2^31, M * N < 2^40,
 *    K <= 2^23, scale ld <= 2^23, and the activation scales of 256 tokens over all K blocks
 *    span less than 4 GiB), and x/q/w/out 16-byte aligned.
 *  - Two calls on one stream are ordered; calls on different streams that share an output
 *    or workspace race.
 */
#ifndef BFQ_H
#define BFQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BFQ_OK = 0,
    BFQ_WARN_DEFAULT_TILE = 1,  /* success; no tuned entry for (N,K,dtype): default tile used */
    BFQ_ERR_NULL = -1,          /* a required pointer is NULL */
    BFQ_ERR_SHAPE = -2,         /* M<0, K or N not a multiple of 128, group/block not 128 */
    BFQ_ERR_DTYPE = -3,         /* unsupported input/output dtype */
    BFQ_ERR_ALIGN = -4,         /* pointer not 16-byte aligned (scales: 4-byte) */
    BFQ_ERR_WORKSPACE = -5,     /* workspace smaller than bfq_gemm_workspace_bytes() */
    BFQ_ERR_TILE = -6,          /* explicit tile is not one of the compiled kernels */
    BFQ_ERR_TABLE = -7,         /* tile table file missing or malformed */
    BFQ_ERR_HIP = -8,           /* a HIP runtime call or launch failed */
    BFQ_ERR_ARG = -9            /* invalid scalar argument (eps, enum value, index) */
} bfq_status;

/* The *_INT32_RANGE_ enumerators below are not values of their enums: they make each enum a
 * 32-bit type in which every int32 is representable, so that an out-of-range argument from a
 * C or ctypes caller is rejected (BFQ_ERR_ARG / BFQ_ERR_DTYPE) rather than undefined. */
typedef enum {
    BFQ_BF16 = 0,
    BFQ_FP16 = 1,
    BFQ_FP32 = 2,
    BFQ_E4M3FN = 3,   /* OCP float8 e4m3fn, max 448 */
    BFQ_INT8 = 4,     /* symmetric int8 in [-127, 127] */
    BFQ_INT32 = 5,
    BFQ_DTYPE_INT32_RANGE_ = 0x7FFFFFFF  /* not a dtype: see below */
} bfq_dtype;

/* Layout of per-(token, group) activation scales, [BENCH] §4.1 (row-major for the Triton
 * kernel, column-major for CUTLASS/DeepGEMM; the TMA-aligned column-major form is
 * column-major with ld = M rounded up to a multiple of 4).
 * BFQ_SCALES_PACKED_UE8M0 ([PR]: the packed output of the per-token-group kernel,
 * output_s_packed): UE8M0 scales as E8M0 codes (2^(code - 127); NaN and Inf -> 255, E8M0
 * has no infinity), four groups per 32-bit word: word (w, m) at ((uint32_t*)s)[w * ld + m],
 * w < ceil(G/4), byte j (bits 8j..8j+7) = group 4w + j, 0 past the last group. The scale
 * pointer then addresses uint32 words. The quantizer needs ld >= M rounded up to a multiple
 * of 4 and writes zero words in rows M .. round_up(M, 4) - 1 (TMA row alignment); the GEMM
 * needs ld >= M. Only with scale_fmt BFQ_SCALE_UE8M0 and 1x128 groups. */
typedef enum {
    BFQ_SCALES_ROW_MAJOR = 0,    /* s[m * ld + g], ld >= K/128 */
    BFQ_SCALES_COL_MAJOR = 1,    /* s[g * ld + m], ld >= M     */
    BFQ_SCALES_PACKED_UE8M0 = 2, /* words[w * ld + m], see above */
    BFQ_SCALES_INT32_RANGE_ = 0x7FFFFFFF
} bfq_scale_layout;

/* Layout of the weight codes in memory. The values are the same bytes either way; the packed
 * layout puts each MFMA fragment's bytes together so that every wave-wide 16-byte-per-lane
 * load reads 1 KB of contiguous memory (a row-major [N][K] matrix can only give each load
 * 16 rows x 64 bytes, which caps the weight stream well below the HBM peak).
 *   BFQ_W_ROW_MAJOR: w[n][k] at byte n*K + k.
 *   BFQ_W_PACKED16 : for every 16-row group f = n/16 and K block kb, 2048 bytes at
 *                    (f*(K/128) + kb)*2048; inside them byte h*1024 + 16*l + b (h in {0,1},
 *                    lane l in [0,64), b in [0,16)) holds w[16f + l%16][128kb + 64h + 16*(l/16) + b].
 *                    The whole matrix still spans N*K bytes, rows in blocks of 16. */
typedef enum {
    BFQ_W_ROW_MAJOR = 0,
    BFQ_W_PACKED16 = 1,
    BFQ_W_INT32_RANGE_ = 0x7FFFFFFF
} bfq_weight_layout;

/* Format of the fp32 scales. UE8M0: every scale is a power of two — the block's
 * max(amax, eps)/Qmax rounded up to the next power of two ([BENCH] §4.1: with use_ue8m0 the
 * scale is first rounded up to a power of two, the format DeepGEMM's hardware scaling path
 * requires). The scales are still stored as fp32 (exact); the codes are encode(x / scale).
 * A GEMM told that both scale arrays are UE8M0 may apply them inside gfx950's
 * block-scaled MFMA instead of with one fp32 FMA per output and K block. */
typedef enum {
    BFQ_SCALE_FP32 = 0,
    BFQ_SCALE_UE8M0 = 1,
    BFQ_SCALE_INT32_RANGE_ = 0x7FFFFFFF
} bfq_scale_format;

/* One launch configuration of the block GEMM ([CONFIG] §2: per-M launch parameters).
 *   variant 0 "standard": bm x bn output tile per workgroup, A and W tiles staged through
 *             LDS (double-buffered), waves_m x waves_n waves, group_m = grouped tile order.
 *   variant 1 "swap_ab": the weight rows stream straight from HBM into the wide MFMA
 *             operand and the bm tokens ride in the narrow one; the output tile is formed
 *             transposed and stored back row-major ([HELION] kernel section). A workgroup
 *             holds waves_n strips of bn/waves_n weight rows; the waves_m waves of a strip
 *             split its K range and are summed in the workgroup, in a fixed order. sched 0:
 *             each wave fetches its token fragments; sched 1: each K block's token fragments
 *             are fetched once per workgroup and shared through LDS.
 *   variant 2 "stream-K": the tiles of variant 0 on a persistent grid of one workgroup per
 *             compute unit; whole tiles in rounds, then the K blocks of the last one to two
 *             rounds of tiles split evenly over the grid; a second kernel sums each split
 *             tile's parked fp32 partials in K order (split_k must be 1). Its workspace holds
 *             two partial tiles per compute unit.
 *   split_k  : K blocks split into split_k contiguous chunks (>= 1), fp32 partials reduced
 *             in a fixed order ([HELION] kernel section).
 *   stages   : LDS stages (variants 0, 2) or weight prefetch depth in K blocks (variant 1).
 *   sched    : variants 0 and 2 instruction schedule (variant 1: see above): 4 = per-token x
 *             per-channel scales (block_shape {1, K}), the MFMA accumulating the whole K; 3 = the scales
 *             applied by the block-scaled MFMA, which accumulates across K blocks (fp8 and
 *             BFQ_SCALE_UE8M0 scales only); 0 = each sub-tile's scale FMAs right after its
 *             MFMAs, 1 = software-pipelined (FMAs one sub-tile behind the MFMAs), 2 = 32x32
 *             sub-tiles (two 32x32x64 MFMAs per K block, FMAs one pair behind; fp8 only).
 *   group_m, raster: variants 0 and 2 tile order (launch arguments, any group_m >= 1): raster 0
 *             gives each of the 8 XCDs a contiguous range of tiles, raster 1 does not.
 *   bk is always 128 (one scale block per K step). */
typedef struct {
    int32_t variant, bm, bn, bk, split_k, waves_m, waves_n, stages, group_m, sched, raster,
        reserved;
} bfq_tile;

/* Per-token-group quantization ([BENCH] §4.1 per_token_group_quant_fp8; [PR] kernel
 * arguments eps/min_8bit/max_8bit). For each row m and 128-wide group g of x:
 *   scale = max(amax, eps) / Qmax   (Qmax = 448 for E4M3FN, 127 for INT8; IEEE division)
 *   q     = encode(x / scale)       (IEEE division; e4m3fn: RNE, saturating; int8: RNE,
 *                                    clamp [-127, 127])
 * scale_fmt BFQ_SCALE_UE8M0 rounds each scale up to a power of two before encoding.
 * A group containing NaN gets a NaN scale and codes 0x7F (e4m3fn) or 0 (int8).
 *   x_bf16 [M][K] row-major bf16; q [M][K] row-major codes (1 byte);
 *   scales: fp32, layout per `layout` with leading dimension scale_ld.
 * group_size 128, or group_size == K for one scale per token (the per-token activation scales
 * of the FP8_Dynamic / W8A8_INT8 formats, [HELION] scope section; K <= 32768): scales then
 * hold one value per row, at scales[m * scale_ld] (row-major, scale_ld >= 1) or scales[m]
 * (column-major, scale_ld >= M). q_dtype must be BFQ_E4M3FN or BFQ_INT8. */
bfq_status bfq_quant_tokens(const void* x_bf16, int64_t M, int64_t K, int32_t group_size,
                            bfq_dtype q_dtype, void* q, float* scales, bfq_scale_layout layout,
                            int64_t scale_ld, float eps, bfq_scale_format scale_fmt,
                            void* stream);

/* Per-block weight quantization, the offline step before the GEMM ([BENCH] §4.1
 * per_block_cast_to_fp8 with fp32 scales): for each block_shape[0] x block_shape[1] block of
 * w [N][K] (fp32, row-major): scale = max(amax, eps)/Qmax, q = encode(w / scale).
 *   q [N][K] codes; scales [N/128][K/128] row-major fp32.
 * block_shape {128, 128}, or {1, K} for one scale per output channel (the per-channel weight
 * scales of FP8_Dynamic / W8A8_INT8, [HELION] scope section; K <= 32768): scales [N]. */
bfq_status bfq_quant_weight_blocks(const float* w, int64_t N, int64_t K,
                                   const int32_t block_shape[2] /* host */, bfq_dtype q_dtype,
                                   void* q, float* scales, float eps,
                                   bfq_scale_format scale_fmt, void* stream);

/* Rearrange weight codes from row-major [N][K] into BFQ_W_PACKED16 (a byte permutation, part
 * of the offline weight preparation like bfq_quant_weight_blocks). w_q and w_packed are
 * separate N*K-byte device buffers (16-byte aligned, not overlapping); q_dtype E4M3FN or
 * INT8 (the permutation does not depend on it). N, K multiples of 128. */
bfq_status bfq_pack_weights(const void* w_q, int64_t N, int64_t K, bfq_dtype q_dtype,
                            void* w_packed, void* stream);

/* Tile selection ([CONFIG] §4.1-§4.2): exact (N, K, dtype, block shape, weight layout, scale format) entry of the loaded
 * tile table, then the bucket nearest to M (ties to the smaller bucket; M past the grid ->
 * last bucket). No entry -> the compiled-in default rule and BFQ_WARN_DEFAULT_TILE ([CONFIG]
 * §4.1 warns and falls back to a default config). tile_out is a host pointer. */
bfq_status bfq_select_tile(int64_t M, int64_t N, int64_t K, const int32_t block_shape[2],
                           bfq_dtype in_dtype, bfq_dtype out_dtype, bfq_weight_layout w_layout,
                           bfq_scale_format scale_fmt, bfq_tile* tile_out);

/* Batch-invariant mode ([CONFIG] §5: with the batch-invariant switch set, tuned configs are
 * not used, so that the output of a token does not depend on how many tokens are in the
 * batch). When enabled, bfq_select_tile ignores the tile table and returns tiles that
 * compute every output element with the same operations in the same order for any M: no
 * split-K, no K split inside a workgroup, no stream-K; with row-major weights only standard
 * tiles (the swap-AB kernels feed the MFMA a different K order there); scales always applied
 * by the fp32 FMA. Rows of the output are then bitwise independent of M. Process-wide;
 * initialized from the environment variable BFQ_BATCH_INVARIANT (1 = on) at first use; must
 * not be changed concurrently with other calls. Explicit tiles passed to bfq_block_gemm are
 * not affected. */
void    bfq_set_batch_invariant(int32_t enable);
int32_t bfq_get_batch_invariant(void);

/* Bytes of device workspace bfq_block_gemm needs for this shape and tile (split-K fp32
 * partials: split_k * M * N * 4 when split_k > 1; stream-K: two partial tiles per compute
 * unit; else 0). tile NULL -> the tile selected for e4m3fn codes in the row-major layout.
 * SIZE_MAX when M * N >= 2^40, a shape bfq_block_gemm rejects. */
size_t bfq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const bfq_tile* tile);

/* Block-scaled GEMM ([BENCH] §4.2, w8a8 block-scaled matmul):
 *   out[m][n] = sum_kb ( sum_{k in kb} a_q[m][k] * w_q[n][k] ) * a_scales[m, kb] * w_scales[n/128][kb]
 * with exact per-block products, an fp32 accumulator and one rounding to out_dtype.
 *   a_q [M][K] codes (K-contiguous); w_q N*K codes in w_layout (row-major [N][K] is the
 *   "NT" form of the page; BFQ_W_PACKED16 from bfq_pack_weights);
 *   a_scales per a_layout/a_scale_ld; w_scales [N/128][K/128] row-major;
 *   scale_fmt BFQ_SCALE_UE8M0 states that every a_scales and w_scales value is a power of
 *   two (as the quantizers write in that format); results are then undefined otherwise.
 *   out [M][N] row-major, out_dtype BF16 | FP16 | FP32.
 *   tile NULL -> bfq_select_tile for (w_layout, scale_fmt); an explicit tile must name a
 *   kernel compiled for w_layout whose scale handling allows scale_fmt (else BFQ_ERR_TILE);
 *   workspace may be NULL when the tile needs none.
 * block_shape {1, K} selects the per-token x per-channel format ([HELION] scope section,
 * FP8_Dynamic / W8A8_INT8; K <= 32768):
 *   out[m][n] = ( sum_k a_q[m][k] * w_q[n][k] ) * a_scales[m] * w_scales[n]
 *   with one scale per token (a_layout row-major: a_scales[m * a_scale_ld], a_scale_ld >= 1;
 *   column-major: a_scales[m], a_scale_ld >= M) and w_scales [N]; the codes' product is
 *   accumulated over the whole K (fp8: fp32 MFMA accumulation; int8: exact int32), then
 *   scaled once. scale_fmt does not change how such scales are applied. Those kernels are
 *   tiles with sched 4 (variants 0 and 2) or the variant 1 tiles built for this format.
 * Returns BFQ_WARN_DEFAULT_TILE when tile was NULL and the default rule was used. */
bfq_status bfq_block_gemm(const void* a_q, const float* a_scales, bfq_scale_layout a_layout,
                          int64_t a_scale_ld, const void* w_q, const float* w_scales,
                          bfq_weight_layout w_layout, bfq_scale_format scale_fmt, void* out,
                          int64_t M, int64_t N, int64_t K,
                          const int32_t block_shape[2] /* host */, bfq_dtype in_dtype,
                          bfq_dtype out_dtype, const bfq_tile* tile /* host */,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The block GEMM for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments and
 * result as bfq_block_gemm without a workspace; split-K partials and stream-K slots go to a
 * static device buffer of the library (bfq_noalloc_scratch_bytes() = 32 MiB, one per GPU,
 * held from the library's load until the process ends). It calls no allocator.
 *   tile NULL -> the tile bfq_select_tile gives, made to fit the buffer: a stream-K tile runs
 *   as the plain grid of the same tile, and the K split drops until the partials fit (the
 *   result stays within the parity bar; it may differ in the last bits from bfq_block_gemm,
 *   which runs the selected tile as is).
 *   An explicit tile whose workspace exceeds the buffer -> BFQ_ERR_WORKSPACE (nothing
 *   launched).
 * Every call on one GPU shares that GPU's buffer: calls that overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller. The buffer keeps the
 * last call's contents; no call reads what an earlier one left. */
bfq_status bfq_block_gemm_noalloc(const void* a_q, const float* a_scales,
                                  bfq_scale_layout a_layout, int64_t a_scale_ld, const void* w_q,
                                  const float* w_scales, bfq_weight_layout w_layout,
                                  bfq_scale_format scale_fmt, void* out, int64_t M, int64_t N,
                                  int64_t K, const int32_t block_shape[2] /* host */,
                                  bfq_dtype in_dtype, bfq_dtype out_dtype,
                                  const bfq_tile* tile /* host */, void* stream);
size_t bfq_noalloc_scratch_bytes(void);

/* Load a tile table (JSON, host path) and replace the current one ([CONFIG] §2 schema:
 * per (N, K, dtype, block_shape) a map "M bucket -> launch parameters"). Must not run
 * concurrently with other calls. NULL reloads the default location. */
bfq_status bfq_load_tile_table(const char* json_path);

/* Number of compiled kernel configurations usable for (block_shape, in_dtype, w_layout,
 * scale_fmt), and the i-th one (split_k = 1; any split_k >= 1 may be combined with it). Used
 * by the on-device sweep. block_shape (host) {128, 128}, or {1, k} (any k > 0) for the
 * per-token x per-channel kernels. */
int32_t bfq_num_tile_candidates(const int32_t block_shape[2], bfq_dtype in_dtype,
                                bfq_weight_layout w_layout, bfq_scale_format scale_fmt);
bfq_status bfq_get_tile_candidate(const int32_t block_shape[2], bfq_dtype in_dtype,
                                  bfq_weight_layout w_layout, bfq_scale_format scale_fmt,
                                  int32_t index, bfq_tile* tile_out);

/* ------------------------------------------------------- MoE grouped block GEMM ----
 * [CONFIG] §5: the MoE kernels take the same per-shape, per-batch-size tuned configs with an
 * expert count E in the key. Token t routed to experts topk_ids[t][0..topk-1] forms pairs
 * q = t*topk + j; out[q][n] (pair order, [T*topk][N]) = the block-scaled GEMM (as
 * bfq_block_gemm) of token row t of a_q with row n of expert topk_ids[t][j]'s weights.
 * e4m3fn codes, block_shape {128, 128}; the combine over a token's experts is not part of it.
 */

/* Group the pairs by expert (stable: ascending pair id within an expert), the routing step
 * the grouped GEMM reads. topk_ids [T][topk] int32 (device); expert_offsets [E+1] int32:
 * pairs of expert e are sorted_pairs[expert_offsets[e] .. expert_offsets[e+1]);
 * sorted_pairs int32, at least T*topk entries (the first T*topk are written). An id
 * outside [0, E) goes after every expert (beyond
 * expert_offsets[E]) and its pair is never computed. 1 <= E <= 1023; workspace of
 * bfq_moe_align_workspace_bytes bytes (may be NULL when that is 0). Asynchronous. */
size_t     bfq_moe_align_workspace_bytes(int64_t T, int32_t topk, int32_t E);
bfq_status bfq_moe_align(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                         int32_t* expert_offsets, int32_t* sorted_pairs, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Tile of the grouped GEMM: the (E, N, K, dtype, weight layout, scale format) table entry,
 * bucket nearest to the token count T; else a default rule from the average rows per active
 * expert and BFQ_WARN_DEFAULT_TILE. Batch-invariant mode applies as in bfq_select_tile. */
bfq_status bfq_moe_select_tile(int64_t T, int32_t topk, int32_t E, int64_t N, int64_t K,
                               const int32_t block_shape[2], bfq_dtype in_dtype,
                               bfq_dtype out_dtype, bfq_weight_layout w_layout,
                               bfq_scale_format scale_fmt, bfq_tile* tile_out);
/* split_k * T * topk * N * 4 bytes when the tile's split_k > 1, else 0; SIZE_MAX when
 * T * topk * N >= 2^40, a shape bfq_moe_block_gemm rejects. */
size_t     bfq_moe_gemm_workspace_bytes(int64_t T, int32_t topk, int64_t N, const bfq_tile* tile);

/* Grouped GEMM over the expert groups of bfq_moe_align.
 *   a_q [T][K] codes and a_scales (a_layout/a_scale_ld over the T tokens; packed UE8M0 words
 *   allowed) as bfq_quant_tokens writes them: each pair's token row is gathered in the kernel;
 *   sorted_pairs, expert_offsets: bfq_moe_align's output (device);
 *   w_q [E][N][K] codes in w_layout (each expert's [N][K] matrix row-major, or packed by
 *   bfq_pack_weights, one after the other); w_scales [E][N/128][K/128];
 *   out [T*topk][N] in pair order; rows of pairs with an expert outside [0, E) are not written
 *   with split_k = 1 and are unspecified with split_k > 1.
 *   tile NULL -> bfq_moe_select_tile. Variants 0 and 1 (grouped forms); T * K < 2^31,
 *   T * topk * N < 2^40. */
bfq_status bfq_moe_block_gemm(const void* a_q, const float* a_scales, bfq_scale_layout a_layout,
                              int64_t a_scale_ld, const int32_t* sorted_pairs,
                              const int32_t* expert_offsets, int32_t topk, const void* w_q,
                              const float* w_scales, bfq_weight_layout w_layout,
                              bfq_scale_format scale_fmt, void* out, int64_t T, int64_t N,
                              int64_t K, int32_t E, const int32_t block_shape[2] /* host */,
                              bfq_dtype in_dtype, bfq_dtype out_dtype,
                              const bfq_tile* tile /* host */, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Compiled grouped kernels usable for (w_layout, scale_fmt) (e4m3fn; split_k = 1). */
int32_t    bfq_moe_num_tile_candidates(bfq_weight_layout w_layout, bfq_scale_format scale_fmt);
bfq_status bfq_moe_get_tile_candidate(bfq_weight_layout w_layout, bfq_scale_format scale_fmt,
                                      int32_t index, bfq_tile* tile_out);

const char* bfq_status_string(bfq_status s);
const char* bfq_last_error(void);

/* Test support: int8 per-K-block int32 partials, layout [K/128][M][N] (exact). */
bfq_status bfq_debug_block_partials_i32(const void* a_q, const void* w_q, int32_t* partials,
                                        int64_t M, int64_t N, int64_t K, void* stream);

/* Measurement support: `blocks` workgroups of 8 waves, each wave running 8 independent
 * chains of `iters` fp8 16x16x128 MFMAs on register operands and nothing else, so that
 * flops / elapsed is the matrix-core throughput the GPU sustains (at the clock it holds under
 * that load), stated beside the published peak. out: blocks * 512 floats (device), written
 * once per lane to keep the chains live; its values mean nothing. Flops of one launch:
 * bfq_probe_mfma_flops(blocks, iters). blocks in [1, 2^31), iters in [1, 2^40). */
bfq_status bfq_probe_mfma_peak(int64_t blocks, int64_t iters, float* out, void* stream);
double     bfq_probe_mfma_flops(int64_t blocks, int64_t iters);

/* Test support: the element encoder the quantizers use, applied to n fp32 values that are
 * finite with |x| < 464 (e4m3fn) or finite (int8). codes [n] bytes. */
bfq_status bfq_debug_encode(const float* x, int64_t n, bfq_dtype q_dtype, void* codes,
                            void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BFQ_H */
