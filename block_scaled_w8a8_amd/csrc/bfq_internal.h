// Internal declarations of libbfq: kernel launchers and the registry of compiled GEMM
// configurations. Not part of the public C-ABI (include/bfq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bfq.h"

namespace bfq {

enum QType { Q_FP8 = 0, Q_INT8 = 1 };
enum OType { O_BF16 = 0, O_FP16 = 1, O_FP32 = 2 };
enum WLayout { W_ROW = 0, W_PACKED16 = 1 };   // bfq_weight_layout
// How a kernel applies scales: per 128-wide K block, any fp32 values (S_FP32) or powers of two
// only (S_UE8M0, bfq_scale_format); or one scale per token and per output channel after the
// whole-K product (S_CHANNEL, block_shape {1, K}); or UE8M0 block scales whose activation
// scales arrive as packed words (S_PACKED, BFQ_SCALES_PACKED_UE8M0). The standard and
// stream-K kernels read packed words through a runtime flag, so every block-scale kernel of
// variants 0 and 2 also serves S_PACKED; the swap-AB kernels have S_PACKED instances.
enum ScaleFmt { S_FP32 = 0, S_UE8M0 = 1, S_CHANNEL = 2, S_PACKED = 3 };

// Largest K of the per-token / per-channel format (the row quantizer keeps a row in registers).
constexpr int64_t kChannelMaxK = 32768;

// packed: BFQ_SCALES_PACKED_UE8M0 words (s_stride_g = words between word rows).
hipError_t launch_quant_tokens(const void* x, void* q, float* scales, int64_t M, int64_t K,
                               int qtype, int64_t s_stride_m, int64_t s_stride_g, float eps,
                               int sfmt, int packed, hipStream_t stream);
hipError_t launch_quant_weight_blocks(const float* w, void* q, float* scales, int64_t N,
                                      int64_t K, int qtype, float eps, int sfmt,
                                      hipStream_t stream);
// One scale per row: bf16 token rows (is_f32 = 0) or fp32 weight rows (is_f32 = 1) of length
// K <= kChannelMaxK; row r's scale goes to scales[r * s_stride].
hipError_t launch_quant_rows(const void* x, int is_f32, void* q, float* scales, int64_t rows,
                             int64_t K, int qtype, int64_t s_stride, float eps, int sfmt,
                             hipStream_t stream);
// Row-major [N][K] codes -> the packed 16-row fragment layout (BFQ_W_PACKED16).
hipError_t launch_pack_weights(const void* w, void* packed, int64_t N, int64_t K,
                               hipStream_t stream);
hipError_t launch_debug_encode(const float* x, int64_t n, int qtype, void* out,
                               hipStream_t stream);

// Arguments of one block-GEMM launch, shared by every kernel variant.
struct GemmArgs {
    const void* a;          // [M][K] codes
    const float* sa;        // activation scales
    int64_t sa_stride_m;    // element stride between tokens
    int64_t sa_stride_k;    // element stride between K blocks (packed: between word rows)
    int sa_packed;          // 1: activation scales are packed UE8M0 words (4 K blocks each)
    const void* w;          // N*K codes, row-major or packed (the kernel's layout)
    const float* sw;        // [N/128][K/128] (S_CHANNEL: [N])
    void* out;              // [M][N]
    float* partials;        // split-K fp32 partials [split][M][N] (split > 1)
    int64_t M, N, K;
    int split;              // K-block chunks
    int group_m;            // tile rows per group of the grouped order (standard kernel)
    int raster;             // 0: XCD-contiguous tile ranges, 1: plain order (standard kernel)
    // stream-K schedule (variant 2) only:
    int64_t dp_tiles;       // tiles [0, dp_tiles) taken whole, in rounds of the grid size
    float* sk_slots;        // [grid][2][BM*BN] fp32 partial tiles
    // MoE grouped GEMM only (M = pairs, the output rows; a holds moe_tokens rows):
    const int32_t* moe_rows;      // [pairs] pair ids q = t*topk + j, grouped by expert
    const int32_t* moe_offsets;   // [E + 1] first grouped row of each expert
    int64_t moe_tokens;           // rows of a and of the activation scales
    int moe_topk, moe_experts;    // token of pair q = q / topk; E
};

// MoE routing: stable sort of pair ids by expert (csrc/moe.hip). counts = workspace of
// moe_align_workspace_bytes(pairs, E) bytes.
constexpr int kMoeMaxExperts = 1023;
size_t moe_align_workspace_bytes(int64_t pairs, int E);
hipError_t launch_moe_align(const int32_t* ids, int64_t pairs, int E, int32_t* offsets,
                            int32_t* sorted, int32_t* counts, hipStream_t stream);
// Upper bound on the per-expert row tiles of height bm over `pairs` rows and E experts (the
// grid height of a grouped launch): sum_e ceil(rows_e / bm) <= ceil(pairs / bm) + min(E, pairs).
inline int64_t moe_max_tiles(int64_t pairs, int64_t E, int64_t bm) {
    return (pairs + bm - 1) / bm + (E < pairs ? E : pairs);
}

typedef hipError_t (*GemmLaunchFn)(const GemmArgs& args, hipStream_t stream);

// A compiled kernel configuration. split_k, group_m and raster are launch arguments.
struct KernelEntry {
    bfq_tile tile;
    int qtype;              // Q_FP8 / Q_INT8
    int otype;              // O_BF16 / O_FP16 / O_FP32 (output of a split=1 launch)
    int wlayout;            // W_ROW / W_PACKED16: the weight layout the kernel reads
    int sfmt;               // S_FP32: any fp32 block scales; S_UE8M0: power-of-two block
                            // scales only; S_CHANNEL: per-token x per-channel scales
    GemmLaunchFn launch;    // writes `out` (split==1) or `partials` (split>1)
    int moe;                // 1: the grouped (MoE) form of the kernel
};

// Registries filled by the kernel translation units.
const KernelEntry* std_kernels(int* count);
const KernelEntry* swapab_kernels(int* count);
const KernelEntry* streamk_kernels(int* count);
// grouped (MoE) forms of variants 0 and 1 (KernelEntry::moe = 1)
const KernelEntry* moe_std_kernels(int* count);
const KernelEntry* moe_swapab_kernels(int* count);

// Stream-K: workspace (two fp32 partial-tile slots per workgroup of a `grid`-workgroup grid),
// the split of `tiles` into whole-tile rounds and the stream-K remainder, and the grid size
// (the device's compute units).
size_t streamk_workspace_bytes(int bm, int bn, int grid);
int64_t streamk_dp_tiles(int64_t tiles, int grid);
int streamk_grid();

// Deterministic split-K reduction: out[m][n] = sum_{s=0..split-1} partials[s][m][n], in
// ascending s, converted once to the output dtype.
hipError_t launch_splitk_reduce(const float* partials, void* out, int64_t M, int64_t N,
                                int split, int otype, hipStream_t stream);

// Measurement support (csrc/probe.hip): fp8 MFMA chains with no memory traffic.
hipError_t launch_mfma_peak(int64_t blocks, int64_t iters, float* out, hipStream_t stream);
int mfma_peak_threads_per_block();
int mfma_peak_mfmas_per_wave_iter();

// int8 per-K-block int32 partials [K/128][M][N] (test support).
hipError_t launch_block_partials_i32(const void* a, const void* w, int32_t* out, int64_t M,
                                     int64_t N, int64_t K, hipStream_t stream);

}  // namespace bfq
