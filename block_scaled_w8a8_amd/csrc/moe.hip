// MoE routing for the grouped block GEMM: the (token, expert) pairs q = t*topk + j are
// grouped by expert with a stable counting sort, giving per-expert row offsets and the pair
// ids in expert order, which the grouped GEMM kernels gather tokens and scatter outputs by.
//
// Page cited by title and section:
//   [CONFIG] "vLLM 量化 Kernel 配置机制 ..." §5: the MoE kernels take the same per-shape,
//            per-batch-size configs with an expert count E in the key.
//
// gfx950 design: three short kernels instead of one workgroup, so that 32K pairs (4096
// tokens x top-8) still sort in a few microseconds.
//   count:   one 1024-thread workgroup per chunk of 1024 pairs; an LDS histogram of the
//            chunk's experts, written to counts[e][chunk] (expert-major).
//   scan:    one workgroup; the exclusive prefix of counts in expert-major order gives each
//            (expert, chunk) its first output row, and offsets[e] = the row of (e, chunk 0).
//   scatter: per chunk again; each wave ranks its 64 pairs among equal experts with ballots
//            (one round per distinct expert in the wave), the per-wave counts are prefixed
//            across the chunk's 16 waves in LDS, and pair q goes to
//            base[e][chunk] + (pairs of e in earlier waves) + (rank in its wave).
// Stable: chunks, waves and lanes are taken in pair order. An expert id outside [0, E)
// falls into an extra bucket E after every expert, so offsets[E] counts the valid pairs.
// E <= kMoeMaxExperts keeps the scatter's per-wave counts within 64 KiB of LDS.
#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

constexpr int kAlignThreads = 1024;   // pairs per chunk, one per thread
constexpr int kAlignWaves = kAlignThreads / 64;

__device__ __forceinline__ int bucket_of(int32_t id, int E) { return (id >= 0 && id < E) ? id : E; }

__global__ __launch_bounds__(kAlignThreads) void moe_count_kernel(const int32_t* __restrict__ ids,
                                                                   int64_t pairs, int E,
                                                                   int32_t* __restrict__ counts) {
    extern __shared__ int32_t hist[];          // E + 1 buckets
    const int64_t g = blockIdx.x, G = gridDim.x;
    for (int b = threadIdx.x; b <= E; b += kAlignThreads) hist[b] = 0;
    __syncthreads();
    const int64_t q = g * kAlignThreads + threadIdx.x;
    if (q < pairs) atomicAdd(&hist[bucket_of(ids[q], E)], 1);
    __syncthreads();
    for (int b = threadIdx.x; b <= E; b += kAlignThreads) counts[(int64_t)b * G + g] = hist[b];
}

// Exclusive prefix over the (E + 1) x G counts in expert-major order, in place; offsets[e] =
// first row of expert e, offsets[E] = number of pairs with a valid expert.
__global__ __launch_bounds__(kAlignThreads) void moe_scan_kernel(int32_t* __restrict__ counts,
                                                                  int64_t G, int E,
                                                                  int32_t* __restrict__ offsets) {
    __shared__ int32_t part[kAlignThreads];
    if (G == 0) {                                  // no pairs: every expert is empty
        for (int b = threadIdx.x; b <= E; b += kAlignThreads) offsets[b] = 0;
        return;
    }
    const int64_t n = (int64_t)(E + 1) * G;
    const int64_t per = (n + kAlignThreads - 1) / kAlignThreads;
    const int64_t lo = threadIdx.x * per, hi = lo + per < n ? lo + per : n;
    int32_t s = 0;
    for (int64_t i = lo; i < hi; ++i) s += counts[i];
    part[threadIdx.x] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan of the per-thread sums
    for (int d = 1; d < kAlignThreads; d <<= 1) {
        const int32_t v = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
        __syncthreads();
        part[threadIdx.x] += v;
        __syncthreads();
    }
    int32_t run = threadIdx.x > 0 ? part[threadIdx.x - 1] : 0;
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t c = counts[i];
        counts[i] = run;
        if (i % G == 0) offsets[i / G] = run;      // (expert i / G, chunk 0)
        run += c;
    }
}

__global__ __launch_bounds__(kAlignThreads) void moe_scatter_kernel(const int32_t* __restrict__ ids,
                                                                     int64_t pairs, int E,
                                                                     const int32_t* __restrict__ base,
                                                                     int32_t* __restrict__ sorted) {
    extern __shared__ int32_t wcnt[];          // [kAlignWaves][E + 1]
    const int64_t g = blockIdx.x, G = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int B = E + 1;
    for (int i = threadIdx.x; i < kAlignWaves * B; i += kAlignThreads) wcnt[i] = 0;
    __syncthreads();
    const int64_t q = g * kAlignThreads + threadIdx.x;
    const bool valid = q < pairs;
    const int b = valid ? bucket_of(ids[q], E) : -1;
    // rank among the wave's earlier lanes with the same bucket, one round per distinct bucket
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int rank = 0;
    uint64_t pending = __ballot(valid);
    while (pending) {
        const int leader = __builtin_ctzll(pending);
        const int bl = __shfl(b, leader, 64);
        const uint64_t m = __ballot(valid && b == bl);
        if (valid && b == bl) rank = __builtin_popcountll(m & below);
        if (lane == leader) wcnt[wave * B + bl] = __builtin_popcountll(m);
        pending &= ~m;
    }
    __syncthreads();
    // exclusive prefix over the waves, per bucket
    for (int bb = threadIdx.x; bb < B; bb += kAlignThreads) {
        int32_t run = 0;
        for (int w = 0; w < kAlignWaves; ++w) {
            const int32_t c = wcnt[w * B + bb];
            wcnt[w * B + bb] = run;
            run += c;
        }
    }
    __syncthreads();
    if (valid) sorted[base[(int64_t)b * G + g] + wcnt[wave * B + b] + rank] = (int32_t)q;
}

size_t moe_align_workspace_bytes(int64_t pairs, int E) {
    const int64_t G = pairs > 0 ? (pairs + kAlignThreads - 1) / kAlignThreads : 0;
    return (size_t)(E + 1) * (size_t)G * sizeof(int32_t);
}

hipError_t launch_moe_align(const int32_t* ids, int64_t pairs, int E, int32_t* offsets,
                            int32_t* sorted, int32_t* counts, hipStream_t stream) {
    const int64_t G = (pairs + kAlignThreads - 1) / kAlignThreads;
    const size_t hist_bytes = (size_t)(E + 1) * sizeof(int32_t);
    if (G == 0) {
        hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(kAlignThreads), 0, stream, counts, G, E,
                           offsets);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)G), dim3(kAlignThreads), hist_bytes, stream,
                       ids, pairs, E, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(kAlignThreads), 0, stream, counts, G, E, offsets);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_scatter_kernel, dim3((unsigned)G), dim3(kAlignThreads),
                       hist_bytes * kAlignWaves, stream, ids, pairs, E, counts, sorted);
    return hipGetLastError();
}

}  // namespace bfq
