// Decode-shaped block-scaled GEMM for gfx950 ("variant 1", swap-AB streaming) plus the
// deterministic split-K reduction and the int8 block-partials probe.
//
// Pages cited by title and section:
//   [HELION] "Building a High-Performance and Portable vLLM Linear Backend with Helion",
//            kernel section: swap-AB computes the product transposed so that a small M
//            does not waste the wide tile dimension; split-K splits the K range over
//            workgroups to add parallelism when M and/or N are small; the Hopper heuristic
//            picks swap-AB below 32 tokens.
//   [BENCH]  "vLLM DeepGEMM FP8 Block GEMM 基准测试 ..." §4.3: for small m the kernel is
//            bandwidth bound, so GB/s is the number that matters.
//
// gfx950 design: with M <= 64 tokens the whole cost is streaming the weight codes once from
// HBM. Each wave owns NWR weight rows and loads their 16x128-byte MFMA fragments straight
// from global memory into registers (no LDS round trip), keeping D K-blocks in flight in a
// register ring. The token codes (at most 64 x K bytes, L2-resident) ride in the second
// MFMA operand, so the result tile is W*A^T: each lane holds one token and four
// consecutive weight rows, stored back row-major into C. Lane l loads 16-byte chunks
// (l/16) and (l/16)+4 of its row, so each load instruction covers 64 contiguous bytes of
// 16 rows. Split-K writes fp32 partials that a second kernel sums in a fixed order.
#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

template <int MT, int NWR, int NWAVES, int D, int QT, int OT>
__global__ __launch_bounds__(64 * NWAVES) void gemm_swapab_kernel(GemmArgs p) {
    constexpr int SM = MT / 16, SN = NWR / 16;
    static_assert(MT % 16 == 0 && NWR % 16 == 0, "tiles are multiples of 16");
    static_assert(128 % NWR == 0, "a wave's rows must lie in one 128-row scale block");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int frow = lane & 15, fgrp = lane >> 4;

    const int64_t M = p.M, N = p.N, K = p.K, KB = K / 128;
    const int64_t n0 = ((int64_t)blockIdx.x * NWAVES + wave) * NWR;
    const int64_t m0 = (int64_t)blockIdx.y * MT;
    const int split = p.split, z = blockIdx.z;
    const int64_t kb_begin = (int64_t)z * KB / split, kb_end = (int64_t)(z + 1) * KB / split;
    const bool wave_live = n0 < N;   // whole-wave predicate (N is a multiple of 16)

    const uint8_t* W = static_cast<const uint8_t*>(p.w);
    const uint8_t* A = static_cast<const uint8_t*>(p.a);

    const uint8_t* wrow[SN];
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
        int64_t n = n0 + sn * 16 + frow;
        n = n < N ? n : N - 1;
        wrow[sn] = W + n * K + fgrp * 16;
    }
    const uint8_t* arow[SM];
    const float* sa_ptr[SM];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        int64_t m = m0 + sm * 16 + frow;
        m = m < M ? m : M - 1;
        arow[sm] = A + m * K + fgrp * 16;
        sa_ptr[sm] = p.sa + m * p.sa_stride_m;
    }
    const float* sw_row = p.sw + ((wave_live ? n0 : 0) / 128) * KB;

    v4i wbuf[D][SN][2];
    v4i abuf[D][SM][2];
    float sab[D][SM];
    float swb[D];

    auto fetch = [&](int slot, int64_t kb) {
        swb[slot] = sw_row[kb];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) sab[slot][sm] = sa_ptr[sm][kb * p.sa_stride_k];
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            wbuf[slot][sn][0] = *reinterpret_cast<const v4i*>(wrow[sn] + kb * 128);
            wbuf[slot][sn][1] = *reinterpret_cast<const v4i*>(wrow[sn] + kb * 128 + 64);
        }
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            abuf[slot][sm][0] = *reinterpret_cast<const v4i*>(arow[sm] + kb * 128);
            abuf[slot][sm][1] = *reinterpret_cast<const v4i*>(arow[sm] + kb * 128 + 64);
        }
    };

    v4f acc[SM][SN];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) acc[sm][sn] = v4f{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](int i) {
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            const float c = sab[i][sm] * swb[i];
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                v4f pb;
                if constexpr (QT == Q_FP8) {
                    const v4i* w2 = wbuf[i][sn];
                    const v4i* a2 = abuf[i][sm];
                    const v8i wf = v8i{w2[0].x, w2[0].y, w2[0].z, w2[0].w,
                                       w2[1].x, w2[1].y, w2[1].z, w2[1].w};
                    const v8i af = v8i{a2[0].x, a2[0].y, a2[0].z, a2[0].w,
                                       a2[1].x, a2[1].y, a2[1].z, a2[1].w};
                    pb = mfma_fp8_16x16x128(wf, af);
                } else {
                    v4i pi = mfma_i8_16x16x64(wbuf[i][sn][0], abuf[i][sm][0], v4i{0, 0, 0, 0});
                    pi = mfma_i8_16x16x64(wbuf[i][sn][1], abuf[i][sm][1], pi);
                    pb = v4f{(float)pi.x, (float)pi.y, (float)pi.z, (float)pi.w};
                }
                acc[sm][sn].x = __builtin_fmaf(pb.x, c, acc[sm][sn].x);
                acc[sm][sn].y = __builtin_fmaf(pb.y, c, acc[sm][sn].y);
                acc[sm][sn].z = __builtin_fmaf(pb.z, c, acc[sm][sn].z);
                acc[sm][sn].w = __builtin_fmaf(pb.w, c, acc[sm][sn].w);
            }
        }
    };

    if (wave_live && kb_begin < kb_end) {
        // Ring of D K-blocks in flight. The steady-state loop is branch-free: a refill past
        // the end of this split re-reads its last block (never used), so the compiler can
        // count outstanding loads exactly instead of draining the queue at every join.
        const int64_t kb_last = kb_end - 1;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int64_t kb = kb_begin + i;
            fetch(i, kb < kb_last ? kb : kb_last);
        }
        int64_t kb0 = kb_begin;
        for (; kb0 + D <= kb_end; kb0 += D) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                // keep each slot's work in its own stage: the scheduler must not hoist the
                // scale products of later slots (that would wait for every load in flight)
                __builtin_amdgcn_sched_barrier(0);
                consume(i);
                const int64_t nk = kb0 + i + D;
                fetch(i, nk < kb_last ? nk : kb_last);
            }
        }
        const int rem = (int)(kb_end - kb0);
#pragma unroll
        for (int i = 0; i < D; ++i)
            if (i < rem) consume(i);

#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            const int64_t m = m0 + sm * 16 + frow;
            if (m >= M) continue;
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const int64_t n = n0 + sn * 16 + 4 * fgrp;
                if (split == 1) store4<OT>(p.out, m * N + n, acc[sm][sn]);
                else store4<O_FP32>(p.partials, ((int64_t)z * M + m) * N + n, acc[sm][sn]);
            }
        }
    }
}

template <int MT, int NWR, int NWAVES, int D, int QT, int OT>
hipError_t launch_swapab(const GemmArgs& a, hipStream_t stream) {
    const int64_t strips = (a.N + NWR * NWAVES - 1) / (NWR * NWAVES);
    dim3 grid((unsigned)strips, (unsigned)((a.M + MT - 1) / MT), (unsigned)a.split);
    hipLaunchKernelGGL((gemm_swapab_kernel<MT, NWR, NWAVES, D, QT, OT>), grid,
                       dim3(64 * NWAVES), 0, stream, a);
    return hipGetLastError();
}

#define BFQ_SAB_ENTRY(MT, NWR, NW, D, QT, OT)                                              \
    KernelEntry{bfq_tile{1, MT, NWR * NW, 128, 1, 1, NW, D, 1, 0, 0, 0}, QT, OT,          \
                &launch_swapab<MT, NWR, NW, D, QT, OT>}
#define BFQ_SAB_ALL_OUT(MT, NWR, NW, D, QT)                                                \
    BFQ_SAB_ENTRY(MT, NWR, NW, D, QT, O_BF16), BFQ_SAB_ENTRY(MT, NWR, NW, D, QT, O_FP16),   \
        BFQ_SAB_ENTRY(MT, NWR, NW, D, QT, O_FP32)

static const KernelEntry kSwapabKernels[] = {
    BFQ_SAB_ALL_OUT(16, 32, 4, 4, Q_FP8),
    BFQ_SAB_ALL_OUT(16, 16, 4, 8, Q_FP8),
    BFQ_SAB_ALL_OUT(16, 16, 8, 8, Q_FP8),
    BFQ_SAB_ALL_OUT(16, 32, 8, 4, Q_FP8),
    BFQ_SAB_ALL_OUT(16, 64, 4, 2, Q_FP8),
    BFQ_SAB_ALL_OUT(16, 32, 4, 8, Q_FP8),
    BFQ_SAB_ALL_OUT(32, 32, 4, 4, Q_FP8),
    BFQ_SAB_ALL_OUT(64, 32, 4, 2, Q_FP8),
    BFQ_SAB_ALL_OUT(16, 32, 4, 4, Q_INT8),
    BFQ_SAB_ALL_OUT(32, 32, 4, 4, Q_INT8),
    BFQ_SAB_ALL_OUT(64, 32, 4, 2, Q_INT8),
};

const KernelEntry* swapab_kernels(int* count) {
    *count = (int)(sizeof(kSwapabKernels) / sizeof(kSwapabKernels[0]));
    return kSwapabKernels;
}

// ------------------------------------------------------------ split-K reduce ----
template <int OT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            void* __restrict__ out,
                                                            int64_t MN, int split) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;                       // MN is a multiple of 128
    v4f s = *reinterpret_cast<const v4f*>(part + i);
    for (int z = 1; z < split; ++z) {
        const v4f t = *reinterpret_cast<const v4f*>(part + (int64_t)z * MN + i);
        s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
    }
    store4<OT>(out, i, s);
}

hipError_t launch_splitk_reduce(const float* partials, void* out, int64_t M, int64_t N,
                                int split, int otype, hipStream_t stream) {
    const int64_t MN = M * N;
    dim3 grid((unsigned)((MN / 4 + 255) / 256));
    if (otype == O_BF16)
        hipLaunchKernelGGL(splitk_reduce_kernel<O_BF16>, grid, dim3(256), 0, stream, partials, out, MN, split);
    else if (otype == O_FP16)
        hipLaunchKernelGGL(splitk_reduce_kernel<O_FP16>, grid, dim3(256), 0, stream, partials, out, MN, split);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<O_FP32>, grid, dim3(256), 0, stream, partials, out, MN, split);
    return hipGetLastError();
}

// ------------------------------------------------------------ int8 partials probe ----
// One wave per (16 weight rows, 16 tokens, K block): the same two chained int8 MFMAs the
// GEMM kernels use, written out as exact int32 block partials [K/128][M][N].
__global__ __launch_bounds__(64) void block_partials_i32_kernel(const int8_t* __restrict__ A,
                                                                const int8_t* __restrict__ W,
                                                                int32_t* __restrict__ out,
                                                                int64_t M, int64_t N, int64_t K) {
    const int lane = threadIdx.x, frow = lane & 15, fgrp = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16, kb = blockIdx.z;
    int64_t n = n0 + frow, m = m0 + frow;
    m = m < M ? m : M - 1;
    const int8_t* wr = W + n * K + kb * 128 + fgrp * 16;
    const int8_t* ar = A + m * K + kb * 128 + fgrp * 16;
    v4i pi = mfma_i8_16x16x64(*reinterpret_cast<const v4i*>(wr), *reinterpret_cast<const v4i*>(ar),
                              v4i{0, 0, 0, 0});
    pi = mfma_i8_16x16x64(*reinterpret_cast<const v4i*>(wr + 64), *reinterpret_cast<const v4i*>(ar + 64), pi);
    const int64_t mo = m0 + frow;
    if (mo < M) {
        int32_t* o = out + (kb * M + mo) * N + n0 + 4 * fgrp;
        *reinterpret_cast<v4i*>(o) = pi;
    }
}

hipError_t launch_block_partials_i32(const void* a, const void* w, int32_t* out, int64_t M,
                                     int64_t N, int64_t K, hipStream_t stream) {
    dim3 grid((unsigned)(N / 16), (unsigned)((M + 15) / 16), (unsigned)(K / 128));
    hipLaunchKernelGGL(block_partials_i32_kernel, grid, dim3(64), 0, stream, (const int8_t*)a,
                       (const int8_t*)w, out, M, N, K);
    return hipGetLastError();
}

}  // namespace bfq
