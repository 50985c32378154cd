// Standard block-scaled GEMM for gfx950 ("variant 0"): one workgroup per BM x BN output
// tile, A (token codes) and W (weight codes) tiles of one 128-wide K block staged through
// LDS with direct global->LDS loads, double-buffered, consumed by MFMA, and the per-K-block
// scale applied in registers right after each block's product.
//
// Pages cited by title and section:
//   [BENCH]  "vLLM DeepGEMM FP8 Block GEMM 基准测试 ..." §4.2: the kernel walks K in
//            block-size steps and multiplies each step's dot product by the activation and
//            weight scales before accumulating; a grouped tile order improves L2 hits.
//   [CONFIG] "vLLM 量化 Kernel 配置机制 ..." §2: a launch is described by its tile sizes,
//            GROUP_SIZE_M, number of warps and pipeline stages.
//   [HELION] "Building a High-Performance and Portable vLLM Linear Backend with Helion",
//            kernel section: split-K divides the K range over several workgroups.
//
// gfx950 design:
//  * MFMA v_mfma_f32_16x16x128_f8f6f4 (e4m3) or v_mfma_i32_16x16x64_i8 (int8): one fp8
//    MFMA covers one whole 128-wide K block for a 16x16 sub-tile, so its result is the
//    block partial P and the scale step is acc = fma(P, sa[m,kb]*sw[nb,kb], acc).
//  * The weight fragment sits in the MFMA's first operand and the token fragment in the
//    second, so each lane ends up owning one token row and four consecutive output columns:
//    one scale product per lane and sub-tile row, and 8-byte (bf16) row-contiguous stores.
//  * LDS rows are 128 bytes (one K block); the 16-byte chunk c of row r is stored at slot
//    c ^ (r & 7) so the 16 rows a fragment read touches fall in different banks.
//  * Workgroup ids are remapped so that each XCD (ids i, i+8, i+16, ...) owns a contiguous
//    range of tiles, ordered in groups of GROUP_M tile rows, keeping shared A/W panels in
//    that XCD's L2.
#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

// Tile id -> (pid_m, pid_n): contiguous range per XCD, then grouped order within it.
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                            int group_m, int64_t& pid_m, int64_t& pid_n) {
    const int64_t T = tiles_m * tiles_n;
    const int64_t xcd = bid & 7, local = bid >> 3;
    const int64_t base = T >> 3, rem = T & 7;
    const int64_t j = xcd * base + (xcd < rem ? xcd : rem) + local;
    const int64_t per_group = (int64_t)group_m * tiles_n;
    const int64_t gid = j / per_group;
    const int64_t first_m = gid * group_m;
    const int64_t gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int64_t in_group = j - gid * per_group;
    pid_m = first_m + in_group % gsize;
    pid_n = in_group / gsize;
}

template <int BM, int BN, int WM, int WN, int QT, int OT, int GROUP_M>
__global__ __launch_bounds__(64 * WM * WN) void gemm_std_kernel(GemmArgs p) {
    constexpr int NWAVES = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;      // wave tile (tokens x weight rows)
    constexpr int SM = TM / 16, SN = TN / 16;      // 16x16 sub-tiles per wave
    constexpr int STAGE = (BM + BN) * 128;         // bytes per LDS stage
    constexpr int CHUNKS = (BM + BN) / 8;          // 1 KB load chunks per stage
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(128 % TN == 0, "a wave's columns must lie in one 128-wide scale block");
    static_assert(CHUNKS % NWAVES == 0, "load chunks must divide evenly over waves");
    constexpr int CPW = CHUNKS / NWAVES;

    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const int64_t M = p.M, N = p.N, K = p.K, KB = K / 128;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int64_t pid_m, pid_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, GROUP_M, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;

    const int split = p.split, z = blockIdx.z;
    const int64_t kb_begin = (int64_t)z * KB / split, kb_end = (int64_t)(z + 1) * KB / split;

    const uint8_t* A = static_cast<const uint8_t*>(p.a);
    const uint8_t* W = static_cast<const uint8_t*>(p.w);

    // Per-lane global source rows for this wave's load chunks (clamped into range so no
    // load ever leaves the buffers; clamped rows are never stored).
    const uint8_t* src[CPW];
    uint32_t lds_off[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int chunk = wave + NWAVES * i;
        const int r = chunk * 8 + (lane >> 3);                 // row within A rows then W rows
        const int slot = lane & 7;
        const int c = slot ^ (lane >> 3);                      // (r & 7) == lane >> 3
        if (r < BM) {
            int64_t m = m0 + r;
            m = m < M ? m : M - 1;
            src[i] = A + m * K + c * 16;
        } else {
            int64_t n = n0 + (r - BM);
            n = n < N ? n : N - 1;
            src[i] = W + n * K + c * 16;
        }
        lds_off[i] = (uint32_t)(chunk * 1024);
    }

    auto issue_stage = [&](int64_t kb, int stage) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            load_lds_16(src[i] + kb * 128, lds, lds_off[i] + stage * STAGE);
        }
    };

    // Token rows this lane owns in each sub-tile row, and their scale addresses.
    const float* sa_ptr[SM];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        int64_t m = m0 + wm * TM + sm * 16 + (lane & 15);
        m = m < M ? m : M - 1;
        sa_ptr[sm] = p.sa + m * p.sa_stride_m;
    }
    const int64_t nb = (n0 + wn * TN < N ? n0 + wn * TN : N - 1) / 128;
    const float* sw_row = p.sw + nb * KB;

    v4f acc[SM][SN];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) acc[sm][sn] = v4f{0.f, 0.f, 0.f, 0.f};

    // Fragment read offsets: lane l reads row (l % 16) of a sub-tile; chunk pair for fp8,
    // single chunk per K half for int8.
    const int frow = lane & 15;
    const int fgrp = lane >> 4;

    // Scales of the next K block are loaded one iteration ahead, before that block's
    // global->LDS loads, so waiting for them never waits for the tile prefetch.
    float sa_next[SM], sw_next = 0.f;
    auto load_scales = [&](int64_t kb) {
        sw_next = sw_row[kb];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) sa_next[sm] = sa_ptr[sm][kb * p.sa_stride_k];
    };

    if (kb_begin < kb_end) {
        load_scales(kb_begin);
        issue_stage(kb_begin, 0);
        wait_vmem_all();
        __syncthreads();
    }

    for (int64_t kb = kb_begin; kb < kb_end; ++kb) {
        const int stage = (int)((kb - kb_begin) & 1);
        float c[SM];
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) c[sm] = sa_next[sm] * sw_next;
        if (kb + 1 < kb_end) {
            load_scales(kb + 1);
            issue_stage(kb + 1, stage ^ 1);
        }

        const uint8_t* sA = lds + stage * STAGE;
        const uint8_t* sW = sA + BM * 128;

        if constexpr (QT == Q_FP8) {
            v8i af[SM];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const int r = wm * TM + sm * 16 + frow;
                const v4i lo = *reinterpret_cast<const v4i*>(sA + r * 128 + (((2 * fgrp) ^ (r & 7)) << 4));
                const v4i hi = *reinterpret_cast<const v4i*>(sA + r * 128 + (((2 * fgrp + 1) ^ (r & 7)) << 4));
                af[sm] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const int r = wn * TN + sn * 16 + frow;
                const v4i lo = *reinterpret_cast<const v4i*>(sW + r * 128 + (((2 * fgrp) ^ (r & 7)) << 4));
                const v4i hi = *reinterpret_cast<const v4i*>(sW + r * 128 + (((2 * fgrp + 1) ^ (r & 7)) << 4));
                const v8i wf = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) {
                    const v4f pb = mfma_fp8_16x16x128(wf, af[sm]);
                    acc[sm][sn].x = __builtin_fmaf(pb.x, c[sm], acc[sm][sn].x);
                    acc[sm][sn].y = __builtin_fmaf(pb.y, c[sm], acc[sm][sn].y);
                    acc[sm][sn].z = __builtin_fmaf(pb.z, c[sm], acc[sm][sn].z);
                    acc[sm][sn].w = __builtin_fmaf(pb.w, c[sm], acc[sm][sn].w);
                }
            }
        } else {
            v4i af[SM][2];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const int r = wm * TM + sm * 16 + frow;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    af[sm][h] = *reinterpret_cast<const v4i*>(sA + r * 128 + (((4 * h + fgrp) ^ (r & 7)) << 4));
            }
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const int r = wn * TN + sn * 16 + frow;
                const v4i w0 = *reinterpret_cast<const v4i*>(sW + r * 128 + (((fgrp) ^ (r & 7)) << 4));
                const v4i w1 = *reinterpret_cast<const v4i*>(sW + r * 128 + (((4 + fgrp) ^ (r & 7)) << 4));
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) {
                    v4i pi = mfma_i8_16x16x64(w0, af[sm][0], v4i{0, 0, 0, 0});
                    pi = mfma_i8_16x16x64(w1, af[sm][1], pi);
                    acc[sm][sn].x = __builtin_fmaf((float)pi.x, c[sm], acc[sm][sn].x);
                    acc[sm][sn].y = __builtin_fmaf((float)pi.y, c[sm], acc[sm][sn].y);
                    acc[sm][sn].z = __builtin_fmaf((float)pi.z, c[sm], acc[sm][sn].z);
                    acc[sm][sn].w = __builtin_fmaf((float)pi.w, c[sm], acc[sm][sn].w);
                }
            }
        }
        wait_vmem_all();
        __syncthreads();
    }

    // Epilogue: lane owns token m and columns n..n+3 of each sub-tile.
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        const int64_t m = m0 + wm * TM + sm * 16 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            const int64_t n = n0 + wn * TN + sn * 16 + 4 * fgrp;
            if (n >= N) continue;
            if (split == 1) store4<OT>(p.out, m * N + n, acc[sm][sn]);
            else store4<O_FP32>(p.partials, ((int64_t)z * M + m) * N + n, acc[sm][sn]);
        }
    }
}

template <int BM, int BN, int WM, int WN, int QT, int OT, int GROUP_M>
hipError_t launch_std(const GemmArgs& a, hipStream_t stream) {
    constexpr int STAGE = (BM + BN) * 128;
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles, 1, (unsigned)a.split);
    static bool attr_set = false;   // one-time opt-in to more than 64 KB of LDS
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_std_kernel<BM, BN, WM, WN, QT, OT, GROUP_M>),
            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemm_std_kernel<BM, BN, WM, WN, QT, OT, GROUP_M>), grid,
                       dim3(64 * WM * WN), 2 * STAGE, stream, a);
    return hipGetLastError();
}

#define BFQ_STD_ENTRY(BM, BN, WM, WN, GM, QT, OT)                                        \
    KernelEntry{bfq_tile{0, BM, BN, 128, 1, WM, WN, 2, GM, {0, 0, 0}}, QT, OT,            \
                &launch_std<BM, BN, WM, WN, QT, OT, GM>}

#define BFQ_STD_ALL_OUT(BM, BN, WM, WN, GM, QT)                                           \
    BFQ_STD_ENTRY(BM, BN, WM, WN, GM, QT, O_BF16), BFQ_STD_ENTRY(BM, BN, WM, WN, GM, QT, O_FP16), \
        BFQ_STD_ENTRY(BM, BN, WM, WN, GM, QT, O_FP32)

static const KernelEntry kStdKernels[] = {
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 8, Q_FP8),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 8, Q_FP8),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 8, Q_FP8),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 8, Q_FP8),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 8, Q_INT8),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 8, Q_INT8),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 8, Q_INT8),
};

const KernelEntry* std_kernels(int* count) {
    *count = (int)(sizeof(kStdKernels) / sizeof(kStdKernels[0]));
    return kStdKernels;
}

}  // namespace bfq
