// Ring block-scaled GEMM for gfx950 ("variant 2"): one workgroup per BM x BN output tile for
// large M. Weight tiles stream through a 4-slot LDS ring; each wave loads its own token rows
// straight into a register ring; the per-K-block scale is applied in registers right after
// each block's product, as in the standard kernel.
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
// Why a second large-tile kernel. With A and W both staged through LDS, a 256x256 tile needs
// 64 KiB per K block, so only two stages fit in 160 KiB and every load has one block of
// compute to land. Here only W goes through LDS (32 KiB per block for BN = 256), so four
// ring slots fit; the tokens skip LDS and go straight to the registers of the waves that
// use them (waves sharing token rows each load them; the second read hits L2).
//
// Vector-memory operations complete in issue order, so a wait for a token fragment also
// waits for every weight DMA issued before it: the slack a load really gets is set by the
// order of issue. Per K block kb a wave issues, after the block's barrier,
//     token fragments of kb+AD-1  (2 x 16 B per lane and 16-token sub-tile, register slot
//                                  (kb+AD-1) % AD)
//     scales and W tile of kb+3   (2 dword DMAs + BN/8/NW 1-KiB DMAs, LDS slot (kb+3) % 4)
// and then computes kb. The W slot written at kb is the one read at kb-1, which every wave
// has left once it passes the barrier of kb. Past the last block the loads are clamped to
// the last block (their targets are slots nobody reads again), so every block issues the
// same loads and the wait counts are constants.
//
// Layout of one wave's work: TM = 16*TS tokens (TS sub-tiles t) x TN = BN/WN weight rows
// (TN/16 sub-tiles s). The weight fragment is the MFMA's first operand, so lane l ends up
// owning token (t*16 + l%16) and four consecutive output columns of sub-tile s; the scale
// of (t, s) is sa[token][kb] * sw[its 128-row block][kb].
#include <type_traits>

#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

template <int WM, int WN, int TS, int AD, int QT, int OT, int SCHED>
__global__ __launch_bounds__(64 * WM * WN) void gemm_ring_kernel(GemmArgs p) {
    constexpr int NW = WM * WN;
    constexpr int BN = 256;                // weight rows per workgroup
    constexpr int TM = 16 * TS;            // tokens per wave
    constexpr int BM = WM * TM;            // tokens per workgroup
    constexpr int TN = BN / WN;            // weight rows per wave
    constexpr int SN = TN / 16;            // weight sub-tiles per wave
    constexpr int NS = 4;                  // LDS ring slots (W tile + scales of one K block)
    constexpr int WSLOT = BN * 128;        // W bytes per slot
    constexpr int CPW = BN / 8 / NW;       // 1-KiB W DMA chunks per wave per block
    constexpr int SC_WAVE = 512;           // per wave and slot: 64 sa words, then 64 sw words
    constexpr int SC_BASE = NS * WSLOT;
    constexpr int SC_SLOT = NW * SC_WAVE;
    constexpr int LOADS_PER_BLOCK = 2 * TS + 2 + CPW;
    static_assert(TS == 2 || TS == 4, "two or four token sub-tiles per wave");
    static_assert(AD == 2 || AD == 3, "token fragments issued one or two blocks ahead");
    static_assert(TN % 128 == 0, "a wave's columns cover whole 128-row scale blocks");
    static_assert((BN / 8) % NW == 0, "W chunks must divide evenly over waves");
    static_assert(NW % 2 == 0, "the swizzle phase of a lane's W chunks needs an even wave count");

    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & 15;     // token within a sub-tile / W row within a sub-tile
    const int fgrp = lane >> 4;     // 32-byte K group (fp8) / 16-byte K chunk (int8)

    const int64_t M = p.M, N = p.N, K = p.K, KB = K / 128;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int64_t pid_m, pid_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, p.group_m, p.raster, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;

    const int split = p.split, z = blockIdx.z;
    const int64_t kb_begin = (int64_t)z * KB / split, kb_end = (int64_t)(z + 1) * KB / split;

    // Buffer resources over this tile's rows: rows past M (N) read as zero and are never
    // stored. K <= 2^23 and at most 256 rows keep every offset below 2^31.
    const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_w = (N - n0) < BN ? (N - n0) : BN;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(static_cast<const uint8_t*>(p.a) + m0 * K, (uint32_t)(rows_a * K));
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(static_cast<const uint8_t*>(p.w) + n0 * K, (uint32_t)(rows_w * K));

    // Token fragments: sub-tile t, lane l reads row wm*TM + t*16 + l%16 at K bytes
    // [32g, 32g+32) (fp8, g = l/16) or chunks g and g+4 (int8: one per 64-wide MFMA).
    constexpr uint32_t A_HI = QT == Q_FP8 ? 16 : 64;
    const uint32_t a_voff = (uint32_t)((wm * TM + frow) * K) + (uint32_t)(QT == Q_FP8 ? 32 * fgrp : 16 * fgrp);

    // Scales. DMA lane l < 16*TS of a wave fetches sa of token wm*TM + (l%TS)*16 + l/TS into
    // word l of the wave's slot region (further lanes repeat, into unused words), so lane l
    // later reads its TS tokens' scales as one vector at word TS*(l%16). Lane l also fetches
    // sw of the tile's 128-row block min(l, blocks-1) into word 64 + l.
    const int64_t ssm = p.sa_stride_m, ssk = p.sa_stride_k;
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
        p.sa + m0 * ssm, (uint32_t)(((rows_a - 1) * ssm + (KB - 1) * ssk + 1) * 4));
    uint32_t sa_voff;
    {
        const int l = lane % (16 * TS);
        const int r = wm * TM + (l % TS) * 16 + l / TS;
        sa_voff = (uint32_t)(r * ssm * 4);
    }
    const int64_t nb0 = n0 / 128, nbs = (rows_w + 127) / 128;
    const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.sw + nb0 * KB, (uint32_t)(nbs * KB * 4));
    const uint32_t sw_voff = (uint32_t)(((int64_t)lane < nbs ? lane : nbs - 1) * KB * 4);
    const int hb = (wn * TN) / 128;     // first scale block of the wave's columns

    // W DMA: chunk i of this wave covers tile rows 8*(wave + NW*i) .. +7; lane l writes LDS
    // slot (l & 7) of row +(l >> 3), which holds global chunk (l & 7) ^ swz(row). As NW is
    // even, swz(row) = (l >> 3) ^ (wave & 1) for every i: one per-lane offset serves all
    // chunks and the chunk's row offset goes into the scalar offset.
    const uint32_t w_dma_voff = (uint32_t)(((lane >> 3) + wave * 8) * K +
                                           (((lane & 7) ^ (lane >> 3) ^ (wave & 1)) << 4));

    auto clampk = [&](int64_t kb) { return kb < kb_end ? kb : kb_end - 1; };

    auto issue_w = [&](int64_t kb, int slot) {
        const uint32_t sc = (uint32_t)(SC_BASE + slot * SC_SLOT + wave * SC_WAVE);
        dma4(rsa, lds, sc, sa_voff, (uint32_t)(kb * ssk * 4));
        dma4(rsw, lds, sc + 256, sw_voff, (uint32_t)(kb * 4));
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            dma16(rw, lds, (uint32_t)(slot * WSLOT + (wave + NW * i) * 1024), w_dma_voff,
                  (uint32_t)(kb * 128) + (uint32_t)(NW * i * 8 * K));
    };

    auto issue_a = [&](int64_t kb, v8i (&dst)[TS]) {
        const uint32_t skb = (uint32_t)(kb * 128);
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            const uint32_t vo = a_voff + (uint32_t)(t * 16 * K);
            const v4i lo = buf_b128(ra, vo, skb), hi = buf_b128(ra, vo + A_HI, skb);
            dst[t] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
    };

    v4f acc[TS][SN];
#pragma unroll
    for (int t = 0; t < TS; ++t)
#pragma unroll
        for (int s = 0; s < SN; ++s) acc[t][s] = v4f{0.f, 0.f, 0.f, 0.f};

    const int fsw = swz(frow);
    // fp8: the lane's 32-byte K group is chunks 2g, 2g+1; int8: chunks g and g+4.
    const uint32_t c0 = (uint32_t)(((QT == Q_FP8 ? 2 * fgrp : fgrp) ^ fsw) << 4);
    const uint32_t c1 = (uint32_t)(((QT == Q_FP8 ? 2 * fgrp + 1 : fgrp + 4) ^ fsw) << 4);
    const uint32_t w_row = (uint32_t)((wn * TN + frow) * 128);

    auto lds16 = [&](uint32_t off) { return *reinterpret_cast<const v4i*>(lds + off); };

    auto fma4 = [](v4f& a, const v4f& q, float cc) {
        a.x = __builtin_fmaf(q.x, cc, a.x);
        a.y = __builtin_fmaf(q.y, cc, a.y);
        a.z = __builtin_fmaf(q.z, cc, a.z);
        a.w = __builtin_fmaf(q.w, cc, a.w);
    };

    // Product of one 16x16 sub-tile for one K block (fp32 for fp8; exact int32 -> fp32 for
    // int8, |P| <= 128*127*127 < 2^24).
    auto block_product = [](const v8i& wf, const v8i& af) -> v4f {
        if constexpr (QT == Q_FP8) {
            return mfma_fp8_16x16x128(wf, af);
        } else {
            v4i pi = mfma_i8_16x16x64(v4i{wf[0], wf[1], wf[2], wf[3]}, v4i{af[0], af[1], af[2], af[3]},
                                      v4i{0, 0, 0, 0});
            pi = mfma_i8_16x16x64(v4i{wf[4], wf[5], wf[6], wf[7]}, v4i{af[4], af[5], af[6], af[7]}, pi);
            return v4f{(float)pi.x, (float)pi.y, (float)pi.z, (float)pi.w};
        }
    };

    // Scale products c[t][h] = sa[token t] * sw[block hb + h] of the block in ring slot
    // `slot`. Read with completed inline-asm LDS loads: a plain load here would make the
    // compiler drain every in-flight DMA first.
    auto read_scales = [&](int slot, float (&c)[TS][2]) {
        const uint32_t sc = (uint32_t)(SC_BASE + slot * SC_SLOT + wave * SC_WAVE);
        const float2 sw2 = lds_read_f32x2(lds, sc + 256 + hb * 4);
        float sa[TS];
        if constexpr (TS == 2) {
            const float2 v = lds_read_f32x2(lds, sc + frow * 8);
            sa[0] = v.x; sa[1] = v.y;
        } else {
            const v4f v = lds_read_f32x4(lds, sc + frow * 16);
            sa[0] = v.x; sa[1] = v.y; sa[2] = v.z; sa[3] = v.w;
        }
#pragma unroll
        for (int t = 0; t < TS; ++t) { c[t][0] = sa[t] * sw2.x; c[t][1] = sa[t] * sw2.y; }
    };

    auto compute = [&](int slot, const v8i (&af)[TS], const float (&c)[TS][2]) {
        const uint32_t wbase = (uint32_t)(slot * WSLOT) + w_row;
        auto read_w = [&](int s) {
            const v4i lo = lds16(wbase + s * 2048 + c0);
            const v4i hi = lds16(wbase + s * 2048 + c1);
            return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        };
        if constexpr (SCHED == 0) {
#pragma unroll
            for (int s = 0; s < SN; ++s) {
                const v8i wf = read_w(s);
#pragma unroll
                for (int t = 0; t < TS; ++t) fma4(acc[t][s], block_product(wf, af[t]), c[t][(s * 16) / 128]);
            }
        } else {
            // software-pipelined: the read of sub-tile s+1 and the MFMAs of s go out before the
            // scale FMAs of s-1, whose MFMAs have finished by then
            v8i wf = read_w(0);
            v4f pb[2][TS];
#pragma unroll
            for (int s = 0; s < SN; ++s) {
#pragma unroll
                for (int t = 0; t < TS; ++t) pb[s & 1][t] = block_product(wf, af[t]);
                if (s + 1 < SN) wf = read_w(s + 1);
                if (s > 0) {
#pragma unroll
                    for (int t = 0; t < TS; ++t) fma4(acc[t][s - 1], pb[(s - 1) & 1][t], c[t][((s - 1) * 16) / 128]);
                }
            }
#pragma unroll
            for (int t = 0; t < TS; ++t) fma4(acc[t][SN - 1], pb[(SN - 1) & 1][t], c[t][((SN - 1) * 16) / 128]);
        }
    };

    v8i afr[AD][TS];

    // One K block. J = (kb - kb_begin) % AD is the register-ring slot of kb's tokens (a
    // compile-time index, so the ring stays in registers).
    auto step = [&](int64_t kb, auto jc) {
        constexpr int J = decltype(jc)::value;
        const int slot = (int)((kb - kb_begin) & (NS - 1));
        // the W tile and scales of kb were issued three blocks ago, and two blocks' loads
        // have been issued since
        wait_vmem_keep(2 * LOADS_PER_BLOCK);
        barrier_no_fence();
        float c[TS][2];
        read_scales(slot, c);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(clampk(kb + AD - 1), afr[(J + AD - 1) % AD]);
        issue_w(clampk(kb + 3), (slot + 3) & (NS - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(slot, afr[J], c);
    };

    if (kb_begin < kb_end) {
        // Prologue: the issues of steps -3, -2, -1 of the steady state (step s issues
        // A(s+AD-1), then W(s+3)), so that at every block exactly two blocks' loads are younger
        // than that block's W tile and the wait above is exact from the first block on.
        // A(-2) / A(-1) would be older than W(0) and are skipped; with AD = 2 step -2's A(-1)
        // is younger than W(0) and is issued as a dummy (block kb_begin again) into the
        // register slot that A(1) overwrites at step 0.
        issue_w(kb_begin, 0);
        if constexpr (AD == 3) {
            issue_a(kb_begin, afr[0]);                   // A(0), step -2
            issue_w(clampk(kb_begin + 1), 1);
            issue_a(clampk(kb_begin + 1), afr[1]);       // A(1), step -1
        } else {
            issue_a(kb_begin, afr[1]);                   // dummy A(-1), step -2
            issue_w(clampk(kb_begin + 1), 1);
            issue_a(kb_begin, afr[0]);                   // A(0), step -1
        }
        issue_w(clampk(kb_begin + 2), 2);
        int64_t kb = kb_begin;
        if constexpr (AD == 2) {
            for (; kb + 2 <= kb_end; kb += 2) {
                step(kb, std::integral_constant<int, 0>{});
                step(kb + 1, std::integral_constant<int, 1>{});
            }
            if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
        } else {
            for (; kb + 3 <= kb_end; kb += 3) {
                step(kb, std::integral_constant<int, 0>{});
                step(kb + 1, std::integral_constant<int, 1>{});
                step(kb + 2, std::integral_constant<int, 2>{});
            }
            if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
            if (kb + 1 < kb_end) step(kb + 1, std::integral_constant<int, 1>{});
        }
        wait_vmem_all();      // no LDS DMA may still be in flight when the wave ends
    }

    // Epilogue: lane owns token m and columns n..n+3 of each sub-tile.
#pragma unroll
    for (int t = 0; t < TS; ++t) {
        const int64_t m = m0 + wm * TM + t * 16 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int s = 0; s < SN; ++s) {
            const int64_t n = n0 + wn * TN + s * 16 + 4 * fgrp;
            if (n >= N) continue;
            if (split == 1) store4<OT>(p.out, m * N + n, acc[t][s]);
            else store4<O_FP32>(p.partials, ((int64_t)z * M + m) * N + n, acc[t][s]);
        }
    }
}

template <int WM, int WN, int TS, int AD, int QT, int OT, int SCHED>
hipError_t launch_ring(const GemmArgs& a, hipStream_t stream) {
    constexpr int NW = WM * WN, BM = WM * 16 * TS, BN = 256;
    constexpr int LDS_BYTES = 4 * BN * 128 + 4 * NW * 512;
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles, 1, (unsigned)a.split);
    static bool attr_set = false;   // one-time opt-in to more than 64 KB of LDS
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_ring_kernel<WM, WN, TS, AD, QT, OT, SCHED>),
            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemm_ring_kernel<WM, WN, TS, AD, QT, OT, SCHED>), grid, dim3(64 * NW),
                       LDS_BYTES, stream, a);
    return hipGetLastError();
}

// bfq_tile of a ring kernel: bm = 16*TS*WM tokens, bn = 256, WM x WN waves, stages = the
// token-fragment lead (AD - 1 blocks) + 1, i.e. 2 or 3; the W ring always has 4 slots.
#define BFQ_RING_ENTRY(WM, WN, TS, AD, SC, QT, OT)                                          \
    KernelEntry{bfq_tile{2, 16 * TS * WM, 256, 128, 1, WM, WN, AD, 8, SC, 0, 0}, QT, OT,     \
                &launch_ring<WM, WN, TS, AD, QT, OT, SC>}

#define BFQ_RING_ALL_OUT(WM, WN, TS, AD, SC, QT)                                            \
    BFQ_RING_ENTRY(WM, WN, TS, AD, SC, QT, O_BF16),                                         \
        BFQ_RING_ENTRY(WM, WN, TS, AD, SC, QT, O_FP16),                                     \
        BFQ_RING_ENTRY(WM, WN, TS, AD, SC, QT, O_FP32)

static const KernelEntry kRingKernels[] = {
    BFQ_RING_ALL_OUT(4, 2, 4, 2, 0, Q_FP8),     // 256 x 256, 64 x 128 per wave
    BFQ_RING_ALL_OUT(8, 1, 2, 3, 1, Q_FP8),     // 256 x 256, 32 x 256 per wave
    BFQ_RING_ALL_OUT(2, 2, 4, 2, 0, Q_FP8),     // 128 x 256, 64 x 128 per wave
    BFQ_RING_ALL_OUT(4, 2, 4, 2, 0, Q_INT8),
};

const KernelEntry* ring_kernels(int* count) {
    *count = (int)(sizeof(kRingKernels) / sizeof(kRingKernels[0]));
    return kRingKernels;
}

}  // namespace bfq
