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
// 16 rows. With packed weights (W_PACKED16) the same two fragment halves are 1 KB of
// contiguous memory each, which is what lets the weight stream approach the HBM peak.
// A workgroup holds NWAVES strips of NWR rows, and KW waves per strip share its K range:
// wave wk streams the wk-th contiguous slice of the strip's K blocks, and the KW partial
// tiles are summed through LDS in ascending wk (deterministic) before one wave stores the
// strip. That gives a weight matrix of few strips (N / 16 = 1536 at N = 24576) enough waves
// to keep HBM busy without a second kernel. Split-K across workgroups writes fp32 partials
// that a second kernel sums in a fixed order.
// CH = 1 (per-token x per-channel scales, [HELION] scope section): no scale loads in the K
// loop; the MFMA accumulates the wave's K range (int8: exact int32 in the accumulator's
// bits) and each wave scales its partial tile by token and channel scale before the
// in-workgroup sum. CH = 2: block scales with the activation scales as packed UE8M0 words
// (four K blocks per word); a compile-time mode, so the other modes keep their registers.
#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

// Scale a wave's partial tile by its tokens' and channels' scales (CH = 1): lane holds token
// m0 + 16*sm + frow and channels n0 + 16*sn + 4*fgrp .. +3; tokens past M take scale 0.
template <int QT, int SM, int SN>
__device__ __forceinline__ void channel_scale(v4f (&acc)[SM][SN], const GemmArgs& p, int64_t m0,
                                              int64_t n0, int frow, int fgrp) {
    float swv[SN][4];
#pragma unroll
    for (int sn = 0; sn < SN; ++sn)
#pragma unroll
        for (int j = 0; j < 4; ++j) swv[sn][j] = p.sw[n0 + sn * 16 + 4 * fgrp + j];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        const int64_t m = m0 + sm * 16 + frow;
        const float sav = m < p.M ? p.sa[m * p.sa_stride_m] : 0.f;
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            v4f a = acc[sm][sn];
            if constexpr (QT == Q_INT8) {
                const v4i pi = __builtin_bit_cast(v4i, a);
                a = v4f{(float)pi.x, (float)pi.y, (float)pi.z, (float)pi.w};
            }
            a.x = (a.x * sav) * swv[sn][0];
            a.y = (a.y * sav) * swv[sn][1];
            a.z = (a.z * sav) * swv[sn][2];
            a.w = (a.w * sav) * swv[sn][3];
            acc[sm][sn] = a;
        }
    }
}

// One MFMA step of the CH = 1 kernels: acc += W fragment x token fragment, no scaling.
template <int QT>
__device__ __forceinline__ void mfma_accumulate(v4f& acc, const v4i (&w)[2], const v4i& a0,
                                                const v4i& a1) {
    if constexpr (QT == Q_FP8) {
        const v8i wf = v8i{w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
        const v8i af = v8i{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        acc = mfma_fp8_16x16x128_acc(wf, af, acc);
    } else {
        v4i pi = __builtin_bit_cast(v4i, acc);
        pi = mfma_i8_16x16x64(w[0], a0, pi);
        pi = mfma_i8_16x16x64(w[1], a1, pi);
        acc = __builtin_bit_cast(v4f, pi);
    }
}

// MOE = 1 (grouped GEMM): blockIdx.y is a per-expert row tile (moe_tile); token rows and
// their scales are gathered through moe_rows, the weights are the expert's, and each output
// row is scattered to its pair's row.
template <int MT, int NWR, int NWAVES, int KW, int D, int QT, int OT, int WL, int CH, int MOE = 0>
__global__ __launch_bounds__(64 * NWAVES * KW) void gemm_swapab_kernel(GemmArgs p) {
    constexpr int SM = MT / 16, SN = NWR / 16;
    static_assert(!MOE || CH != 1, "grouped tiles take block scales");
    static_assert(MT % 16 == 0 && NWR % 16 == 0, "tiles are multiples of 16");
    static_assert(128 % NWR == 0, "a wave's rows must lie in one 128-row scale block");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wn = wave % NWAVES, wk = wave / NWAVES;   // strip, K slice
    const int frow = lane & 15, fgrp = lane >> 4;

    const int64_t M = p.M, N = p.N, K = p.K, KB = K / 128;
    const int64_t n0 = ((int64_t)blockIdx.x * NWAVES + wn) * NWR;
    MoeSpan sp{0, 0, 0};
    if constexpr (MOE) {
        if (!moe_tile(p.moe_offsets, p.moe_experts, M, MT, blockIdx.y, sp)) return;   // uniform
    }
    const int64_t m0 = MOE ? sp.p0 : (int64_t)blockIdx.y * MT;
    const int split = p.split, z = blockIdx.z;
    const int64_t ks0 = (int64_t)z * KB / split, ks1 = (int64_t)(z + 1) * KB / split;
    const int64_t kb_begin = ks0 + (ks1 - ks0) * wk / KW, kb_end = ks0 + (ks1 - ks0) * (wk + 1) / KW;
    const bool wave_live = n0 < N;   // whole-wave predicate (N is a multiple of 16)

    // Loads go through buffer resources: a scalar base per stream, a 32-bit per-lane offset
    // fixed for the whole K loop and the K block in the scalar offset. Rows past M read as
    // zero (past the resource), and a refill past this wave's slice uses an offset past every
    // resource, so it returns zero without touching memory.
    constexpr uint32_t KSTEP = WL == W_ROW ? 128u : 2048u;   // bytes between K blocks
    constexpr uint32_t HOFF = WL == W_ROW ? 64u : 1024u;     // second half of a fragment
    constexpr uint32_t kNoLoad = 0x80000000u;                 // past every resource here
    const int64_t nb0 = wave_live ? n0 : 0;
    const uint8_t* w_e = static_cast<const uint8_t*>(p.w) + (MOE ? sp.e * N * K : 0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_e + nb0 * K, (uint32_t)(NWR * K));
    uint32_t w_voff[SN], w_sn[SN];
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
        if constexpr (WL == W_ROW) {
            w_voff[sn] = (uint32_t)((sn * 16 + frow) * K + fgrp * 16);
            w_sn[sn] = 0;
        } else {
            w_voff[sn] = (uint32_t)(lane * 16);
            w_sn[sn] = (uint32_t)(sn * KB * 2048);
        }
    }
    const int64_t rows_a = MOE ? sp.p1 - sp.p0 : (M - m0) < MT ? (M - m0) : MT;
    const int64_t ssm = p.sa_stride_m, ssk = p.sa_stride_k;
    constexpr bool CHAN = CH == 1, PK = CH == 2;   // PK: block kb in word row kb / 4
    const int64_t sa_krows = PK ? (KB - 1) / 4 : KB - 1;
    // grouped: resources over every token; a tile row's offsets are those of its token
    const __amdgpu_buffer_rsrc_t ra =
        MOE ? make_rsrc(p.a, (uint32_t)(p.moe_tokens * K))
            : make_rsrc(static_cast<const uint8_t*>(p.a) + m0 * K, (uint32_t)(rows_a * K));
    const __amdgpu_buffer_rsrc_t rsa =
        MOE ? make_rsrc(p.sa, (uint32_t)(((p.moe_tokens - 1) * ssm + sa_krows * ssk + 1) * 4))
            : make_rsrc(p.sa + m0 * ssm, (uint32_t)(((rows_a - 1) * ssm + sa_krows * ssk + 1) * 4));
    uint32_t a_voff[SM], sa_voff[SM];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        const int r = sm * 16 + frow;
        if constexpr (MOE) {
            const int64_t t = r < rows_a ? (int64_t)p.moe_rows[sp.p0 + r] / p.moe_topk : -1;
            a_voff[sm] = t >= 0 ? (uint32_t)(t * K + fgrp * 16) : kNoLoad;
            sa_voff[sm] = t >= 0 ? (uint32_t)(t * ssm * 4) : kNoLoad;
        } else {
            a_voff[sm] = (uint32_t)(r * K + fgrp * 16);
            sa_voff[sm] = (uint32_t)(r * ssm * 4);
        }
    }
    const float* sw_row = p.sw + (MOE ? sp.e * (N / 128) * KB : 0) + (nb0 / 128) * KB;
    const int64_t L = kb_end - kb_begin;
    const int64_t kb_hi = L > 0 ? kb_end - 1 : kb_begin < KB ? kb_begin : KB - 1;

    v4i wbuf[D][SN][2];
    v4i abuf[D][SM][2];
    float sab[D][SM];
    float swb[D];
    int kbs[D];         // PK: K block % 4 of each ring slot (the byte of its scale word)

    // the loads of step i (K block kb_begin + i) into ring slot `slot`
    auto fetch = [&](int slot, int64_t i) {
        const bool live = i < L;
        const int64_t kb = live ? kb_begin + i : kb_hi;
        const uint32_t ws = live ? (uint32_t)kb * KSTEP : kNoLoad;
        const uint32_t as = live ? (uint32_t)kb * 128u : kNoLoad;
        const uint32_t ss = live ? (uint32_t)((PK ? kb >> 2 : kb) * ssk * 4) : kNoLoad;
        if constexpr (!CHAN) {
            swb[slot] = sw_row[kb];
            if constexpr (PK) kbs[slot] = (int)(kb & 3);
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) sab[slot][sm] = buf_f32(rsa, sa_voff[sm], ss);
        }
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            // streamed once: non-temporal, so the weight stream does not evict the tokens
            wbuf[slot][sn][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff[sn], w_sn[sn] + ws, kCachePolicyNT);
            wbuf[slot][sn][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff[sn], w_sn[sn] + ws + HOFF, kCachePolicyNT);
        }
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            abuf[slot][sm][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff[sm], as, 0);
            abuf[slot][sm][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff[sm], as + 64u, 0);
        }
    };

    v4f acc[SM][SN];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) acc[sm][sn] = v4f{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](int i) {
        if constexpr (CHAN) {
#pragma unroll
            for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                for (int sn = 0; sn < SN; ++sn)
                    mfma_accumulate<QT>(acc[sm][sn], wbuf[i][sn], abuf[i][sm][0], abuf[i][sm][1]);
            return;
        }
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            const float c = (PK ? e8m0_value(e8m0_byte(__float_as_uint(sab[i][sm]), kbs[i]))
                                : sab[i][sm]) * swb[i];
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

    if (wave_live && L > 0) {
        // Ring of D K blocks in flight. The steady-state loop is branch-free: a refill past the
        // end of the slice re-reads its last block (never used). (Measured: a single loop with
        // predicated steps instead is ~5 % slower on the short slices of an in-workgroup split.)
#pragma unroll
        for (int i = 0; i < D; ++i) fetch(i, i < L ? i : L - 1);
        int64_t i0 = 0;
        for (; i0 + D <= L; i0 += D) {
#pragma unroll
            for (int r = 0; r < D; ++r) {
                // keep each slot's work in its own stage: the scheduler must not hoist the
                // scale products of later slots (that would wait for every load in flight)
                __builtin_amdgcn_sched_barrier(0);
                consume(r);
                const int64_t ni = i0 + r + D;
                fetch(r, ni < L ? ni : L - 1);
            }
        }
        const int rem = (int)(L - i0);
#pragma unroll
        for (int r = 0; r < D; ++r)
            if (r < rem) consume(r);
    }
    if constexpr (CHAN) {
        if (wave_live) channel_scale<QT, SM, SN>(acc, p, m0, n0, frow, fgrp);
    }

    if constexpr (KW > 1) {
        // strip partials of K slices 1..KW-1 go through LDS; slice 0's wave adds them in order
        __shared__ v4f red[KW - 1][NWAVES][SM * SN][64];
        if (wk > 0) {
#pragma unroll
            for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) red[wk - 1][wn][sm * SN + sn][lane] = acc[sm][sn];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j)
#pragma unroll
                for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                    for (int sn = 0; sn < SN; ++sn) acc[sm][sn] += red[j][wn][sm * SN + sn][lane];
        }
    }

    if (wk == 0 && wave_live) {
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            const int64_t r = sm * 16 + frow;   // tile row; grouped: pair row moe_rows[p0 + r]
            if (MOE ? r >= rows_a : m0 + r >= M) continue;
            const int64_t m = MOE ? (int64_t)p.moe_rows[sp.p0 + r] : m0 + r;
            if (MOE && (m < 0 || m >= M)) continue;   // a pair id outside the output
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const int64_t n = n0 + sn * 16 + 4 * fgrp;
                if (split == 1) store4<OT>(p.out, m * N + n, acc[sm][sn]);
                else store4<O_FP32>(p.partials, ((int64_t)z * M + m) * N + n, acc[sm][sn]);
            }
        }
    }
}

// Swap-AB with the token fragments shared through LDS (sched 1). The waves of a workgroup
// that work on the same K slice (the NWAVES strips of one wk group) need the same token
// fragments, so instead of every wave fetching them from L2 (MT/NWR times the bytes of its
// weight stream), each K block's MT x 128 token bytes are fetched once per wk group: the MT/8
// loads of 8 whole token rows (1 KB) are dealt over the group's waves, and the token scales go to the
// group's last wave. Those loads travel in the same D-deep register ring as the weights (so
// the in-order completion of vector loads never shortens the weight prefetch distance); at
// step i they are written to LDS buffer i & 1, one barrier later every wave reads them back
// in lane order (conflict-free) for its MFMAs. Buffer i & 1 was last read at step i - 2, before
// the previous step's barrier. Every wave runs the same number of steps (the longest K slice
// of the workgroup) so the barriers match; a wave with a shorter slice idles on its last one.
template <int MT, int NWR, int NWAVES, int KW, int D, int QT, int OT, int WL, int CH, int MOE = 0>
__global__ __launch_bounds__(64 * NWAVES * KW) void gemm_swapab_lds_kernel(GemmArgs p) {
    static_assert(!MOE || CH != 1, "grouped tiles take block scales");
    constexpr int SM = MT / 16, SN = NWR / 16;
    constexpr int AI = 2 * SM;                              // 1 KB token loads per K block
    constexpr int API = (AI + NWAVES - 1) / NWAVES;         // at most this many per wave
    constexpr int SLOT = MT * 128 + MT * 4;                 // token codes + token scales
    constexpr int SCW = (MT + 63) / 64;                     // token scales per lane of the scale wave
    static_assert(MT % 16 == 0 && NWR % 16 == 0 && MT <= 128, "tiles are multiples of 16, MT <= 128");
    static_assert(128 % NWR == 0, "a wave's rows must lie in one 128-row scale block");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % NWAVES, wk = wave / NWAVES;
    const int frow = lane & 15, fgrp = lane >> 4;

    const int64_t M = p.M, N = p.N, K = p.K, KB = K / 128;
    const int64_t n0 = ((int64_t)blockIdx.x * NWAVES + wn) * NWR;
    MoeSpan sp{0, 0, 0};
    if constexpr (MOE) {
        if (!moe_tile(p.moe_offsets, p.moe_experts, M, MT, blockIdx.y, sp)) return;   // uniform
    }
    const int64_t m0 = MOE ? sp.p0 : (int64_t)blockIdx.y * MT;
    const int split = p.split, z = blockIdx.z;
    const int64_t ks0 = (int64_t)z * KB / split, ks1 = (int64_t)(z + 1) * KB / split;
    const int64_t len = ks1 - ks0;                          // >= 1 (split <= K/128)
    const int64_t kb_begin = ks0 + len * wk / KW, kb_end = ks0 + len * (wk + 1) / KW;
    const int64_t L = kb_end - kb_begin, Lmax = (len + KW - 1) / KW;
    const int64_t kb_hi = L > 0 ? kb_end - 1 : ks0;        // weight-scale index past the slice
    const bool wave_live = n0 < N;

    // Loads go through buffer resources: one scalar base per stream, a 32-bit per-lane offset
    // that is the same for every K block, and the K block in the scalar offset, so the ring
    // costs only its data registers. Rows past M (N) lie past the resource and read as zero.
    constexpr uint32_t KSTEP = WL == W_ROW ? 128u : 2048u;   // bytes between K blocks
    constexpr uint32_t HOFF = WL == W_ROW ? 64u : 1024u;     // second half of a fragment
    const int64_t nb0 = wave_live ? n0 : 0;
    const uint8_t* w_e = static_cast<const uint8_t*>(p.w) + (MOE ? sp.e * N * K : 0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_e + nb0 * K, (uint32_t)(NWR * K));
    // weight sub-tile sn: per-lane offset and the scalar offset of K block 0
    uint32_t w_voff[SN];
    uint32_t w_sn[SN];
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
        if constexpr (WL == W_ROW) {
            w_voff[sn] = (uint32_t)((sn * 16 + frow) * K + fgrp * 16);
            w_sn[sn] = 0;
        } else {
            w_voff[sn] = (uint32_t)(lane * 16);
            w_sn[sn] = (uint32_t)(sn * KB * 2048);
        }
    }
    const int64_t rows_a = MOE ? sp.p1 - sp.p0 : (M - m0) < MT ? (M - m0) : MT;
    const __amdgpu_buffer_rsrc_t ra =
        MOE ? make_rsrc(p.a, (uint32_t)(p.moe_tokens * K))
            : make_rsrc(static_cast<const uint8_t*>(p.a) + m0 * K, (uint32_t)(rows_a * K));
    // Every wave issues the same loads every step, so the compiler's count of loads in flight
    // is exact and each wait lets the whole ring stay outstanding; loads a wave does not need
    // use an offset past the resource (they return zero without a memory access).
    constexpr uint32_t kNoLoad = 0x80000000u;   // past every resource here (all < 2^31 bytes)
    // grouped: the token of tile row r (-1 past the expert's rows)
    auto src_row = [&](int64_t r) -> int64_t {
        return r < rows_a ? (int64_t)p.moe_rows[sp.p0 + r] / p.moe_topk : -1;
    };
    // Token rows this wave fetches: load t covers the 8 rows 8q .. 8q+7 of a K block
    // (q = wn + NWAVES * t), each as one whole 128-byte line: lane l reads row 8q + (l & 7),
    // bytes 16c .. 16c+15 with c = l >> 3. (Loading fragment halves directly would request
    // every line twice, 64 bytes each time.) In LDS those bytes belong to fragment half
    // j = 2*(r/16) + c/4 at the slot of the lane that feeds row r % 16 with K chunk c % 4,
    // so the readers below take lane-ordered fragment halves; the 8 lanes of one chunk write
    // 128 contiguous bytes (no bank conflicts).
    uint32_t a_voff[API], a_lds[API];
#pragma unroll
    for (int t = 0; t < API; ++t) {
        const int q = wn + NWAVES * t;
        const int c = lane >> 3;
        const int64_t r = q * 8 + (lane & 7);
        a_lds[t] = (uint32_t)((2 * (r >> 4) + (c >> 2)) * 1024 + ((c & 3) * 16 + (r & 15)) * 16);
        if constexpr (MOE) {
            const int64_t tok = q < AI ? src_row(r) : -1;
            a_voff[t] = tok >= 0 ? (uint32_t)(tok * K + 16 * c) : kNoLoad;
        } else {
            a_voff[t] = q < AI ? (uint32_t)(r * K + 16 * c) : kNoLoad;
        }
    }
    // token scales (last wave of the group): scale slot x = r * SM + s holds token s * 16 + r,
    // so each lane later reads its SM scales as one contiguous run; lane l fills slots l + 64q
    const bool scale_wave = wn == NWAVES - 1;
    const int64_t ssm = p.sa_stride_m, ssk = p.sa_stride_k;
    constexpr bool CHAN = CH == 1, PK = CH == 2;   // PK: block kb in word row kb / 4
    const int64_t sa_krows = PK ? (KB - 1) / 4 : KB - 1;
    const __amdgpu_buffer_rsrc_t rsa =
        MOE ? make_rsrc(p.sa, (uint32_t)(((p.moe_tokens - 1) * ssm + sa_krows * ssk + 1) * 4))
            : make_rsrc(p.sa + m0 * ssm, (uint32_t)(((rows_a - 1) * ssm + sa_krows * ssk + 1) * 4));
    uint32_t sa_voff[SCW];
#pragma unroll
    for (int q = 0; q < SCW; ++q) {
        const int x = lane + 64 * q;
        const int64_t r = (x % SM) * 16 + x / SM;
        if constexpr (MOE) {
            const int64_t tok = scale_wave && x < MT ? src_row(r) : -1;
            sa_voff[q] = tok >= 0 ? (uint32_t)(tok * ssm * 4) : kNoLoad;
        } else {
            sa_voff[q] = scale_wave ? (uint32_t)(r * ssm * 4) : kNoLoad;
        }
    }
    const float* sw_row = p.sw + (MOE ? sp.e * (N / 128) * KB : 0) + (nb0 / 128) * KB;

    __shared__ __attribute__((aligned(16))) uint8_t tok[KW][2][SLOT];

    v4i wbuf[D][SN][2];
    v4i abuf[D][API];
    float sab[D][SCW];
    float swb[D];

    // the loads of step i (K block kb_begin + i) into ring slot `slot`; a step past this
    // wave's slice loads nothing (offsets past the resources)
    auto fetch = [&](int slot, int64_t i) {
        const bool live = i < L;
        const int64_t kb = live ? kb_begin + i : kb_hi;
        const uint32_t ws = live ? (uint32_t)kb * KSTEP : kNoLoad;
        const uint32_t as = live ? (uint32_t)kb * 128u : kNoLoad;
        const uint32_t ss = live ? (uint32_t)((PK ? kb >> 2 : kb) * ssk * 4) : kNoLoad;
        if constexpr (!CHAN) {
            swb[slot] = sw_row[kb];
#pragma unroll
            for (int q = 0; q < SCW; ++q) sab[slot][q] = buf_f32(rsa, sa_voff[q], ss);
        }
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            // streamed once: non-temporal, so the weight stream does not evict the tokens
            wbuf[slot][sn][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff[sn], w_sn[sn] + ws, kCachePolicyNT);
            wbuf[slot][sn][1] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff[sn], w_sn[sn] + ws + HOFF, kCachePolicyNT);
        }
#pragma unroll
        for (int t = 0; t < API; ++t)
            abuf[slot][t] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff[t], as, 0);
    };

    v4f acc[SM][SN];
#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) acc[sm][sn] = v4f{0.f, 0.f, 0.f, 0.f};

    // step i: publish ring slot r's token data in buffer i & 1, barrier, then (if this wave's
    // slice has a block i) the MFMAs and scale FMAs of block kb_begin + i
    auto step = [&](int r, int64_t i) {
        uint8_t* buf = tok[wk][i & 1];
#pragma unroll
        for (int t = 0; t < API; ++t)
            if (wn + NWAVES * t < AI) *reinterpret_cast<v4i*>(buf + a_lds[t]) = abuf[r][t];
        if (!CHAN && scale_wave) {
            // packed words are decoded here, once per token, so every wave reads fp32 scales
#pragma unroll
            for (int q = 0; q < SCW; ++q)
                if (lane + 64 * q < MT)
                    *reinterpret_cast<float*>(buf + MT * 128 + (lane + 64 * q) * 4) =
                        PK ? e8m0_value(e8m0_byte(__float_as_uint(sab[r][q]), (int)((kb_begin + i) & 3)))
                           : sab[r][q];
        }
        __syncthreads();
        if (CHAN && i < L && wave_live) {
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const v4i a0 = *reinterpret_cast<const v4i*>(buf + (2 * sm) * 1024 + lane * 16);
                const v4i a1 = *reinterpret_cast<const v4i*>(buf + (2 * sm + 1) * 1024 + lane * 16);
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) mfma_accumulate<QT>(acc[sm][sn], wbuf[r][sn], a0, a1);
            }
        } else if (!CHAN && i < L && wave_live) {
            float c[SM];
            const float* sp = reinterpret_cast<const float*>(buf + MT * 128) + frow * SM;
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) c[sm] = sp[sm] * swb[r];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const v4i a0 = *reinterpret_cast<const v4i*>(buf + (2 * sm) * 1024 + lane * 16);
                const v4i a1 = *reinterpret_cast<const v4i*>(buf + (2 * sm + 1) * 1024 + lane * 16);
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) {
                    v4f pb;
                    if constexpr (QT == Q_FP8) {
                        const v4i* w2 = wbuf[r][sn];
                        const v8i wf = v8i{w2[0].x, w2[0].y, w2[0].z, w2[0].w,
                                           w2[1].x, w2[1].y, w2[1].z, w2[1].w};
                        const v8i af = v8i{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                        pb = mfma_fp8_16x16x128(wf, af);
                    } else {
                        v4i pi = mfma_i8_16x16x64(wbuf[r][sn][0], a0, v4i{0, 0, 0, 0});
                        pi = mfma_i8_16x16x64(wbuf[r][sn][1], a1, pi);
                        pb = v4f{(float)pi.x, (float)pi.y, (float)pi.z, (float)pi.w};
                    }
                    acc[sm][sn].x = __builtin_fmaf(pb.x, c[sm], acc[sm][sn].x);
                    acc[sm][sn].y = __builtin_fmaf(pb.y, c[sm], acc[sm][sn].y);
                    acc[sm][sn].z = __builtin_fmaf(pb.z, c[sm], acc[sm][sn].z);
                    acc[sm][sn].w = __builtin_fmaf(pb.w, c[sm], acc[sm][sn].w);
                }
            }
        }
    };

    // the ring: steps 0 .. D-1 in flight before the loop; step i refills its slot for i + D.
    // One loop for every step (Lmax >= 1): the prologue's loads flow into it on its only
    // entry path, so no register copies wait for them.
#pragma unroll
    for (int i = 0; i < D; ++i) fetch(i, i);
    int64_t i0 = 0;
    do {
#pragma unroll
        for (int r = 0; r < D; ++r) {
            __builtin_amdgcn_sched_barrier(0);
            if (i0 + r < Lmax) step(r, i0 + r);      // uniform over the workgroup
            fetch(r, i0 + r + D);
        }
        i0 += D;
    } while (i0 < Lmax);
    if constexpr (CHAN) {
        if (wave_live) channel_scale<QT, SM, SN>(acc, p, m0, n0, frow, fgrp);
    }

    if constexpr (KW > 1) {
        __shared__ v4f red[KW - 1][NWAVES][SM * SN][64];
        if (wk > 0) {
#pragma unroll
            for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) red[wk - 1][wn][sm * SN + sn][lane] = acc[sm][sn];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int j = 0; j < KW - 1; ++j)
#pragma unroll
                for (int sm = 0; sm < SM; ++sm)
#pragma unroll
                    for (int sn = 0; sn < SN; ++sn) acc[sm][sn] += red[j][wn][sm * SN + sn][lane];
        }
    }

    if (wk == 0 && wave_live) {
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            const int64_t r = sm * 16 + frow;   // tile row; grouped: pair row moe_rows[p0 + r]
            if (MOE ? r >= rows_a : m0 + r >= M) continue;
            const int64_t m = MOE ? (int64_t)p.moe_rows[sp.p0 + r] : m0 + r;
            if (MOE && (m < 0 || m >= M)) continue;   // a pair id outside the output
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const int64_t n = n0 + sn * 16 + 4 * fgrp;
                if (split == 1) store4<OT>(p.out, m * N + n, acc[sm][sn]);
                else store4<O_FP32>(p.partials, ((int64_t)z * M + m) * N + n, acc[sm][sn]);
            }
        }
    }
}

template <int MT, int NWR, int NWAVES, int KW, int D, int QT, int OT, int WL, int CH>
hipError_t launch_swapab(const GemmArgs& a, hipStream_t stream) {
    const int64_t strips = (a.N + NWR * NWAVES - 1) / (NWR * NWAVES);
    dim3 grid((unsigned)strips, (unsigned)((a.M + MT - 1) / MT), (unsigned)a.split);
    hipLaunchKernelGGL((gemm_swapab_kernel<MT, NWR, NWAVES, KW, D, QT, OT, WL, CH>), grid,
                       dim3(64 * NWAVES * KW), 0, stream, a);
    return hipGetLastError();
}

template <int MT, int NWR, int NWAVES, int KW, int D, int QT, int OT, int WL, int CH>
hipError_t launch_swapab_lds(const GemmArgs& a, hipStream_t stream) {
    const int64_t strips = (a.N + NWR * NWAVES - 1) / (NWR * NWAVES);
    dim3 grid((unsigned)strips, (unsigned)((a.M + MT - 1) / MT), (unsigned)a.split);
    hipLaunchKernelGGL((gemm_swapab_lds_kernel<MT, NWR, NWAVES, KW, D, QT, OT, WL, CH>), grid,
                       dim3(64 * NWAVES * KW), 0, stream, a);
    return hipGetLastError();
}

// grouped (MoE) forms: grid height = the per-expert row tiles' upper bound
template <int MT, int NWR, int NWAVES, int KW, int D, int QT, int OT, int WL, int CH>
hipError_t launch_moe_swapab(const GemmArgs& a, hipStream_t stream) {
    const int64_t strips = (a.N + NWR * NWAVES - 1) / (NWR * NWAVES);
    dim3 grid((unsigned)strips, (unsigned)moe_max_tiles(a.M, a.moe_experts, MT), (unsigned)a.split);
    hipLaunchKernelGGL((gemm_swapab_kernel<MT, NWR, NWAVES, KW, D, QT, OT, WL, CH, 1>), grid,
                       dim3(64 * NWAVES * KW), 0, stream, a);
    return hipGetLastError();
}

template <int MT, int NWR, int NWAVES, int KW, int D, int QT, int OT, int WL, int CH>
hipError_t launch_moe_swapab_lds(const GemmArgs& a, hipStream_t stream) {
    const int64_t strips = (a.N + NWR * NWAVES - 1) / (NWR * NWAVES);
    dim3 grid((unsigned)strips, (unsigned)moe_max_tiles(a.M, a.moe_experts, MT), (unsigned)a.split);
    hipLaunchKernelGGL((gemm_swapab_lds_kernel<MT, NWR, NWAVES, KW, D, QT, OT, WL, CH, 1>), grid,
                       dim3(64 * NWAVES * KW), 0, stream, a);
    return hipGetLastError();
}

// bfq_tile for variant 1: bm = MT tokens, bn = NWR * NW rows per workgroup, waves_m = KW
// waves sharing each strip's K range, waves_n = NW strips, stages = D K blocks in flight,
// sched 0 = tokens per wave from L2, sched 1 = tokens shared through LDS.
#define BFQ_SAB_ENTRY(MT, NWR, NW, KW, D, QT, OT, WL, CH)                                  \
    KernelEntry{bfq_tile{1, MT, NWR * NW, 128, 1, KW, NW, D, 1, 0, 0, 0}, QT, OT, WL,         \
                (CH) == 1 ? S_CHANNEL : (CH) == 2 ? S_PACKED : S_FP32,                   \
                &launch_swapab<MT, NWR, NW, KW, D, QT, OT, WL, CH>}
#define BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, WL, CH)                                    \
    BFQ_SAB_ENTRY(MT, NWR, NW, KW, D, QT, O_BF16, WL, CH),                                 \
        BFQ_SAB_ENTRY(MT, NWR, NW, KW, D, QT, O_FP16, WL, CH),                             \
        BFQ_SAB_ENTRY(MT, NWR, NW, KW, D, QT, O_FP32, WL, CH)
#define BFQ_SAB_BOTH(MT, NWR, NW, KW, D, QT)                                                \
    BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, W_ROW, 0), BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, W_PACKED16, 0)
// per-token x per-channel scales
#define BFQ_SAB_CH(MT, NWR, NW, KW, D, QT)                                                  \
    BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, W_ROW, 1), BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, W_PACKED16, 1)
// block scales, activation scales as packed UE8M0 words
#define BFQ_SAB_PK(MT, NWR, NW, KW, D, QT)                                                  \
    BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, W_ROW, 2), BFQ_SAB_ALL_OUT(MT, NWR, NW, KW, D, QT, W_PACKED16, 2)

#define BFQ_SABL_ENTRY(MT, NWR, NW, KW, D, QT, OT, WL, CH)                                 \
    KernelEntry{bfq_tile{1, MT, NWR * NW, 128, 1, KW, NW, D, 1, 1, 0, 0}, QT, OT, WL,         \
                (CH) == 1 ? S_CHANNEL : (CH) == 2 ? S_PACKED : S_FP32,                   \
                &launch_swapab_lds<MT, NWR, NW, KW, D, QT, OT, WL, CH>}
#define BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, WL, CH)                                   \
    BFQ_SABL_ENTRY(MT, NWR, NW, KW, D, QT, O_BF16, WL, CH),                                \
        BFQ_SABL_ENTRY(MT, NWR, NW, KW, D, QT, O_FP16, WL, CH),                            \
        BFQ_SABL_ENTRY(MT, NWR, NW, KW, D, QT, O_FP32, WL, CH)
#define BFQ_SABL_BOTH(MT, NWR, NW, KW, D, QT)                                               \
    BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, W_ROW, 0), BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, W_PACKED16, 0)
#define BFQ_SABL_CH(MT, NWR, NW, KW, D, QT)                                                 \
    BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, W_ROW, 1), BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, W_PACKED16, 1)
#define BFQ_SABL_PK(MT, NWR, NW, KW, D, QT)                                                 \
    BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, W_ROW, 2), BFQ_SABL_ALL_OUT(MT, NWR, NW, KW, D, QT, W_PACKED16, 2)

static const KernelEntry kSwapabKernels[] = {
    BFQ_SABL_BOTH(16, 16, 8, 1, 8, Q_FP8),
    BFQ_SABL_BOTH(16, 16, 4, 2, 8, Q_FP8),
    BFQ_SABL_BOTH(32, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(32, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(32, 16, 4, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(48, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(48, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(64, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(64, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(64, 16, 4, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(64, 32, 4, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(96, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(96, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(128, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(128, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(32, 16, 6, 1, 8, Q_FP8),
    BFQ_SABL_BOTH(32, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(64, 16, 6, 1, 8, Q_FP8),
    BFQ_SABL_BOTH(64, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(96, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(128, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(96, 32, 4, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(128, 32, 4, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(128, 32, 6, 1, 4, Q_FP8),
    BFQ_SABL_BOTH(64, 32, 6, 2, 4, Q_FP8),
    BFQ_SABL_BOTH(16, 16, 8, 1, 8, Q_INT8),
    BFQ_SABL_BOTH(32, 16, 8, 1, 4, Q_INT8),
    BFQ_SABL_BOTH(64, 16, 8, 1, 4, Q_INT8),
    BFQ_SABL_BOTH(128, 16, 8, 1, 4, Q_INT8),
    BFQ_SAB_BOTH(16, 32, 4, 1, 4, Q_FP8),
    BFQ_SAB_BOTH(16, 16, 4, 1, 8, Q_FP8),
    BFQ_SAB_BOTH(16, 16, 8, 1, 8, Q_FP8),
    BFQ_SAB_BOTH(16, 32, 8, 1, 4, Q_FP8),
    BFQ_SAB_BOTH(16, 64, 4, 1, 2, Q_FP8),
    BFQ_SAB_BOTH(16, 32, 4, 1, 8, Q_FP8),
    BFQ_SAB_BOTH(32, 32, 4, 1, 4, Q_FP8),
    BFQ_SAB_BOTH(64, 32, 4, 1, 2, Q_FP8),
    BFQ_SAB_BOTH(16, 16, 1, 4, 4, Q_FP8),
    BFQ_SAB_BOTH(16, 16, 1, 4, 8, Q_FP8),
    BFQ_SAB_BOTH(16, 16, 2, 2, 8, Q_FP8),
    BFQ_SAB_BOTH(16, 16, 1, 8, 4, Q_FP8),
    BFQ_SAB_BOTH(16, 32, 1, 4, 4, Q_FP8),
    BFQ_SAB_BOTH(32, 16, 1, 4, 4, Q_FP8),
    BFQ_SAB_BOTH(64, 16, 1, 4, 2, Q_FP8),
    BFQ_SAB_BOTH(32, 32, 1, 4, 4, Q_FP8),
    BFQ_SAB_BOTH(16, 32, 4, 1, 4, Q_INT8),
    BFQ_SAB_BOTH(32, 32, 4, 1, 4, Q_INT8),
    BFQ_SAB_BOTH(64, 32, 4, 1, 2, Q_INT8),
    BFQ_SAB_BOTH(16, 16, 1, 4, 4, Q_INT8),
    BFQ_SAB_BOTH(32, 16, 1, 4, 4, Q_INT8),
    BFQ_SAB_BOTH(64, 16, 1, 4, 2, Q_INT8),
    BFQ_SABL_CH(16, 16, 8, 1, 8, Q_FP8),
    BFQ_SABL_CH(32, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_CH(32, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_CH(32, 16, 4, 2, 4, Q_FP8),
    BFQ_SABL_CH(64, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_CH(64, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_CH(64, 16, 4, 2, 4, Q_FP8),
    BFQ_SABL_CH(96, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_CH(128, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_CH(128, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_CH(16, 16, 8, 1, 8, Q_INT8),
    BFQ_SABL_CH(32, 16, 8, 1, 4, Q_INT8),
    BFQ_SABL_CH(64, 16, 8, 1, 4, Q_INT8),
    BFQ_SABL_CH(128, 16, 8, 1, 4, Q_INT8),
    BFQ_SAB_CH(16, 32, 4, 1, 4, Q_FP8),
    BFQ_SAB_CH(16, 16, 4, 1, 8, Q_FP8),
    BFQ_SAB_CH(16, 16, 8, 1, 8, Q_FP8),
    BFQ_SAB_CH(32, 32, 4, 1, 4, Q_FP8),
    BFQ_SAB_CH(16, 16, 1, 4, 4, Q_FP8),
    BFQ_SAB_CH(16, 16, 1, 4, 8, Q_FP8),
    BFQ_SAB_CH(16, 32, 1, 4, 4, Q_FP8),
    BFQ_SAB_CH(32, 16, 1, 4, 4, Q_FP8),
    BFQ_SAB_CH(64, 16, 1, 4, 2, Q_FP8),
    BFQ_SAB_CH(16, 32, 4, 1, 4, Q_INT8),
    BFQ_SAB_CH(32, 32, 4, 1, 4, Q_INT8),
    BFQ_SAB_CH(16, 16, 1, 4, 4, Q_INT8),
    BFQ_SAB_CH(32, 16, 1, 4, 4, Q_INT8),
    // fp8 block scales read as packed UE8M0 activation-scale words
    BFQ_SABL_PK(96, 32, 4, 1, 4, Q_FP8),
    BFQ_SABL_PK(128, 32, 4, 1, 4, Q_FP8),
    BFQ_SABL_PK(128, 32, 6, 1, 4, Q_FP8),
    BFQ_SABL_PK(64, 32, 6, 2, 4, Q_FP8),
    BFQ_SABL_PK(16, 16, 8, 1, 8, Q_FP8),
    BFQ_SABL_PK(16, 16, 4, 2, 8, Q_FP8),
    BFQ_SABL_PK(32, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_PK(32, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_PK(32, 16, 4, 2, 4, Q_FP8),
    BFQ_SABL_PK(48, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_PK(48, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_PK(64, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_PK(64, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_PK(64, 16, 4, 2, 4, Q_FP8),
    BFQ_SABL_PK(64, 32, 4, 1, 4, Q_FP8),
    BFQ_SABL_PK(96, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_PK(96, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_PK(128, 16, 8, 1, 4, Q_FP8),
    BFQ_SABL_PK(128, 16, 6, 1, 4, Q_FP8),
    BFQ_SABL_PK(32, 16, 6, 1, 8, Q_FP8),
    BFQ_SABL_PK(32, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_PK(64, 16, 6, 1, 8, Q_FP8),
    BFQ_SABL_PK(64, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_PK(96, 16, 6, 2, 4, Q_FP8),
    BFQ_SABL_PK(128, 16, 6, 2, 4, Q_FP8),
    BFQ_SAB_PK(16, 32, 4, 1, 4, Q_FP8),
    BFQ_SAB_PK(16, 16, 4, 1, 8, Q_FP8),
    BFQ_SAB_PK(16, 16, 8, 1, 8, Q_FP8),
    BFQ_SAB_PK(16, 32, 8, 1, 4, Q_FP8),
    BFQ_SAB_PK(16, 64, 4, 1, 2, Q_FP8),
    BFQ_SAB_PK(16, 32, 4, 1, 8, Q_FP8),
    BFQ_SAB_PK(32, 32, 4, 1, 4, Q_FP8),
    BFQ_SAB_PK(64, 32, 4, 1, 2, Q_FP8),
    BFQ_SAB_PK(16, 16, 1, 4, 4, Q_FP8),
    BFQ_SAB_PK(16, 16, 1, 4, 8, Q_FP8),
    BFQ_SAB_PK(16, 16, 2, 2, 8, Q_FP8),
    BFQ_SAB_PK(16, 16, 1, 8, 4, Q_FP8),
    BFQ_SAB_PK(16, 32, 1, 4, 4, Q_FP8),
    BFQ_SAB_PK(32, 16, 1, 4, 4, Q_FP8),
    BFQ_SAB_PK(64, 16, 1, 4, 2, Q_FP8),
    BFQ_SAB_PK(32, 32, 1, 4, 4, Q_FP8),
};

// grouped (MoE) swap-AB kernels, fp8, fp32 or UE8M0 block scales (S_FP32 serves both) and
// packed UE8M0 words
#define BFQ_MOE_SAB_ENTRY(MT, NWR, NW, KW, D, OT, WL, CH)                                      \
    KernelEntry{bfq_tile{1, MT, NWR * NW, 128, 1, KW, NW, D, 1, 0, 0, 0}, Q_FP8, OT, WL,         \
                (CH) == 2 ? S_PACKED : S_FP32, &launch_moe_swapab<MT, NWR, NW, KW, D, Q_FP8, OT, WL, CH>, 1}
#define BFQ_MOE_SABL_ENTRY(MT, NWR, NW, KW, D, OT, WL, CH)                                     \
    KernelEntry{bfq_tile{1, MT, NWR * NW, 128, 1, KW, NW, D, 1, 1, 0, 0}, Q_FP8, OT, WL,         \
                (CH) == 2 ? S_PACKED : S_FP32,                                                 \
                &launch_moe_swapab_lds<MT, NWR, NW, KW, D, Q_FP8, OT, WL, CH>, 1}
#define BFQ_MOE_X6(ENTRY, MT, NWR, NW, KW, D, CH)                                               \
    ENTRY(MT, NWR, NW, KW, D, O_BF16, W_ROW, CH), ENTRY(MT, NWR, NW, KW, D, O_FP16, W_ROW, CH),   \
        ENTRY(MT, NWR, NW, KW, D, O_FP32, W_ROW, CH),                                          \
        ENTRY(MT, NWR, NW, KW, D, O_BF16, W_PACKED16, CH),                                     \
        ENTRY(MT, NWR, NW, KW, D, O_FP16, W_PACKED16, CH),                                     \
        ENTRY(MT, NWR, NW, KW, D, O_FP32, W_PACKED16, CH)
#define BFQ_MOE_SAB(MT, NWR, NW, KW, D)                                                        \
    BFQ_MOE_X6(BFQ_MOE_SAB_ENTRY, MT, NWR, NW, KW, D, 0), BFQ_MOE_X6(BFQ_MOE_SAB_ENTRY, MT, NWR, NW, KW, D, 2)
#define BFQ_MOE_SABL(MT, NWR, NW, KW, D)                                                       \
    BFQ_MOE_X6(BFQ_MOE_SABL_ENTRY, MT, NWR, NW, KW, D, 0), BFQ_MOE_X6(BFQ_MOE_SABL_ENTRY, MT, NWR, NW, KW, D, 2)

static const KernelEntry kMoeSwapabKernels[] = {
    BFQ_MOE_SAB(16, 32, 4, 1, 4),
    BFQ_MOE_SAB(16, 16, 4, 1, 8),
    BFQ_MOE_SAB(16, 16, 1, 4, 4),
    BFQ_MOE_SAB(32, 32, 4, 1, 4),
    BFQ_MOE_SABL(16, 16, 8, 1, 8),
    BFQ_MOE_SABL(32, 16, 8, 1, 4),
    BFQ_MOE_SABL(32, 16, 6, 1, 4),
    BFQ_MOE_SABL(32, 16, 4, 2, 4),
    BFQ_MOE_SABL(64, 16, 8, 1, 4),
    BFQ_MOE_SABL(64, 16, 6, 1, 4),
    BFQ_MOE_SABL(64, 16, 4, 2, 4),
    BFQ_MOE_SABL(96, 16, 6, 1, 4),
    BFQ_MOE_SABL(128, 16, 8, 1, 4),
    BFQ_MOE_SABL(128, 16, 6, 1, 4),
};

const KernelEntry* moe_swapab_kernels(int* count) {
    *count = (int)(sizeof(kMoeSwapabKernels) / sizeof(kMoeSwapabKernels[0]));
    return kMoeSwapabKernels;
}

const KernelEntry* swapab_kernels(int* count) {
    *count = (int)(sizeof(kSwapabKernels) / sizeof(kSwapabKernels[0]));
    return kSwapabKernels;
}

// ------------------------------------------------------------ split-K reduce ----
// out[i] = sum over z of part[z][i], added in z order (so results are run-to-run identical
// and do not depend on the split kernel's timing). The partial loads of B splits are all
// issued before any is waited on (B >= split: one memory round trip, rather than one per
// split, which is what the reduce of a small output costs); slots past the last split
// re-read the last partial, which stays in cache, and are not added.
template <int OT, int B>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            void* __restrict__ out,
                                                            int64_t MN, int split) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;                       // MN is a multiple of 128
    const float* p = part + i;
    v4f s = *reinterpret_cast<const v4f*>(p);
    for (int z0 = 1; z0 < split; z0 += B) {
        v4f t[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int z = z0 + j < split ? z0 + j : split - 1;
            t[j] = *reinterpret_cast<const v4f*>(p + (int64_t)z * MN);
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const bool live = z0 + j < split;
            const v4f u = {s.x + t[j].x, s.y + t[j].y, s.z + t[j].z, s.w + t[j].w};
            s = live ? u : s;
        }
    }
    store4<OT>(out, i, s);
}

template <int OT>
static void launch_reduce_ot(const float* partials, void* out, int64_t MN, int split,
                             hipStream_t stream) {
    dim3 grid((unsigned)((MN / 4 + 255) / 256));
    if (split <= 3)
        hipLaunchKernelGGL((splitk_reduce_kernel<OT, 2>), grid, dim3(256), 0, stream, partials, out, MN, split);
    else if (split <= 5)
        hipLaunchKernelGGL((splitk_reduce_kernel<OT, 4>), grid, dim3(256), 0, stream, partials, out, MN, split);
    else if (split <= 9)
        hipLaunchKernelGGL((splitk_reduce_kernel<OT, 8>), grid, dim3(256), 0, stream, partials, out, MN, split);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<OT, 16>), grid, dim3(256), 0, stream, partials, out, MN, split);
}

hipError_t launch_splitk_reduce(const float* partials, void* out, int64_t M, int64_t N,
                                int split, int otype, hipStream_t stream) {
    const int64_t MN = M * N;
    if (otype == O_BF16)
        launch_reduce_ot<O_BF16>(partials, out, MN, split, stream);
    else if (otype == O_FP16)
        launch_reduce_ot<O_FP16>(partials, out, MN, split, stream);
    else
        launch_reduce_ot<O_FP32>(partials, out, MN, split, stream);
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
