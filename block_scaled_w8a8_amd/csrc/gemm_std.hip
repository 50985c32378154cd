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
//    sched 2 instead uses 32x32 sub-tiles: two v_mfma_f32_32x32x64_f8f6f4 per K block
//    (each weight fragment feeds twice the MFMA work per LDS read; a lane owns one token and
//    four groups of four output columns).
//  * sched 3 (power-of-two scales only): the scales are applied inside the block-scaled MFMA
//    as E8M0 exponents — the weight scale (one per 128-row block, uniform over a wave) for
//    the first operand, each lane's token scale for the second — and the MFMA accumulates
//    across K blocks itself: no block partial, no FMA. A power-of-two fp32 scale's E8M0
//    byte is its exponent field.
//  * sched 4 (per-token x per-channel scales, [HELION] scope section): no per-block scale at
//    all; the MFMA accumulates the whole K range (fp8 in fp32; int8 in int32, exact, kept in
//    the accumulator registers' bits) and the tile routine multiplies each element by its
//    token and channel scale once at the end.
//  * The weight fragment sits in the MFMA's first operand and the token fragment in the
//    second, so each lane ends up owning one token row and four consecutive output columns:
//    one scale product per lane and sub-tile row, and 8-byte (bf16) row-contiguous stores.
//  * LDS rows are 128 bytes (one K block); the 16-byte chunk c of row r is stored at slot
//    c ^ swz(r) so the 16 rows a fragment read touches fall in different banks.
//  * Workgroup ids are remapped so that each XCD (ids i, i+8, i+16, ...) owns a contiguous
//    range of tiles, ordered in groups of group_m tile rows, keeping shared A/W panels in
//    that XCD's L2.
//  * Weights row-major (W_ROW) or packed (W_PACKED16, see bfq_weight_layout): packed W
//    arrives as whole 1 KB fragment halves, lands in LDS in lane order and is read back by
//    each lane at 16*lane (conflict-free without a swizzle). A 16x16x128 MFMA's K order is
//    free as long as both operands share it, so with packed W the token fragment takes
//    16-byte chunks (l/16) and (l/16)+4 of its row, the placement the packed weights carry
//    (the int8 path uses that placement for both layouts).
#include <type_traits>

#include "bfq_internal.h"
#include "device_common.h"

namespace bfq {

// Wave-tile geometry of one configuration.
template <int BM, int BN, int WM, int WN, int SCHED>
struct StdShape {
    static constexpr int NWAVES = WM * WN;
    static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile (tokens x weight rows)
    // sched 2: 32x32x64 MFMAs (two per K block and sub-tile), else 16x16 MFMAs
    static constexpr int MF = SCHED == 2 ? 32 : 16;    // sub-tile edge
    static constexpr int SM = TM / MF, SN = TN / MF;   // MF x MF sub-tiles per wave
    using AccT = typename std::conditional<MF == 32, v16f, v4f>::type;
    // LDS: two tile stages, the optional L2-touch scratch, two scale stages
    static constexpr int STAGE = (BM + BN) * 128;
    static constexpr int lds_bytes(int stages) {
        return 2 * STAGE + (stages > 2 ? 256 * NWAVES : 0) + 2 * (BM + 64) * 4;
    }
};

// K blocks [kb_begin, kb_end) of the output tile at (m0, n0) into acc (zeroed here). Every
// wave of the workgroup calls it with the same arguments; it leaves no LDS DMA in flight and
// ends on a barrier, so the next call may reuse the LDS at once.
// MOE = 1 (grouped GEMM): the tile's rows are grouped rows [sp.p0, sp.p1) of expert sp.e;
// each A row (and its activation scales) is gathered from token moe_rows[row] / topk, and
// the weights are expert e's.
template <int BM, int BN, int WM, int WN, int QT, int SCHED, int STAGES, int WL, int MOE = 0>
__device__ __forceinline__ void std_tile(
    const GemmArgs& p, uint8_t* lds, int64_t m0, int64_t n0, int64_t kb_begin, int64_t kb_end,
    typename StdShape<BM, BN, WM, WN, SCHED>::AccT (&acc)[StdShape<BM, BN, WM, WN, SCHED>::SM]
                                                          [StdShape<BM, BN, WM, WN, SCHED>::SN],
    const MoeSpan& sp = MoeSpan{0, 0, 0}) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    constexpr int NWAVES = Shape::NWAVES;
    constexpr int TM = Shape::TM, TN = Shape::TN;
    constexpr int MF = Shape::MF, SM = Shape::SM, SN = Shape::SN;
    using AccT = typename Shape::AccT;
    static_assert(SCHED != 2 || (QT == Q_FP8 && WL == W_ROW && TM % 32 == 0 && TN % 32 == 0),
                  "the 32x32 schedule is fp8 only, row-major W, and needs 32-multiple wave tiles");
    static_assert(SCHED != 3 || QT == Q_FP8, "the block-scaled MFMA schedule is fp8 only");
    static_assert(SCHED <= 4, "schedules 0-4");
    static_assert(!MOE || (STAGES == 2 && SCHED != 4), "grouped tiles: two stages, block scales");
    constexpr int STAGE = (BM + BN) * 128;         // bytes per LDS stage
    constexpr int CHUNKS = (BM + BN) / 8;          // 1 KB load chunks per stage
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BM % 16 == 0, "the W region must start on a 16-row boundary");
    // A wave's columns lie in one 128-wide weight-scale block, or (SPLIT_SW: 96-column wave
    // tiles of 192-wide tiles, fp8 FMA schedules) in at most two adjacent ones: the sub-tiles
    // before the wave-uniform boundary sn_split take the first block's scale, the rest the next.
    constexpr bool SPLIT_SW = 128 % TN != 0;
    static_assert(!SPLIT_SW || (TN == 96 && QT == Q_FP8 && SCHED <= 1 && !MOE),
                  "a wave's columns must lie in one 128-wide scale block (or 96 of them in two)");
    static_assert(CHUNKS % NWAVES == 0, "load chunks must divide evenly over waves");
    static_assert((BM / 8) % NWAVES == 0, "A chunks must divide evenly over waves");
    static_assert(NWAVES % 2 == 0, "the swizzle phase of a lane's chunks needs an even wave count");
    constexpr int CPW = CHUNKS / NWAVES;
    constexpr int CPW_A = BM / 8 / NWAVES;                 // chunks i < CPW_A hold A rows
    // Scale staging in LDS after the tile stages (and the L2-touch scratch): per stage BM
    // activation scales ordered [wave row][lane row][sub-tile row], then 64 weight-scale slots.
    constexpr int SC_BASE = 2 * STAGE + (STAGES > 2 ? 256 * NWAVES : 0);
    constexpr int SC_STAGE = (BM + 64) * 4;
    static_assert(BM % 64 == 0 && BM / 64 <= NWAVES, "one activation-scale DMA per wave");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & (MF - 1);   // fragment row within a sub-tile
    const int fgrp = lane >> 4;         // 16x16: 32-byte K group (fp8) / 16-byte K chunk (int8)
    const int khalf = lane >> 5;        // 32x32: 32-byte K group within a 64-wide K half

    const int64_t M = p.M, N = p.N, K = p.K, KB = K / 128;

    // Buffer resources over this tile's rows: rows past M (N) read as zero and are never
    // stored, so ragged tiles need no clamping. K <= 2^23 keeps every offset below 2^32.
    const int64_t rows_a = MOE ? sp.p1 - sp.p0 : (M - m0) < BM ? (M - m0) : BM;
    const int64_t rows_w = (N - n0) < BN ? (N - n0) : BN;
    // grouped: A over every token (rows are gathered), W and its scales those of expert e
    const __amdgpu_buffer_rsrc_t ra =
        MOE ? make_rsrc(p.a, (uint32_t)(p.moe_tokens * K))
            : make_rsrc(static_cast<const uint8_t*>(p.a) + m0 * K, (uint32_t)(rows_a * K));
    const uint8_t* w_e = static_cast<const uint8_t*>(p.w) + (MOE ? sp.e * N * K : 0);
    const float* sw_e = p.sw + (MOE ? sp.e * (N / 128) * KB : 0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_e + n0 * K, (uint32_t)(rows_w * K));
    constexpr uint32_t kNoLoad = 0x80000000u;   // past every resource: reads zero, no access
    // grouped: token row of tile row r (rows past the expert's last read nothing)
    auto src_row = [&](int64_t r) -> int64_t {
        return r < rows_a ? (int64_t)p.moe_rows[sp.p0 + r] / p.moe_topk : -1;
    };

    // Scale buffers. Activation-scale DMA slot s = wave*64 + lane holds token row
    // r(s) = wm*TM + sm*MF + frow for s = wm*TM + frow*SM + sm, so each lane later reads its
    // SM scales as one contiguous LDS vector. Rows past M and blocks past N read as zero.
    // Packed UE8M0 scales: one 32-bit word per token and 4 K blocks, so block kb reads word
    // row kb / 4 and the byte kb % 4 is picked when the scale is used.
    const int64_t ssm = p.sa_stride_m, ssk = p.sa_stride_k;
    const int packed = p.sa_packed;
    const int64_t sa_rows = packed ? (KB - 1) / 4 : KB - 1;
    const __amdgpu_buffer_rsrc_t rsa =
        MOE ? make_rsrc(p.sa, (uint32_t)(((p.moe_tokens - 1) * ssm + sa_rows * ssk + 1) * 4))
            : make_rsrc(p.sa + m0 * ssm, (uint32_t)(((rows_a - 1) * ssm + sa_rows * ssk + 1) * 4));
    uint32_t sa_dma_voff;
    {
        const int sl = wave * 64 + lane;
        const int swm = sl / TM, rem = sl % TM;
        const int r = swm * TM + (rem % SM) * MF + rem / SM;
        if constexpr (MOE) {
            const int64_t t = src_row(r);
            sa_dma_voff = t >= 0 ? (uint32_t)(t * ssm * 4) : kNoLoad;
        } else {
            sa_dma_voff = (uint32_t)(r * ssm * 4);
        }
    }
    const int64_t nb0 = n0 / 128, nbs = (rows_w + 127) / 128;
    const __amdgpu_buffer_rsrc_t rsw = make_rsrc(sw_e + nb0 * KB, (uint32_t)(nbs * KB * 4));
    const uint32_t sw_dma_voff = (uint32_t)(lane * KB * 4);
    const uint32_t sa_lds = (uint32_t)((wm * TM + frow * SM) * 4);
    // the wave's first column n0 + wn*TN is a multiple of 32 (n0 of 64), so 16-column
    // sub-tiles never straddle a scale block
    const int64_t wcol0 = n0 + (int64_t)wn * TN;
    const uint32_t sw_lds = SPLIT_SW ? (uint32_t)(BM * 4 + (wcol0 / 128 - nb0) * 4)
                                     : (uint32_t)(BM * 4 + ((wn * TN) / 128) * 4);
    const int sn_split = SPLIT_SW ? (int)((128 - wcol0 % 128) / 16) : SN;   // may exceed SN
    (void)sn_split;

    // Load chunk i of this wave covers region rows 8*(wave + NWAVES*i) .. +7; lane l writes
    // LDS slot (l & 7) of row +(l >> 3), which holds global chunk (l & 7) ^ swz(row). As
    // NWAVES is even, swz(row) = (l >> 3) ^ (wave & 1) for every i, so one per-lane byte
    // offset serves all chunks and the chunk index goes into the scalar offset.
    const uint32_t chunk_off = (uint32_t)(((lane & 7) ^ (lane >> 3) ^ (wave & 1)) << 4);
    const uint32_t dma_voff = (uint32_t)(((lane >> 3) + wave * 8) * K) + chunk_off;
    // grouped: the gathered A rows of this lane's load chunks (tile row (lane>>3) + 8*(wave +
    // NWAVES*i)), as full byte offsets; the K block goes in the scalar offset
    uint32_t a_voff[MOE ? CPW_A : 1];
    if constexpr (MOE) {
#pragma unroll
        for (int i = 0; i < CPW_A; ++i) {
            const int64_t t = src_row((lane >> 3) + 8 * (wave + NWAVES * i));
            a_voff[i] = t >= 0 ? (uint32_t)(t * K) + chunk_off : kNoLoad;
        }
    }
    // packed W: lane offset within a 1 KB half, bytes between 16-row fragments
    const uint32_t lane16 = (uint32_t)(lane * 16);
    const uint32_t frag_stride = (uint32_t)(KB * 2048);
    (void)lane16;
    (void)frag_stride;
    auto issue_stage = [&](int64_t kb, int stage) {
        const uint32_t skb = (uint32_t)(kb * 128);
        // scales of block kb: waves 0 .. BM/64-1 fetch 64 activation scales each, wave 0 also
        // the weight scales of the tile's 128-row blocks
        const uint32_t sc = (uint32_t)(SC_BASE + stage * SC_STAGE);
        if constexpr (SCHED != 4) {   // sched 4 has no per-block scales
            if (wave < BM / 64)
                dma4(rsa, lds, sc + wave * 256, sa_dma_voff,
                     (uint32_t)((packed ? kb >> 2 : kb) * ssk * 4));
            if (wave == 0) dma4(rsw, lds, sc + BM * 4, sw_dma_voff, (uint32_t)(kb * 4));
        }
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const uint32_t lds_off = (uint32_t)((wave + NWAVES * i) * 1024 + stage * STAGE);
            if (i < CPW_A) {
                if constexpr (MOE) dma16(ra, lds, lds_off, a_voff[i < CPW_A ? i : 0], skb);
                else dma16(ra, lds, lds_off, dma_voff, skb + (uint32_t)(NWAVES * i * 8 * K));
            } else if constexpr (WL == W_ROW) {
                dma16(rw, lds, lds_off, dma_voff, skb + (uint32_t)((NWAVES * i - BM / 8) * 8 * K));
            } else {
                // W chunk c of the stage is half (c & 1) of the tile's fragment c >> 1: 1 KB
                // contiguous at (fragment * KB + kb) * 2048 + half * 1024
                const uint32_t c = (uint32_t)(wave + NWAVES * i - BM / 8);
                dma16(rw, lds, lds_off, lane16,
                      (c >> 1) * frag_stride + (c & 1) * 1024u + (uint32_t)(kb * 2048));
            }
        }
    };

    // STAGES == 3: besides the two LDS stages, the 128-byte line of every tile row for
    // K block kb+2 is touched one block early with a 4-byte DMA into a per-wave scratch slot
    // of LDS, so the next block's tile loads hit L2. Each lane covers one row.
    static_assert(STAGES == 2 || STAGES == 3, "two LDS stages, optionally one L2 stage");
    static_assert(STAGES == 2 || WL == W_ROW, "the L2 stage touches row-major W lines");
    constexpr int PF_ROUNDS = (BM + BN + 64 * NWAVES - 1) / (64 * NWAVES);
    static_assert(BM % 64 == 0, "prefetch rounds split A and W rows on 64-row boundaries");
    const uint32_t lane_k = (uint32_t)(lane * K);
    auto prefetch_l2 = [&](int64_t kb) {
        const uint32_t skb = (uint32_t)(kb * 128);
        const uint32_t scratch = (uint32_t)(2 * STAGE + wave * 256);
#pragma unroll
        for (int j = 0; j < PF_ROUNDS; ++j) {
            const int row0 = (j * NWAVES + wave) * 64;          // uniform
            if (row0 < BM)
                dma4(ra, lds, scratch, lane_k, skb + (uint32_t)(row0 * K));
            else if (row0 < BM + BN)
                dma4(rw, lds, scratch, lane_k, skb + (uint32_t)((row0 - BM) * K));
        }
    };

#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) acc[sm][sn] = AccT{};

    // Per-lane LDS byte offsets of the fragment rows (sub-tile 0), chunk slots resolved.
    // A sub-tile row sm adds sm*MF*128, a W sub-tile sn adds sn*MF*128 (swz depends on r & 15).
    const int fsw = swz(frow);
    const uint32_t a_row = (uint32_t)((wm * TM + frow) * 128);
    // W fragment base of sub-tile 0 (sub-tile sn adds sn*16*128 = sn*2048 in both layouts)
    const uint32_t w_row = WL == W_ROW ? (uint32_t)((BM + wn * TN + frow) * 128)
                                       : (uint32_t)((BM + wn * TN) * 128 + lane * 16);
    // 16-byte K chunks a lane feeds to a 16x16 MFMA: fp8 row-major 2g, 2g+1 (32 contiguous
    // bytes); fp8 packed and int8 g, g+4. Slot offsets within a row (A; W row-major) and
    // within a fragment (W packed).
    const int kc0 = (QT == Q_FP8 && WL == W_ROW) ? 2 * fgrp : fgrp;
    const int kc1 = (QT == Q_FP8 && WL == W_ROW) ? 2 * fgrp + 1 : fgrp + 4;
    const uint32_t a_s0 = (uint32_t)((kc0 ^ fsw) << 4), a_s1 = (uint32_t)((kc1 ^ fsw) << 4);
    const uint32_t w_s0 = WL == W_ROW ? a_s0 : 0u, w_s1 = WL == W_ROW ? a_s1 : 1024u;

    auto lds16 = [&](uint32_t off) { return *reinterpret_cast<const v4i*>(lds + off); };

    // SPLIT_SW: c2[sm] is the scale product with the next block's weight scale
    float c2[SM];
    auto cs = [&](const float (&c)[SM], int sm, int sn) {
        if constexpr (SPLIT_SW) return sn < sn_split ? c[sm] : c2[sm];
        else { (void)sn; return c[sm]; }
    };
    (void)cs;
    // One K block on LDS stage `stage`: fragments from LDS, MFMA, scale fusion. c[sm] is the
    // scale product of sub-tile row sm (sched 0-2); ea[sm] and ew the E8M0 exponents of the
    // token and weight scales (sched 3).
    auto compute = [&](uint32_t sbase, const float (&c)[SM], const int (&ea)[SM], int ew) {
        if constexpr (SCHED == 4) {
            // accumulate the raw products; int8 keeps its exact int32 sum in acc's bits
            const uint32_t abase = sbase + a_row, wbase = sbase + w_row;
            if constexpr (QT == Q_FP8) {
                v8i af[SM];
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) {
                    const v4i lo = lds16(abase + sm * 2048 + a_s0);
                    const v4i hi = lds16(abase + sm * 2048 + a_s1);
                    af[sm] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                }
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) {
                    const v4i lo = lds16(wbase + sn * 2048 + w_s0);
                    const v4i hi = lds16(wbase + sn * 2048 + w_s1);
                    const v8i wf = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm)
                        acc[sm][sn] = mfma_fp8_16x16x128_acc(wf, af[sm], acc[sm][sn]);
                }
            } else {
                v4i af[SM][2];
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) {
                    af[sm][0] = lds16(abase + sm * 2048 + a_s0);
                    af[sm][1] = lds16(abase + sm * 2048 + a_s1);
                }
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) {
                    const v4i w0 = lds16(wbase + sn * 2048 + w_s0);
                    const v4i w1 = lds16(wbase + sn * 2048 + w_s1);
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm) {
                        v4i pi = __builtin_bit_cast(v4i, acc[sm][sn]);
                        pi = mfma_i8_16x16x64(w0, af[sm][0], pi);
                        pi = mfma_i8_16x16x64(w1, af[sm][1], pi);
                        acc[sm][sn] = __builtin_bit_cast(v4f, pi);
                    }
                }
            }
            (void)c;
            (void)ea;
            (void)ew;
        } else if constexpr (SCHED == 3) {
            const uint32_t abase = sbase + a_row, wbase = sbase + w_row;
            v8i af[SM];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const v4i lo = lds16(abase + sm * 2048 + a_s0);
                const v4i hi = lds16(abase + sm * 2048 + a_s1);
                af[sm] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const v4i lo = lds16(wbase + sn * 2048 + w_s0);
                const v4i hi = lds16(wbase + sn * 2048 + w_s1);
                const v8i wf = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int sm = 0; sm < SM; ++sm)
                    acc[sm][sn] = mfma_fp8_16x16x128_e8(wf, af[sm], acc[sm][sn], ew, ea[sm]);
            }
        } else if constexpr (MF == 32) {
            // Lane l covers row l % 32 of each 32-row sub-tile and, in K half h, the 16-byte
            // chunks 4h + 2*(l/32) and 4h + 2*(l/32) + 1. Each W fragment feeds SM pairs of
            // MFMAs (64 K each) whose sum is the block partial of a 32x32 sub-tile.
            uint32_t slo[2], shi[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                slo[h] = (uint32_t)(((4 * h + 2 * khalf) ^ fsw) << 4);
                shi[h] = (uint32_t)(((4 * h + 2 * khalf + 1) ^ fsw) << 4);
            }
            const uint32_t abase = sbase + a_row, wbase = sbase + w_row;
            auto frag = [&](uint32_t base, int h) {
                const v4i lo = lds16(base + slo[h]);
                const v4i hi = lds16(base + shi[h]);
                return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            };
            v8i af[SM][2];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                af[sm][0] = frag(abase + sm * 4096, 0);
                af[sm][1] = frag(abase + sm * 4096, 1);
            }
            // Pairs p = sn*SM + sm in order. Software-pipelined: pair p's two MFMAs go out,
            // then (on a new W sub-tile) the next W fragment's reads, then the 16 scale FMAs
            // of pair p-1, whose product has finished while p's MFMAs were issued. Two
            // product buffers and two W fragments alternate; group barriers pin the order.
            constexpr int P = SM * SN;
            v8i wf[2][2];
            wf[0][0] = frag(wbase, 0);
            wf[0][1] = frag(wbase, 1);
            v16f qb[2];
            auto scale_fma = [&](int pp) {
                v16f& a = acc[pp % SM][pp / SM];
                const v16f& q = qb[pp & 1];
                const float cc = c[pp % SM];
#pragma unroll
                for (int e = 0; e < 16; ++e) a[e] = __builtin_fmaf(q[e], cc, a[e]);
            };
#pragma unroll
            for (int pp = 0; pp < P; ++pp) {
                const int sn = pp / SM, sm = pp % SM;
                const v8i(&w)[2] = wf[sn & 1];
                qb[pp & 1] = mfma_fp8_32x32x64(w[0], af[sm][0], v16f{});
                qb[pp & 1] = mfma_fp8_32x32x64(w[1], af[sm][1], qb[pp & 1]);
                if (sm == 0 && sn + 1 < SN) {
                    wf[(sn + 1) & 1][0] = frag(wbase + (sn + 1) * 4096, 0);
                    wf[(sn + 1) & 1][1] = frag(wbase + (sn + 1) * 4096, 1);
                }
                if (pp > 0) scale_fma(pp - 1);
            }
            scale_fma(P - 1);
#pragma unroll
            for (int pp = 0; pp < P; ++pp) {
                const int sn = pp / SM, sm = pp % SM;
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                       // MFMA
                if (sm == 0 && sn + 1 < SN) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
                if (pp > 0) __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);          // VALU
            }
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        } else if constexpr (QT == Q_FP8) {
            const uint32_t abase = sbase + a_row, wbase = sbase + w_row;
            v8i af[SM];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                const v4i lo = lds16(abase + sm * 2048 + a_s0);
                const v4i hi = lds16(abase + sm * 2048 + a_s1);
                af[sm] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
            auto fma4 = [&](v4f& a, const v4f& q, float cc) {
                a.x = __builtin_fmaf(q.x, cc, a.x);
                a.y = __builtin_fmaf(q.y, cc, a.y);
                a.z = __builtin_fmaf(q.z, cc, a.z);
                a.w = __builtin_fmaf(q.w, cc, a.w);
            };
            auto read_w = [&](int sn) {
                const v4i lo = lds16(wbase + sn * 2048 + w_s0);
                const v4i hi = lds16(wbase + sn * 2048 + w_s1);
                return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            };
            if constexpr (SCHED == 0) {
                // per W sub-tile: read it, its MFMAs, their scale FMAs
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) {
                    const v8i wf = read_w(sn);
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm) fma4(acc[sm][sn], mfma_fp8_16x16x128(wf, af[sm]), cs(c, sm, sn));
                }
            } else {
                // software-pipelined: MFMAs of sub-tile sn, the read of sn+1, then the scale
                // FMAs of sn-1 (whose MFMAs finished while sn's were issued); the group
                // barriers pin that interleave so the register allocator cannot serialise it
                v8i wf = read_w(0);
                v4f pb[2][SM];
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) {
#pragma unroll
                    for (int sm = 0; sm < SM; ++sm) pb[sn & 1][sm] = mfma_fp8_16x16x128(wf, af[sm]);
                    if (sn + 1 < SN) wf = read_w(sn + 1);
                    if (sn > 0) {
#pragma unroll
                        for (int sm = 0; sm < SM; ++sm) fma4(acc[sm][sn - 1], pb[(sn - 1) & 1][sm], cs(c, sm, sn - 1));
                    }
                }
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) fma4(acc[sm][SN - 1], pb[(SN - 1) & 1][sm], cs(c, sm, SN - 1));
#pragma unroll
                for (int sn = 0; sn < SN; ++sn) {
                    __builtin_amdgcn_sched_group_barrier(0x008, SM, 0);          // MFMA
                    if (sn + 1 < SN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
                    if (sn > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4 * SM, 0);   // VALU
                }
                __builtin_amdgcn_sched_group_barrier(0x002, 4 * SM, 0);
            }
        } else {
            const uint32_t abase = sbase + a_row, wbase = sbase + w_row;
            v4i af[SM][2];
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                af[sm][0] = lds16(abase + sm * 2048 + a_s0);
                af[sm][1] = lds16(abase + sm * 2048 + a_s1);
            }
#pragma unroll
            for (int sn = 0; sn < SN; ++sn) {
                const v4i w0 = lds16(wbase + sn * 2048 + w_s0);
                const v4i w1 = lds16(wbase + sn * 2048 + w_s1);
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) {
                    v4i pi = mfma_i8_16x16x64(w0, af[sm][0], v4i{0, 0, 0, 0});
                    pi = mfma_i8_16x16x64(w1, af[sm][1], pi);
                    v4f& a = acc[sm][sn];
                    a.x = __builtin_fmaf((float)pi.x, c[sm], a.x);
                    a.y = __builtin_fmaf((float)pi.y, c[sm], a.y);
                    a.z = __builtin_fmaf((float)pi.z, c[sm], a.z);
                    a.w = __builtin_fmaf((float)pi.w, c[sm], a.w);
                }
            }
        }
    };

    auto kblock = [&](int64_t kb, int stage) {
        float c[SM];
        int ea[SM], ew = 0;
        if constexpr (SCHED == 4) {
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) { c[sm] = 0.f; ea[sm] = 0; }
        } else if constexpr (SCHED == 3) {
            const uint32_t sc = (uint32_t)(SC_BASE + stage * SC_STAGE);
            ew = (int)e8m0_of(*reinterpret_cast<const float*>(lds + sc + sw_lds));
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) {
                ea[sm] = act_scale_e8(*reinterpret_cast<const float*>(lds + sc + sa_lds + sm * 4),
                                      packed, kb);
                c[sm] = 0.f;
            }
        } else {
            const uint32_t sc = (uint32_t)(SC_BASE + stage * SC_STAGE);
            const float swv = *reinterpret_cast<const float*>(lds + sc + sw_lds);
#pragma unroll
            for (int sm = 0; sm < SM; ++sm) ea[sm] = 0;
            if constexpr (SPLIT_SW) {
                // the next block's slot is staged whenever the wave reaches into it (else unused)
                const float swv2 = *reinterpret_cast<const float*>(lds + sc + sw_lds + 4);
#pragma unroll
                for (int sm = 0; sm < SM; ++sm) {
                    const float a = act_scale(*reinterpret_cast<const float*>(lds + sc + sa_lds + sm * 4),
                                              packed, kb);
                    c[sm] = a * swv;
                    c2[sm] = a * swv2;
                }
            } else if constexpr (SM == 4) {
                const v4f sa4 = *reinterpret_cast<const v4f*>(lds + sc + sa_lds);
                c[0] = act_scale(sa4.x, packed, kb) * swv;
                c[1] = act_scale(sa4.y, packed, kb) * swv;
                c[2] = act_scale(sa4.z, packed, kb) * swv;
                c[3] = act_scale(sa4.w, packed, kb) * swv;
            } else {
#pragma unroll
                for (int sm = 0; sm < SM; ++sm)
                    c[sm] = act_scale(*reinterpret_cast<const float*>(lds + sc + sa_lds + sm * 4),
                                      packed, kb) * swv;
            }
        }
        if (kb + 1 < kb_end) issue_stage(kb + 1, stage ^ 1);
        if constexpr (STAGES == 3) {
            // near the end this re-touches the last block (harmless, keeps the loop uniform)
            __builtin_amdgcn_sched_barrier(0);
            prefetch_l2(kb + 2 < kb_end ? kb + 2 : kb_end - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        compute((uint32_t)(stage * STAGE), c, ea, ew);
        // the L2 touches (issued last) may stay in flight; everything before them must land
        if constexpr (STAGES == 3) wait_vmem_keep(PF_ROUNDS);
        else wait_vmem_all();
        __syncthreads();
    };

    if (kb_begin < kb_end) {
        issue_stage(kb_begin, 0);
        if constexpr (STAGES == 3) prefetch_l2(kb_begin + 1 < kb_end ? kb_begin + 1 : kb_begin);
        wait_vmem_all();
        __syncthreads();
        for (int64_t kb = kb_begin; kb < kb_end; ++kb) kblock(kb, (int)((kb - kb_begin) & 1));
        wait_vmem_all();      // no LDS DMA may still be in flight when the wave ends
    }

    if constexpr (SCHED == 4) {
        // acc[m][n] = ((float)P * sa[m]) * sw[n] for the lane's token m (one per sub-tile row)
        // and columns n..n+3; rows past M and columns past N take scale 0 (never stored)
        float swv[SN][4];
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            const int64_t n = n0 + wn * TN + sn * 16 + 4 * fgrp;
#pragma unroll
            for (int j = 0; j < 4; ++j) swv[sn][j] = n + j < N ? p.sw[n + j] : 0.f;
        }
#pragma unroll
        for (int sm = 0; sm < SM; ++sm) {
            const int64_t m = m0 + wm * TM + sm * 16 + frow;
            const float sav = m < M ? p.sa[m * ssm] : 0.f;
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
}

// Store a tile's accumulators: element (m, n) goes to base[base_off + m*N + n] as OT.
// Lane owns token m and, per sub-tile, columns n..n+3 (16x16) or the four column groups
// 8j + 4*(l/32) .. +3, j = 0..3 (32x32).
template <int OT, int BM, int BN, int WM, int WN, int SCHED>
__device__ __forceinline__ void std_store(
    void* base, int64_t base_off, int64_t M, int64_t N, int64_t m0, int64_t n0,
    const typename StdShape<BM, BN, WM, WN, SCHED>::AccT (
        &acc)[StdShape<BM, BN, WM, WN, SCHED>::SM][StdShape<BM, BN, WM, WN, SCHED>::SN]) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    constexpr int TM = Shape::TM, TN = Shape::TN, MF = Shape::MF, SM = Shape::SM, SN = Shape::SN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & (MF - 1), fgrp = lane >> 4, khalf = lane >> 5;
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        const int64_t m = m0 + wm * TM + sm * MF + frow;
        if (m >= M) continue;
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            if constexpr (MF == 32) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t n = n0 + wn * TN + sn * 32 + 8 * j + 4 * khalf;
                    if (n >= N) continue;
                    const auto& a = acc[sm][sn];
                    const v4f v = {a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
                    store4<OT>(base, base_off + m * N + n, v);
                }
            } else {
                const int64_t n = n0 + wn * TN + sn * 16 + 4 * fgrp;
                if (n >= N) continue;
                store4<OT>(base, base_off + m * N + n, acc[sm][sn]);
            }
        }
    }
}

// Grouped (MoE) store: tile row r < rows holds pair rows[r]; it goes to base[base_off +
// rows[r]*N + n] (the output in pair order); a pair id outside [0, M) is not stored. 16x16
// sub-tiles only.
template <int OT, int BM, int BN, int WM, int WN, int SCHED>
__device__ __forceinline__ void std_store_rows(
    void* base, int64_t base_off, int64_t M, int64_t N, int64_t n0, const int32_t* __restrict__ rows,
    int64_t nrows,
    const typename StdShape<BM, BN, WM, WN, SCHED>::AccT (
        &acc)[StdShape<BM, BN, WM, WN, SCHED>::SM][StdShape<BM, BN, WM, WN, SCHED>::SN]) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    constexpr int TM = Shape::TM, TN = Shape::TN, SM = Shape::SM, SN = Shape::SN;
    static_assert(Shape::MF == 16, "grouped tiles use 16x16 sub-tiles");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & 15, fgrp = lane >> 4;
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
        const int64_t r = wm * TM + sm * 16 + frow;
        if (r >= nrows) continue;
        const int64_t m = rows[r];
        if (m < 0 || m >= M) continue;
#pragma unroll
        for (int sn = 0; sn < SN; ++sn) {
            const int64_t n = n0 + wn * TN + sn * 16 + 4 * fgrp;
            if (n >= N) continue;
            store4<OT>(base, base_off + m * N + n, acc[sm][sn]);
        }
    }
}

// Grouped (MoE) GEMM, standard tiles: grid = N tiles x moe_max_tiles(pairs, E, BM) x split;
// blockIdx.y is the per-expert row tile (moe_tile), workgroups past the last tile exit at
// once (before any LDS traffic, uniformly).
template <int BM, int BN, int WM, int WN, int QT, int OT, int SCHED, int WL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_moe_std_kernel(GemmArgs p) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    MoeSpan sp;
    if (!moe_tile(p.moe_offsets, p.moe_experts, p.M, BM, blockIdx.y, sp)) return;
    const int64_t N = p.N, KB = p.K / 128;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int split = p.split, z = blockIdx.z;
    const int64_t kb_begin = (int64_t)z * KB / split, kb_end = (int64_t)(z + 1) * KB / split;
    typename Shape::AccT acc[Shape::SM][Shape::SN];
    std_tile<BM, BN, WM, WN, QT, SCHED, 2, WL, 1>(p, lds, sp.p0, n0, kb_begin, kb_end, acc, sp);
    const int32_t* rows = p.moe_rows + sp.p0;
    if (split == 1)
        std_store_rows<OT, BM, BN, WM, WN, SCHED>(p.out, 0, p.M, N, n0, rows, sp.p1 - sp.p0, acc);
    else
        std_store_rows<O_FP32, BM, BN, WM, WN, SCHED>(p.partials, (int64_t)z * p.M * N, p.M, N, n0,
                                                      rows, sp.p1 - sp.p0, acc);
}

// One workgroup per (tile, K split): grid = tiles x 1 x split.
template <int BM, int BN, int WM, int WN, int QT, int OT, int SCHED, int STAGES, int WL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_std_kernel(GemmArgs p) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const int64_t M = p.M, N = p.N, KB = p.K / 128;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int64_t pid_m, pid_n;
    tile_coords(blockIdx.x, tiles_m, tiles_n, p.group_m, p.raster, pid_m, pid_n);
    const int64_t m0 = pid_m * BM, n0 = pid_n * BN;
    const int split = p.split, z = blockIdx.z;
    const int64_t kb_begin = (int64_t)z * KB / split, kb_end = (int64_t)(z + 1) * KB / split;
    typename Shape::AccT acc[Shape::SM][Shape::SN];
    std_tile<BM, BN, WM, WN, QT, SCHED, STAGES, WL>(p, lds, m0, n0, kb_begin, kb_end, acc);
    if (split == 1) std_store<OT, BM, BN, WM, WN, SCHED>(p.out, 0, M, N, m0, n0, acc);
    else std_store<O_FP32, BM, BN, WM, WN, SCHED>(p.partials, (int64_t)z * M * N, M, N, m0, n0, acc);
}

// Stream-K schedule ("variant 2"): a persistent grid of G workgroups (one per CU) takes
// tiles [0, dp_tiles) whole, in rounds of G, then splits the K blocks of the remaining tiles
// evenly: workgroup w owns iterations [w*I/G, (w+1)*I/G) of the I = (tiles - dp_tiles) * KB
// (tile, K block) iterations, in tile-major order, so it may end with part of a tile and
// start with part of another. This fills the last, partial wave of tiles that a plain grid
// leaves half idle. A tile one workgroup covers whole is stored at once; a partial tile is
// parked, as fp32 in the thread's own register order, in the workgroup's slot (0 for the
// first tile of its range, 1 for the last), and a second kernel on the same stream sums each
// split tile's segments in K order and stores it. The kernel boundary publishes the slots,
// so no workgroup ever waits for or synchronises with another, and the sum order is fixed,
// so results are deterministic.
// The iterations are spread over the first Gs = min(G, I) workgroups, so each of those owns at
// least one; the owner of iteration x is max{w : floor(w*I/Gs) <= x} = ceil((x+1)*Gs/I) - 1,
// and a tile's segments are exactly the owners of its first through last iteration.
template <int BM, int BN, int WM, int WN, int SCHED>
struct SlotIO {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    using AccT = typename Shape::AccT;
    static constexpr int SM = Shape::SM, SN = Shape::SN, NT = 64 * WM * WN;
    static constexpr int64_t SLOT = (int64_t)BM * BN;   // floats per partial-tile slot
    // AccT element (sm, sn) is NQ 16-byte pieces; piece q of thread tid sits at byte
    // ((sm*SN + sn)*NQ + q)*NT*16 + tid*16 of the slot: coalesced, one per-lane offset plus a
    // constant scalar offset per access.
    static constexpr int NQ = sizeof(AccT) / 16;
    static __device__ __forceinline__ v4f piece(const AccT& a, int q) {
        if constexpr (NQ == 1) { (void)q; return a; }
        else return v4f{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
    }
    static __device__ __forceinline__ void set_piece(AccT& a, int q, const v4f& v) {
        if constexpr (NQ == 1) { (void)q; a = v; }
        else { a[4 * q] = v.x; a[4 * q + 1] = v.y; a[4 * q + 2] = v.z; a[4 * q + 3] = v.w; }
    }
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(float* slots, int64_t slot) {
        return make_rsrc(slots + uniform_i64(slot) * SLOT, (uint32_t)(SLOT * 4));
    }
    static __device__ __forceinline__ void park(float* slots, int64_t slot, const AccT (&acc)[SM][SN]) {
        const __amdgpu_buffer_rsrc_t r = rsrc(slots, slot);
        const uint32_t voff = threadIdx.x * 16;
#pragma unroll
        for (int sm = 0; sm < SM; ++sm)
#pragma unroll
            for (int sn = 0; sn < SN; ++sn)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    buf_store_v4f(r, piece(acc[sm][sn], q), voff, (uint32_t)(((sm * SN + sn) * NQ + q) * NT * 16));
    }
    // row band sm of the tile: acc_row = slot (first) or acc_row + slot
    static __device__ __forceinline__ void add_row(float* slots, int64_t slot, bool first, int sm,
                                                   AccT (&acc_row)[SN]) {
        const __amdgpu_buffer_rsrc_t r = rsrc(slots, slot);
        const uint32_t voff = threadIdx.x * 16;
#pragma unroll
        for (int sn = 0; sn < SN; ++sn)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const v4f v = buf_load_v4f(r, voff, (uint32_t)(((sm * SN + sn) * NQ + q) * NT * 16));
                set_piece(acc_row[sn], q, first ? v : piece(acc_row[sn], q) + v);
            }
    }
};

// Iteration-range helpers shared by the stream-K kernel and its fixup kernel.
__device__ __forceinline__ int64_t sk_owner(int64_t x, int64_t G, int64_t I) {
    return ((x + 1) * G + I - 1) / I - 1;
}

template <int BM, int BN, int WM, int WN, int QT, int OT, int SCHED, int STAGES, int WL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_streamk_kernel(GemmArgs p) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    using IO = SlotIO<BM, BN, WM, WN, SCHED>;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const int64_t M = p.M, N = p.N, KB = p.K / 128;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t G = gridDim.x, w = blockIdx.x;
    typename Shape::AccT acc[Shape::SM][Shape::SN];

    // Work items in order: this workgroup's whole tiles t = w, w+G, ... < dp_tiles (with G a
    // multiple of 8, tile t runs on the XCD that tile_coords assumes), then its stream-K
    // iteration range. One call site of the tile routine keeps the register budget of the
    // plain kernel.
    const int64_t n_whole = w < p.dp_tiles ? (p.dp_tiles - w + G - 1) / G : 0;
    const int64_t I = (tiles - p.dp_tiles) * KB;
    const int64_t Gs = I < G ? I : G;
    const int64_t it_lo = w < Gs ? w * I / Gs : 0, it_hi = w < Gs ? (w + 1) * I / Gs : 0;
    int64_t it = it_lo;
    for (int64_t item = 0;; ++item) {
        int64_t t, ts = 0, k0 = 0, k1 = KB;
        if (item < n_whole) {
            t = w + item * G;
        } else {
            if (it >= it_hi) break;
            ts = it / KB;
            k0 = it - ts * KB;
            k1 = (KB - k0) <= (it_hi - it) ? KB : k0 + (it_hi - it);
            t = p.dp_tiles + ts;
            it += k1 - k0;
        }
        int64_t pm, pn;
        tile_coords(uniform_i64(t), tiles_m, tiles_n, p.group_m, p.raster, pm, pn);
        const int64_t m0 = uniform_i64(pm * BM), n0 = uniform_i64(pn * BN);
        k0 = uniform_i64(k0);
        k1 = uniform_i64(k1);
        std_tile<BM, BN, WM, WN, QT, SCHED, STAGES, WL>(p, lds, m0, n0, k0, k1, acc);
        if (k0 == 0 && k1 == KB) std_store<OT, BM, BN, WM, WN, SCHED>(p.out, 0, M, N, m0, n0, acc);
        else IO::park(p.sk_slots, w * 2 + (ts == it_lo / KB ? 0 : 1), acc);
    }
}

// One workgroup per (stream-K tile, sub-tile row band sm = blockIdx.y): a tile split over
// several workgroups is summed from their parked slots in K order (ascending owner) and
// stored, one band of SM per workgroup so the sum fills the chip; a tile one workgroup covered
// whole was stored by it already. Same block shape as the GEMM, so each thread reads back
// exactly the accumulator pieces it will store.
template <int BM, int BN, int WM, int WN, int OT, int SCHED>
__global__ __launch_bounds__(64 * WM * WN) void gemm_streamk_fixup_kernel(GemmArgs p, int grid) {
    using Shape = StdShape<BM, BN, WM, WN, SCHED>;
    using IO = SlotIO<BM, BN, WM, WN, SCHED>;
    constexpr int TM = Shape::TM, TN = Shape::TN, MF = Shape::MF, SN = Shape::SN;
    const int64_t M = p.M, N = p.N, KB = p.K / 128;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t ts = blockIdx.x;
    const int sm = blockIdx.y;
    const int64_t I = (tiles - p.dp_tiles) * KB;
    const int64_t Gs = I < grid ? I : grid;
    const int64_t w_first = sk_owner(ts * KB, Gs, I), w_last = sk_owner(ts * KB + KB - 1, Gs, I);
    if (w_first == w_last) return;
    typename Shape::AccT acc[SN];
    for (int64_t ws = w_first; ws <= w_last; ++ws) {
        const int sl = ts == (ws * I / Gs) / KB ? 0 : 1;
        IO::add_row(p.sk_slots, ws * 2 + sl, ws == w_first, sm, acc);
    }
    int64_t pm, pn;
    tile_coords(p.dp_tiles + ts, tiles_m, tiles_n, p.group_m, p.raster, pm, pn);
    // the rows of band sm, as std_store writes them
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & (MF - 1), fgrp = lane >> 4, khalf = lane >> 5;
    const int64_t m = pm * BM + wm * TM + sm * MF + frow;
    if (m >= M) return;
    const int64_t n0 = pn * BN + wn * TN;
#pragma unroll
    for (int sn = 0; sn < SN; ++sn) {
        if constexpr (MF == 32) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + sn * 32 + 8 * j + 4 * khalf;
                if (n >= N) continue;
                const auto& a = acc[sn];
                const v4f v = {a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
                store4<OT>(p.out, m * N + n, v);
            }
        } else {
            (void)khalf;
            const int64_t n = n0 + sn * 16 + 4 * fgrp;
            if (n >= N) continue;
            store4<OT>(p.out, m * N + n, acc[sn]);
        }
    }
}

// Whole rounds first; only the tiles of the last, partial round are split (each split tile
// costs a parked fp32 partial per segment, written and read back once).
int64_t streamk_dp_tiles(int64_t tiles, int grid) { return (tiles / grid) * grid; }

size_t streamk_workspace_bytes(int bm, int bn, int grid) {
    return (size_t)grid * 2 * (size_t)bm * (size_t)bn * sizeof(float);
}

// Workgroups of the stream-K grid: the device's compute units (one resident workgroup each).
int streamk_grid() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus - cus % 8;                   // keep the XCD round-robin aligned
        if (cached[dev] <= 0) cached[dev] = cus;
    }
    return cached[dev];
}

template <int BM, int BN, int WM, int WN, int QT, int OT, int SCHED, int STAGES, int WL>
hipError_t launch_streamk(const GemmArgs& a, hipStream_t stream) {
    constexpr int LDS_BYTES = StdShape<BM, BN, WM, WN, SCHED>::lds_bytes(STAGES);
    const int G = streamk_grid();
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    GemmArgs b = a;
    b.dp_tiles = streamk_dp_tiles(tiles, G);
    const int64_t I = (tiles - b.dp_tiles) * (a.K / 128);
    const int64_t grid = b.dp_tiles > 0 ? G : (I < G ? I : G);
    b.sk_slots = a.partials;
    static bool attr_set = false;   // one-time opt-in to more than 64 KB of LDS
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_streamk_kernel<BM, BN, WM, WN, QT, OT, SCHED, STAGES, WL>),
            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemm_streamk_kernel<BM, BN, WM, WN, QT, OT, SCHED, STAGES, WL>),
                       dim3((unsigned)grid), dim3(64 * WM * WN), LDS_BYTES, stream, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || tiles == b.dp_tiles) return e;
    hipLaunchKernelGGL((gemm_streamk_fixup_kernel<BM, BN, WM, WN, OT, SCHED>),
                       dim3((unsigned)(tiles - b.dp_tiles), (unsigned)StdShape<BM, BN, WM, WN, SCHED>::SM),
                       dim3(64 * WM * WN), 0, stream, b, (int)grid);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int QT, int OT, int SCHED, int STAGES, int WL>
hipError_t launch_std(const GemmArgs& a, hipStream_t stream) {
    constexpr int LDS_BYTES = StdShape<BM, BN, WM, WN, SCHED>::lds_bytes(STAGES);
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles, 1, (unsigned)a.split);
    static bool attr_set = false;   // one-time opt-in to more than 64 KB of LDS
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_std_kernel<BM, BN, WM, WN, QT, OT, SCHED, STAGES, WL>),
            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemm_std_kernel<BM, BN, WM, WN, QT, OT, SCHED, STAGES, WL>), grid,
                       dim3(64 * WM * WN), LDS_BYTES, stream, a);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int QT, int OT, int SCHED, int WL>
hipError_t launch_moe_std(const GemmArgs& a, hipStream_t stream) {
    constexpr int LDS_BYTES = StdShape<BM, BN, WM, WN, SCHED>::lds_bytes(2);
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)moe_max_tiles(a.M, a.moe_experts, BM),
              (unsigned)a.split);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_moe_std_kernel<BM, BN, WM, WN, QT, OT, SCHED, WL>),
            hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemm_moe_std_kernel<BM, BN, WM, WN, QT, OT, SCHED, WL>), grid,
                       dim3(64 * WM * WN), LDS_BYTES, stream, a);
    return hipGetLastError();
}

#define BFQ_STD_ENTRY(BM, BN, WM, WN, ST, SC, QT, OT, WL)                                \
    KernelEntry{bfq_tile{0, BM, BN, 128, 1, WM, WN, ST, 8, SC, 0, 0}, QT, OT, WL,         \
                (SC) == 3 ? S_UE8M0 : (SC) == 4 ? S_CHANNEL : S_FP32,                      \
                &launch_std<BM, BN, WM, WN, QT, OT, SC, ST, WL>}

#define BFQ_STD_ALL_OUT(BM, BN, WM, WN, ST, SC, QT, WL)                                   \
    BFQ_STD_ENTRY(BM, BN, WM, WN, ST, SC, QT, O_BF16, WL),                                \
        BFQ_STD_ENTRY(BM, BN, WM, WN, ST, SC, QT, O_FP16, WL),                            \
        BFQ_STD_ENTRY(BM, BN, WM, WN, ST, SC, QT, O_FP32, WL)

static const KernelEntry kStdKernels[] = {
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 0, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 1, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 192, 4, 2, 2, 0, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 3, 1, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 2, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 2, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 0, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 3, 1, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 128, 4, 1, 3, 1, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 0, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 0, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 0, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 0, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 0, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 1, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 192, 4, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 1, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 128, 4, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 128, 4, 2, 2, 1, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 0, Q_INT8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 0, Q_INT8, W_PACKED16),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 0, Q_INT8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 3, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 3, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 3, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 3, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 3, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 3, Q_FP8, W_PACKED16),
    // per-token x per-channel scales
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 4, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 4, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 4, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 4, Q_FP8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 4, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 4, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 4, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 4, Q_FP8, W_PACKED16),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 4, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 4, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 4, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 4, Q_INT8, W_ROW),
    BFQ_STD_ALL_OUT(256, 256, 4, 2, 2, 4, Q_INT8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 256, 2, 2, 2, 4, Q_INT8, W_PACKED16),
    BFQ_STD_ALL_OUT(128, 128, 2, 2, 2, 4, Q_INT8, W_PACKED16),
    BFQ_STD_ALL_OUT(64, 128, 1, 2, 2, 4, Q_INT8, W_PACKED16),
};

#define BFQ_SK_ENTRY(BM, BN, WM, WN, ST, SC, QT, OT, WL)                                 \
    KernelEntry{bfq_tile{2, BM, BN, 128, 1, WM, WN, ST, 8, SC, 0, 0}, QT, OT, WL,         \
                (SC) == 3 ? S_UE8M0 : (SC) == 4 ? S_CHANNEL : S_FP32,                      \
                &launch_streamk<BM, BN, WM, WN, QT, OT, SC, ST, WL>}

#define BFQ_SK_ALL_OUT(BM, BN, WM, WN, ST, SC, QT, WL)                                    \
    BFQ_SK_ENTRY(BM, BN, WM, WN, ST, SC, QT, O_BF16, WL),                                 \
        BFQ_SK_ENTRY(BM, BN, WM, WN, ST, SC, QT, O_FP16, WL),                             \
        BFQ_SK_ENTRY(BM, BN, WM, WN, ST, SC, QT, O_FP32, WL)

static const KernelEntry kStreamKKernels[] = {
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 0, Q_FP8, W_ROW),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 1, Q_FP8, W_ROW),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 0, Q_INT8, W_ROW),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 0, Q_FP8, W_PACKED16),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 1, Q_FP8, W_PACKED16),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 0, Q_INT8, W_PACKED16),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 3, Q_FP8, W_ROW),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 3, Q_FP8, W_PACKED16),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 4, Q_FP8, W_ROW),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 4, Q_FP8, W_PACKED16),
    BFQ_SK_ALL_OUT(256, 256, 4, 2, 2, 4, Q_INT8, W_PACKED16),
};

#define BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, OT, WL)                                  \
    KernelEntry{bfq_tile{0, BM, BN, 128, 1, WM, WN, 2, 1, SC, 0, 0}, QT, OT, WL,              \
                (SC) == 3 ? S_UE8M0 : S_FP32, &launch_moe_std<BM, BN, WM, WN, QT, OT, SC, WL>, 1}
#define BFQ_MOE_STD(BM, BN, WM, WN, SC, QT)                                                 \
    BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, O_BF16, W_ROW),                              \
        BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, O_FP16, W_ROW),                          \
        BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, O_FP32, W_ROW),                          \
        BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, O_BF16, W_PACKED16),                     \
        BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, O_FP16, W_PACKED16),                     \
        BFQ_MOE_STD_ENTRY(BM, BN, WM, WN, SC, QT, O_FP32, W_PACKED16)

// grouped (MoE) standard tiles, fp8 (the gathered rows cost registers: 256x256 with sched 0
// spills with packed weights, the software-pipelined sched 1 fits in 240 VGPRs; it takes
// large token counts, where one 256-row tile covers each expert's rows and its weights
// stream once per expert)
static const KernelEntry kMoeStdKernels[] = {
    BFQ_MOE_STD(128, 256, 2, 2, 0, Q_FP8),
    BFQ_MOE_STD(128, 128, 2, 2, 0, Q_FP8),
    BFQ_MOE_STD(64, 128, 1, 2, 0, Q_FP8),
    BFQ_MOE_STD(256, 256, 4, 2, 1, Q_FP8),
    BFQ_MOE_STD(256, 256, 4, 2, 3, Q_FP8),
    BFQ_MOE_STD(128, 128, 2, 2, 3, Q_FP8),
};

const KernelEntry* moe_std_kernels(int* count) {
    *count = (int)(sizeof(kMoeStdKernels) / sizeof(kMoeStdKernels[0]));
    return kMoeStdKernels;
}

const KernelEntry* streamk_kernels(int* count) {
    *count = (int)(sizeof(kStreamKKernels) / sizeof(kStreamKKernels[0]));
    return kStreamKKernels;
}

const KernelEntry* std_kernels(int* count) {
    *count = (int)(sizeof(kStdKernels) / sizeof(kStdKernels[0]));
    return kStdKernels;
}

}  // namespace bfq
