"""Benchmark of the block-scaled W8A8 hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: for every M of the
workload, per-token-group quantization of the bf16 activations (bfq_quant_tokens) followed
by the block-scaled GEMM against pre-quantized weights (bfq_block_gemm, tile chosen by
bfq_select_tile). Weights are quantized on the device before timing (the offline step of
the block GEMM benchmark page §4.1). Inputs are resident in HBM when timing starts.

Default workload: N=24576, K=7168 (DeepSeek-V3 wide MoE up-projection) over the 18-point M
grid 1..4096. To keep the weight stream honest against the 256 MB Infinity Cache, launches
rotate over R copies of the weights (default 3 -> 528 MB working set, over twice the cache).
The weight codes sit in HBM in the packed fragment layout by default (--w-layout row for the
row-major [N, K] form); packing, like the weight quantization, is an offline step.

Prints ONE JSON line (metric, value = GEMM TFLOPS over the whole step including the
quantization time, per-M detail, roofline of the dominant kernel, CPU-oracle baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

METRIC = "block-FP8 GEMM TFLOPS & HBM GB/s vs M (1-4096) at DeepSeek-V3 N/K, 1 MI355X"

M_GRID = [1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512, 1024, 1536, 2048, 3072, 4096]
WORKLOADS = {
    "mgrid": {"shapes": [(24576, 7168)], "M": M_GRID, "qtype": "fp8",
              "desc": "block-FP8 linear N=24576 K=7168, M grid 1..4096 (18 points): "
                      "token-group quant + block GEMM per M"},
    "decode": {"shapes": [(7168, 1536), (1536, 7168)],
               "M": [1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128], "qtype": "fp8",
               "desc": "decode sweep (N,K) in {(7168,1536),(1536,7168)}, M 1..128"},
    "dense": {"shapes": [(4096, 7168), (7168, 18432), (18432, 7168)], "M": [8, 64, 128, 4096],
              "qtype": "fp8", "desc": "dense comparison shapes, M in {8,64,128,4096}"},
    "int8": {"shapes": [(1536, 7168)], "M": [1, 16, 128, 1024, 4096], "qtype": "int8",
             "desc": "int8_w8a8 block variant N=1536 K=7168"},
    "tiny": {"shapes": [(1536, 1536)], "M": [8], "qtype": "fp8", "desc": "M=8 N=1536 K=1536"},
    # one GPU's share of an 8-way tensor-parallel split: the 24576x7168 layer column-parallel
    # (N/8 per GPU, no exchange) and the 7168x18432 layer row-parallel (K/8 per GPU, whose
    # fp32 partials an all-reduce would then sum: not measured here)
    "tp8": {"shapes": [(3072, 7168), (7168, 2304)], "M": M_GRID, "qtype": "fp8",
            "desc": "per-GPU shard shapes of 8-way tensor parallelism: N=3072 K=7168 "
                    "(column-parallel 24576x7168) and N=7168 K=2304 (row-parallel 7168x18432), "
                    "M grid 1..4096"},
    "moe": {"kind": "moe", "E": 256, "topk": 8, "shapes": [(4096, 7168)], "M": M_GRID,
            "qtype": "fp8",
            "desc": "MoE grouped block-FP8, DeepSeek-V3 routed experts E=256 top-8, gate+up "
                    "N=4096 K=7168, tokens T over the 18-point grid: token-group quant + routing "
                    "sort + grouped GEMM per T (uniform synthetic routing)"},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_name(t, qtype: str, wl: int, out: str = "bf16", channel: bool = False) -> str:
    """The demangled name of the device kernel a tile launches (as rocprofv3 prints it)."""
    q = 0 if qtype == "fp8" else 1
    o = {"bf16": 0, "fp16": 1, "fp32": 2}[out]
    d = t.as_dict()
    if d["variant"] in (0, 2):
        kern = "gemm_std_kernel" if d["variant"] == 0 else "gemm_streamk_kernel"
        return (f"bfq::{kern}<{d['bm']}, {d['bn']}, {d['waves_m']}, {d['waves_n']}, "
                f"{q}, {o}, {d['sched']}, {d['stages']}, {wl}>")
    nwr = d["bn"] // d["waves_n"]
    kern = "gemm_swapab_lds_kernel" if d["sched"] == 1 else "gemm_swapab_kernel"
    return (f"bfq::{kern}<{d['bm']}, {nwr}, {d['waves_n']}, {d['waves_m']}, "
            f"{d['stages']}, {q}, {o}, {wl}, {int(channel)}>")


def grid_threads(t, M, N) -> int:
    d = t.as_dict()
    if d["variant"] == 2:
        return 256 * 64 * d["waves_m"] * d["waves_n"]
    if d["variant"] == 0:
        wg = -(-M // d["bm"]) * -(-N // d["bn"]) * d["split_k"]
        return wg * 64 * d["waves_m"] * d["waves_n"]
    wg = -(-N // d["bn"]) * -(-M // d["bm"]) * d["split_k"]
    return wg * 64 * d["waves_n"] * d["waves_m"]


def tile_key(t) -> str:
    d = t.as_dict()
    return "v{variant}_bm{bm}_bn{bn}_w{waves_m}x{waves_n}_s{stages}_c{sched}_g{group_m}_r{raster}_k{split_k}".format(**d)


def run_gpu(args, wl):
    import torch

    from block_scaled_w8a8_amd import bfq, perf, synth

    dev = torch.device("cuda:0")
    qd = bfq.BFQ_E4M3FN if wl["qtype"] == "fp8" else bfq.BFQ_INT8
    wlay = bfq.BFQ_W_PACKED16 if args.w_layout == "packed" else bfq.BFQ_W_ROW_MAJOR
    sfmt = bfq.BFQ_SCALE_UE8M0 if args.scales == "ue8m0" else bfq.BFQ_SCALE_FP32
    channel = args.scales == "channel"       # per-token x per-channel scales
    m_max = max(wl["M"])
    packed = args.scale_layout == "packed"     # UE8M0 codes, four groups per 32-bit word
    col = args.scale_layout == "col" or packed  # both address every M through one ld
    if packed and args.scales != "ue8m0":
        raise SystemExit("--scale-layout packed needs --scales ue8m0")
    if packed and wl["qtype"] != "fp8":
        raise SystemExit("--scale-layout packed is read by the e4m3fn GEMM only")
    shapes = []
    host = {}
    for (N, K) in wl["shapes"]:
        log(f"[bench] setup N={N} K={K}: generating and quantizing weights on the device")
        w = synth.weights(N, K, seed=0)
        x = synth.activations(m_max, K, seed=0)
        wd = w.to(dev)
        copies = []
        for r in range(args.rotate):
            qw, sw = bfq.quant_weight_blocks(wd, q_dtype=qd, scale_fmt=sfmt, per_channel=channel)
            if wlay == bfq.BFQ_W_PACKED16:        # offline layout step, like the quantization
                qw = bfq.pack_weights(qw)
            copies.append((qw, sw))
        del wd
        xd = x.to(dev)
        qa = torch.empty((m_max, K), dtype=torch.uint8 if qd == bfq.BFQ_E4M3FN else torch.int8,
                         device=dev)
        G = 1 if channel else K // 128       # activation scales per token
        bs = bfq.channel_block_shape(K) if channel else bfq.BLOCK_SHAPE
        if packed:
            sa = torch.empty(((G + 3) // 4, (m_max + 3) // 4 * 4), dtype=torch.int32, device=dev)
        else:
            sa = torch.empty((G, m_max) if col else (m_max, G), dtype=torch.float32, device=dev)
        out = torch.empty((m_max, N), dtype=torch.bfloat16, device=dev)
        plans = []
        for M in wl["M"]:
            st, tile = bfq.bfq_select_tile(M, N, K, qd, bfq.BFQ_BF16, w_layout=wlay,
                                           scale_fmt=sfmt, block_shape=bs)
            ws_bytes = bfq.bfq_gemm_workspace_bytes(M, N, K, tile)
            plans.append((M, tile, ws_bytes, st))
        ws_max = max(p[2] for p in plans)
        ws = torch.empty(max(ws_max, 16), dtype=torch.uint8, device=dev)
        shapes.append(dict(N=N, K=K, copies=copies, xd=xd, qa=qa, sa=sa, out=out, plans=plans,
                           ws=ws, ws_max=ws_max, bs=bs, group=K if channel else 128))
        host[(N, K)] = (w, x)
    torch.cuda.synchronize()

    launch_counter = [0]

    def one_step():
        for sh in shapes:
            for (M, tile, ws_bytes, _st) in sh["plans"]:
                qw, sw = sh["copies"][launch_counter[0] % len(sh["copies"])]
                launch_counter[0] += 1
                lay = (bfq.BFQ_SCALES_PACKED_UE8M0 if packed else
                       bfq.BFQ_SCALES_COL_MAJOR if col else bfq.BFQ_SCALES_ROW_MAJOR)
                sa_m = sh["sa"] if col else sh["sa"][:M]
                bfq.bfq_quant_tokens(sh["xd"][:M], sh["qa"][:M], sa_m, layout=lay,
                                     scale_ld=sh["sa"].stride(0), scale_fmt=sfmt,
                                     group_size=sh["group"])
                bfq.bfq_block_gemm(sh["qa"][:M], sa_m, qw, sw, sh["out"][:M], a_layout=lay,
                                   a_scale_ld=sh["sa"].stride(0), tile=tile, workspace=sh["ws"],
                                   workspace_bytes=sh["ws_max"], w_layout=wlay, scale_fmt=sfmt,
                                   block_shape=sh["bs"])

    one_step()                        # eager reference result for the graph check
    torch.cuda.synchronize()
    eager_out = [sh["out"].clone() for sh in shapes]

    # One step captured as a HIP graph: the timed region replays it, so host launch cost
    # (ctypes + Python, ~10 us per call) does not leak into the measurement.
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        launch_counter[0] = 0
        with torch.cuda.graph(graph):
            one_step()
        torch.cuda.synchronize()

    def replay():
        if graph is not None:
            graph.replay()
        else:
            one_step()

    # untimed warm-up steps (the pages' protocol warms up 100 iterations before timing; the
    # first tens of milliseconds of sustained load run measurably slower)
    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()

    # timed region: wall clock around exactly `steps` steps, fenced by synchronize
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for sh, ref in zip(shapes, eager_out):          # replayed graph == eager result
        if not torch.equal(sh["out"], ref):
            raise RuntimeError("graph replay output differs from the eager step")

    # Per-launch durations, per M: R back-to-back launches of the quantizer, then of the GEMM
    # (rotating the weight copies as the step does), each captured in a graph and replayed
    # between two HIP events on the stream the kernels run on; duration = elapsed / R. A
    # single launch bracketed by events would add the event overhead (several us) to
    # kernels of ~30 us.
    stream = torch.cuda.current_stream()
    lay = (bfq.BFQ_SCALES_PACKED_UE8M0 if packed else
           bfq.BFQ_SCALES_COL_MAJOR if col else bfq.BFQ_SCALES_ROW_MAJOR)
    R = args.launch_reps
    per = {}
    for sh in shapes:
        N, K = sh["N"], sh["K"]
        sa_all = sh["sa"]
        for (M, tile, ws_bytes, _st) in sh["plans"]:
            sa_m = sa_all if col else sa_all[:M]

            def q_once():
                bfq.bfq_quant_tokens(sh["xd"][:M], sh["qa"][:M], sa_m, layout=lay,
                                     scale_ld=sa_all.stride(0), scale_fmt=sfmt,
                                     group_size=sh["group"])

            def g_once(i, rotate=True):
                qw, sw = sh["copies"][i % len(sh["copies"]) if rotate else 0]
                bfq.bfq_block_gemm(sh["qa"][:M], sa_m, qw, sw, sh["out"][:M], a_layout=lay,
                                   a_scale_ld=sa_all.stride(0), tile=tile, workspace=sh["ws"],
                                   workspace_bytes=sh["ws_max"], w_layout=wlay, scale_fmt=sfmt,
                                   block_shape=sh["bs"])

            res = {}
            # "h": the same GEMM with one weight copy for every launch (hot caches, the pages'
            # style of timing), a secondary figure beside the rotating one
            for name, fn in (("q", lambda i: q_once()), ("g", g_once),
                             ("h", lambda i: g_once(i, rotate=False))):
                fn(0)
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for i in range(R):
                        fn(i)
                gr.replay()                          # warm
                torch.cuda.synchronize()
                vals = []
                for _ in range(args.launch_rounds):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    gr.replay()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    vals.append(e0.elapsed_time(e1) * 1e-3 / R)
                del gr
                res[name] = vals
            per[(N, K, M)] = {"key": tile_key(tile), "q": res["q"], "g": res["g"], "h": res["h"]}

    flops_step = sum(perf.gemm_flops(M, sh["N"], sh["K"]) for sh in shapes
                     for (M, *_r) in sh["plans"])
    step_s = wall / args.steps
    rows = []
    groups = {}
    for sh in shapes:
        N, K = sh["N"], sh["K"]
        for (M, tile, ws_bytes, st) in sh["plans"]:
            r = per[(N, K, M)]
            g = sum(r["g"]) / len(r["g"])
            q = sum(r["q"]) / len(r["q"])
            rows.append({
                "M": M, "N": N, "K": K, "tile": tile.as_dict(), "tuned": st == 0,
                "gemm_us": round(g * 1e6, 2),
                "gemm_us_hot": round(sum(r["h"]) / len(r["h"]) * 1e6, 2),
                "quant_us": round(q * 1e6, 2),
                "tflops": round(perf.tflops(M, N, K, g), 2),
                "gbs_page": round(perf.gbs_page(M, N, K, g), 1),
                "gbs_all": round(perf.gbs_all(M, N, K, g, channel=channel), 1),
                "bound": perf.bound(M, N, K, channel=channel),
                "roofline_frac": round(perf.roofline_time_s(M, N, K, channel=channel) / g, 4),
                "quant_gbs": round(perf.quant_bytes(M, K, channel) / q / 1e9, 1),
            })
            gr = groups.setdefault(r["key"], {"t": 0.0, "n": 0, "flops": 0.0, "bytes": 0.0,
                                              "name": kernel_name(tile, wl["qtype"], wlay,
                                                                  channel=channel),
                                              "grids": set()})
            gr["grids"].add(grid_threads(tile, M, N))
            gr["t"] += sum(r["g"]) * R
            gr["n"] += len(r["g"]) * R
            gr["flops"] += perf.gemm_flops(M, N, K) * len(r["g"]) * R
            gr["bytes"] += perf.gemm_bytes_all(M, N, K, channel=channel) * len(r["g"]) * R
    dom_key = max(groups, key=lambda k: groups[k]["t"])
    dom = groups[dom_key]
    t_flop = dom["flops"] / (perf.FP8_PEAK_TFLOPS * 1e12)
    t_byte = dom["bytes"] / (perf.HBM_PEAK_GBS * 1e9)
    peak_tf = perf.FP8_PEAK_TFLOPS if wl["qtype"] == "fp8" else perf.INT8_PEAK_TOPS
    if t_flop >= t_byte:
        achieved = dom["flops"] / dom["t"] / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4)}
    else:
        achieved = dom["bytes"] / dom["t"] / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": perf.HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / perf.HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_for(args, dom, wl)
    roof["kernel"] = dom["name"]
    roof["tile"] = dom_key
    roof["grid_threads"] = sorted(dom["grids"])
    roof["launches"] = dom["n"]
    roof["avg_launch_us"] = round(dom["t"] / dom["n"] * 1e6, 2)
    return {
        "value": flops_step / step_s / 1e12,
        "ms_per_step": step_s * 1e3,
        "rows": rows,
        "roofline": roof,
        "ceilings": measured_ceilings(),
        "host": host,
        "batch_invariant": bfq.bfq_get_batch_invariant(),
    }


def measured_ceilings():
    """What this GPU sustains in practice, beside the published peaks: the fp8 MFMA-only probe
    of the library (register operands, no memory traffic, 16 waves per CU) and a plain 1 GiB
    device-to-device copy (torch's copy kernel; bytes read + bytes written per second). Each
    is the best of three event-timed launches on the current stream."""
    import torch

    from block_scaled_w8a8_amd import bfq
    stream = torch.cuda.current_stream()
    blocks, iters = 512, 20000
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    flops = float(bfq.lib.bfq_probe_mfma_flops(blocks, iters))
    t_mfma = best(lambda: bfq.bfq_probe_mfma_peak(blocks, iters, out))
    t_copy = best(lambda: dst.copy_(src))
    del src, dst, out
    return {"mfma_fp8_tflops": round(flops / t_mfma / 1e12, 1),
            "copy_gbs": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "how": "fp8 16x16x128 MFMA chains on register operands, 512 workgroups x 8 waves; "
                   "1 GiB device copy, read + write bytes"}


def run_gpu_moe(args, wl):
    """The grouped (MoE) workload: per token count T, quantize T tokens, sort their top-k
    routes by expert, run the grouped GEMM. Expert weights are drawn and quantized on the
    device before timing (offline, like the dense weights); launches rotate over
    args.rotate copies of the 7.5 GB expert stack."""
    import torch

    from block_scaled_w8a8_amd import bfq, perf, synth

    dev = torch.device("cuda:0")
    E, topk = wl["E"], wl["topk"]
    (N, K), = wl["shapes"]
    wlay = bfq.BFQ_W_PACKED16 if args.w_layout == "packed" else bfq.BFQ_W_ROW_MAJOR
    sfmt = bfq.BFQ_SCALE_UE8M0 if args.scales == "ue8m0" else bfq.BFQ_SCALE_FP32
    if args.scales == "channel":
        raise SystemExit("the grouped GEMM takes block scales")
    t_max = max(wl["M"])
    log(f"[bench] moe setup: {E} experts of N={N} K={K}, {args.rotate} copies")
    copies = []
    for r in range(args.rotate):
        qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            q, s_ = bfq.quant_weight_blocks(synth.expert_weight_on(dev, e, N, K, seed=0),
                                            scale_fmt=sfmt)
            qw[e].copy_(q)
            sw[e].copy_(s_)
        if wlay == bfq.BFQ_W_PACKED16:
            qw = bfq.pack_weights(qw)
        copies.append((qw, sw))
    torch.cuda.synchronize()
    x = synth.activations(t_max, K, seed=0)
    ids_host = synth.routing(t_max, E, topk, seed=0)
    xd, ids = x.to(dev), ids_host.to(dev)
    qa = torch.empty((t_max, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, t_max), dtype=torch.float32, device=dev)   # column-major
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(t_max * topk, dtype=torch.int32, device=dev)
    aws = torch.empty(max(int(bfq.lib.bfq_moe_align_workspace_bytes(t_max, topk, E)), 16),
                      dtype=torch.uint8, device=dev)
    out = torch.empty((t_max * topk, N), dtype=torch.bfloat16, device=dev)
    plans = []
    for T in wl["M"]:
        st, tile = bfq.bfq_moe_select_tile(T, topk, E, N, K, bfq.BFQ_BF16, wlay, sfmt)
        plans.append((T, tile, bfq.bfq_moe_gemm_workspace_bytes(T, topk, N, tile), st))
    ws_max = max(p_[2] for p_ in plans)
    ws = torch.empty(max(ws_max, 16), dtype=torch.uint8, device=dev)
    col = bfq.BFQ_SCALES_COL_MAJOR
    counter = [0]

    def q_once(T):
        bfq.bfq_quant_tokens(xd[:T], qa[:T], sa, layout=col, scale_ld=t_max, scale_fmt=sfmt)

    def a_once(T):
        bfq.bfq_moe_align(ids[:T], E, off, srt, workspace=aws)

    def g_once(T, tile, i):
        qw, sw = copies[i % len(copies)]
        bfq.bfq_moe_block_gemm(qa[:T], sa, srt, off, topk, qw, sw, out[:T * topk], a_layout=col,
                               a_scale_ld=t_max, tile=tile, workspace=ws, workspace_bytes=ws_max,
                               w_layout=wlay, scale_fmt=sfmt)

    def one_step():
        for (T, tile, _b, _st) in plans:
            q_once(T)
            a_once(T)
            g_once(T, tile, counter[0])
            counter[0] += 1

    one_step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    counter[0] = 0
    with torch.cuda.graph(graph):
        one_step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):      # untimed warm-up steps
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stream = torch.cuda.current_stream()
    R = args.launch_reps
    rows, groups = [], {}
    flops_step = 0.0
    for (T, tile, _b, st) in plans:
        res = {}
        for name, fn in (("q", lambda i: q_once(T)), ("a", lambda i: a_once(T)),
                         ("g", lambda i: g_once(T, tile, i))):
            fn(0)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for i in range(R):
                    fn(i)
            gr.replay()
            torch.cuda.synchronize()
            vals = []
            for _ in range(args.launch_rounds):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                gr.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                vals.append(e0.elapsed_time(e1) * 1e-3 / R)
            del gr
            res[name] = sum(vals) / len(vals)
        P = T * topk
        active = len(set(ids_host[:T].reshape(-1).tolist()))
        flops = perf.gemm_flops(P, N, K)
        byts = perf.moe_gemm_bytes(T, topk, active, N, K)
        flops_step += flops
        g = res["g"]
        rows.append({"T": T, "pairs": P, "active_experts": active, "tile": tile.as_dict(),
                     "tuned": st == 0, "gemm_us": round(g * 1e6, 2),
                     "quant_us": round(res["q"] * 1e6, 2), "align_us": round(res["a"] * 1e6, 2),
                     "tflops": round(flops / g / 1e12, 2), "gbs_all": round(byts / g / 1e9, 1),
                     "roofline_frac": round(max(byts / (perf.HBM_PEAK_GBS * 1e9),
                                                flops / (perf.FP8_PEAK_TFLOPS * 1e12)) / g, 4)})
        key = tile_key(tile)
        gr_ = groups.setdefault(key, {"t": 0.0, "flops": 0.0, "bytes": 0.0, "n": 0,
                                      "name": moe_kernel_name(tile, wlay)})
        gr_["t"] += g
        gr_["flops"] += flops
        gr_["bytes"] += byts
        gr_["n"] += 1
    dom_key = max(groups, key=lambda k: groups[k]["t"])
    dom = groups[dom_key]
    if dom["flops"] / (perf.FP8_PEAK_TFLOPS * 1e12) >= dom["bytes"] / (perf.HBM_PEAK_GBS * 1e9):
        a_ = dom["flops"] / dom["t"] / 1e12
        roof = {"bound": "mfma", "achieved": round(a_, 2), "peak": perf.FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a_ / perf.FP8_PEAK_TFLOPS, 4)}
    else:
        a_ = dom["bytes"] / dom["t"] / 1e9
        roof = {"bound": "hbm", "achieved": round(a_, 1), "peak": perf.HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(a_ / perf.HBM_PEAK_GBS, 4)}
    roof.update({"traffic": None, "kernel": dom["name"], "tile": dom_key,
                 "avg_launch_us": round(dom["t"] / dom["n"] * 1e6, 2), "launches": dom["n"] * R})
    step_s = wall / args.steps
    return {"value": flops_step / step_s / 1e12, "ms_per_step": step_s * 1e3, "rows": rows,
            "roofline": roof, "host": {"moe": (x, ids_host)},
            "batch_invariant": bfq.bfq_get_batch_invariant()}


def moe_kernel_name(t, wl: int) -> str:
    d = t.as_dict()
    if d["variant"] == 0:
        return (f"bfq::gemm_moe_std_kernel<{d['bm']}, {d['bn']}, {d['waves_m']}, {d['waves_n']}, "
                f"0, 0, {d['sched']}, {wl}>")
    nwr = d["bn"] // d["waves_n"]
    kern = "gemm_swapab_lds_kernel" if d["sched"] == 1 else "gemm_swapab_kernel"
    return (f"bfq::{kern}<{d['bm']}, {nwr}, {d['waves_n']}, {d['waves_m']}, {d['stages']}, "
            f"0, 0, {wl}, 0, 1>")


def cpu_baseline_moe(wl, host, target_s: float, scales: str = "fp32"):
    """The oracle on a bounded sample of the grouped workload: quantization and grouped GEMM of
    the first r tokens against their experts' weights (only those experts are drawn and
    quantized, untimed)."""
    import numpy as np
    import torch

    import oracle
    from block_scaled_w8a8_amd import perf, synth

    E, topk = wl["E"], wl["topk"]
    (N, K), = wl["shapes"]
    x, ids = host["moe"]
    sf = oracle.SCALE_UE8M0 if scales == "ue8m0" else oracle.SCALE_FP32
    xb = synth.bf16_bits(x)
    cache = {}

    def experts_for(rows):
        used = list(dict.fromkeys(ids[:rows].reshape(-1).tolist()))
        for e in used:
            if e not in cache:
                cache[e] = oracle.quant_blocks(
                    synth.expert_weight_on("cuda:0", e, N, K, seed=0).cpu().numpy(), scale_fmt=sf)
        remap = {e: i for i, e in enumerate(used)}
        sub = np.vectorize(remap.get)(ids[:rows].numpy()).astype(np.int32)
        return (np.stack([cache[e][0] for e in used]), np.stack([cache[e][1] for e in used]), sub)

    def run(rows):
        qw, sw, sub = experts_for(rows)
        t0 = time.perf_counter()
        qa, sa = oracle.quant_groups(np.ascontiguousarray(xb[:rows]), scale_fmt=sf)
        oracle.moe_gemm(qa, sa, sub, qw, sw)
        return time.perf_counter() - t0

    # a few tokens (their experts are drawn on the device and quantized by the oracle,
    # untimed), the timed part repeated to about target_s
    rows = 8
    run(rows)
    reps, total = 0, 0.0
    while total < target_s and reps < 10000:
        total += run(rows)
        reps += 1
    t = total / reps
    log(f"[bench] cpu baseline (moe): {rows} tokens, {reps} repetitions, {t:.3f} s each")
    return {"value": perf.gemm_flops(rows * topk, N, K) / t / 1e12, "unit": "TFLOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"quant + grouped GEMM of {rows} tokens x top-{topk} against their experts "
                      f"(N={N} K={K}), {reps} repetitions, {total:.1f} s"}


def traffic_for(args, dom, wl):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 --pmc summary,
    if it was taken on this kernel (same name, same grid sizes, same kernel sources)."""
    from block_scaled_w8a8_amd import profile_summary
    path = os.path.join(REPO, "profiles", f"gemm_traffic_{args.workload}.txt")
    if not os.path.exists(path):
        return None
    t = profile_summary.read_traffic(path)
    if (t.get("kernel_sources") != profile_summary.source_hash()
            or dom["name"] not in t.get("kernel", "")
            or t.get("grid_threads") != ",".join(str(g) for g in sorted(dom["grids"]))):
        return None
    return float(t["hbm_bytes_per_dispatch"])


def cpu_baseline(wl, host, target_s: float, scales: str = "fp32"):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: the
    quantization and GEMM of a few token rows of the largest M against the full weights."""
    import numpy as np

    import oracle
    from block_scaled_w8a8_amd import perf, synth

    qt = oracle.FP8 if wl["qtype"] == "fp8" else oracle.INT8
    (N, K) = wl["shapes"][0]
    w, x = host[(N, K)]
    sf = oracle.SCALE_UE8M0 if scales == "ue8m0" else oracle.SCALE_FP32
    channel = scales == "channel"
    log(f"[bench] cpu baseline: oracle weight quantization N={N} K={K} (untimed)")
    qw, sw = oracle.quant_blocks(w.numpy(), block=(1, K) if channel else (128, 128), qtype=qt,
                                 scale_fmt=sf)
    xb = synth.bf16_bits(x)

    def run(rows):
        t0 = time.perf_counter()
        qa, sa = oracle.quant_groups(np.ascontiguousarray(xb[:rows]), group=K if channel else 128,
                                     qtype=qt, scale_fmt=sf)
        if channel:
            oracle.channel_gemm(qa, sa, qw, sw, qtype=qt)
        else:
            oracle.block_gemm(qa, sa, qw, sw, qtype=qt)
        return time.perf_counter() - t0

    t1 = run(1)
    rows = int(max(1, min(xb.shape[0], target_s / max(t1, 1e-6))))
    log(f"[bench] cpu baseline: {rows} rows (1 row took {t1:.2f} s)")
    t = run(rows)
    return {"value": perf.gemm_flops(rows, N, K) / t / 1e12, "unit": "TFLOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"quant + GEMM of {rows} token rows against the full N={N} K={K} "
                      f"weights ({t:.1f} s)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed ones (the pages warm up 100 iterations)")
    ap.add_argument("--workload", default="mgrid", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate", type=int, default=3, help="weight copies rotated per launch")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--launch-reps", type=int, default=20,
                    help="back-to-back launches per graph when timing one kernel")
    ap.add_argument("--launch-rounds", type=int, default=3, help="graph replays per kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--scale-layout", default="col", choices=["row", "col", "packed"],
                    help="activation-scale layout written by the quantizer and read by the GEMM")
    ap.add_argument("--scales", default="fp32", choices=["fp32", "ue8m0", "channel"],
                    help="scale format: 1x128 / 128x128 block scales as fp32 amax/Qmax "
                         "(default) or rounded up to a power of two (UE8M0); or 'channel', "
                         "one fp32 scale per token and per output channel")
    ap.add_argument("--w-layout", default="packed", choices=["row", "packed"],
                    help="weight-code layout in HBM (packed: bfq_pack_weights, done offline)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)
    wl = WORKLOADS[args.workload]
    moe = wl.get("kind") == "moe"
    if moe and args.rotate == 3:
        args.rotate = 2          # 2 x 7.5 GB of expert weights already spill the 256 MB cache
    res = run_gpu_moe(args, wl) if moe else run_gpu(args, wl)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = (cpu_baseline_moe if moe else cpu_baseline)(wl, res["host"], args.cpu_seconds,
                                                          args.scales)
    line = {
        "metric": METRIC,
        "value": round(res["value"], 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn" if wl["qtype"] == "fp8" else "int8",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "shapes_NK": wl["shapes"], "M": wl["M"],
                   **({"E": wl["E"], "topk": wl["topk"], "M_is": "tokens"} if moe else {}),
                   "block_shape": [1, wl["shapes"][0][1]] if args.scales == "channel" else [128, 128],
                   "out_dtype": "bf16",
                   "weight_copies_rotated": args.rotate,
                   "activation_scale_layout": ("packed_ue8m0_words" if args.scale_layout == "packed"
                                               else args.scale_layout + "_major"),
                   "weight_layout": "packed16" if args.w_layout == "packed" else "row_major",
                   "batch_invariant": bool(res.get("batch_invariant")),
                   "scales": args.scales},
        "roofline": res["roofline"],
        "ceilings": res.get("ceilings"),
        "cpu_baseline": cpu,
        "per_m": res["rows"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
