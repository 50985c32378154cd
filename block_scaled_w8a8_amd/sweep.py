"""On-device tile sweep that fills the tile table, and a single-shape runner for profiling.

  python -m block_scaled_w8a8_amd.sweep tune  --reference PATH [--shapes N,K ...]
                                             [--dtype fp8|int8] [--scales fp32|ue8m0|channel]
                                             [--w-layout row|packed] [--out PATH]
                                             [--grid M ...] [--force | --merge]
  python -m block_scaled_w8a8_amd.sweep run   --M 4096 --N 24576 --K 7168 [--tile JSON] [--iters 50]
                                             [--w-layout row|packed]
  python -m block_scaled_w8a8_amd.sweep tune-moe [--E 256 --topk 8 --shape 4096,7168]
                                             [--w-layout row|packed] [--scales fp32|ue8m0]
                                             [--grid T ...] [--merge]
  python -m block_scaled_w8a8_amd.sweep copy  [--bytes N]   (byte-counter calibration)
  python -m block_scaled_w8a8_amd.sweep libref --M 4096 --N 24576 --K 7168 [--eager 10]
                                             (the vendor library's per-tensor fp8 GEMM)

`tune` follows the tuning flow of the config-mechanism page ("vLLM 量化 Kernel 配置机制 ...",
§3.3): for every (N, K) and every M of the 18-point grid, every compiled kernel configuration
(combined with split-K factors) is launched after warm-up and timed with events; the fastest
one whose output meets the parity bar against expected values is kept. The expected values
are the oracle's fp32 outputs at seeded sample positions of the same seeded inputs, read
from a numpy file that `python -m oracle.sweep_reference` writes (--reference); this module
never imports the oracle. Configurations the library
rejects (grid or workspace limits) are skipped, like the page's OutOfResources candidates.
Results are written to a JSON tile table after every shape, and shapes already present in the
output file are skipped, so an interrupted sweep resumes where it stopped (--force retunes
them; --merge retunes only the --grid sizes of an existing entry and keeps its other
configurations, e.g. after a new kernel is added for some range of M). Each weight layout
(row-major or packed) and scale format has entries of its own; "channel" is the per-token x
per-channel format (block_shape [1, K]).

Timing rotates over enough copies of the weights and activations to exceed the 256 MB
Infinity Cache, so the weight stream is measured from HBM.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_TABLE = os.path.join(HERE, "tables", "gfx950.json")
M_GRID = [1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512, 1024, 1536, 2048, 3072, 4096]
DEFAULT_SHAPES = {"fp8": [(24576, 7168), (7168, 1536), (1536, 7168), (4096, 7168), (7168, 18432),
                          (18432, 7168), (1536, 1536), (3072, 7168), (7168, 2304)],
                  "int8": [(1536, 7168)]}
SPLITS = (1, 2, 3, 4, 6, 8, 12, 16)
NUM_CUS = 256
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Problem:
    """Device buffers for one (N, K) and the largest M, with rotation copies."""

    def __init__(self, N, K, m_max, qname, rotate=None, layout="col", w_layout="row",
                 scales="fp32"):
        import torch

        from . import bfq, synth
        self.N, self.K, self.qname = N, K, qname
        self.qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
        dev = torch.device("cuda:0")
        x = synth.activations(m_max, K, seed=0).to(dev)
        w = synth.weights(N, K, seed=0).to(dev)
        self.sf = bfq.BFQ_SCALE_UE8M0 if scales == "ue8m0" else bfq.BFQ_SCALE_FP32
        self.channel = scales == "channel"
        self.bs = bfq.channel_block_shape(K) if self.channel else bfq.BLOCK_SHAPE
        qw, sw = bfq.quant_weight_blocks(w, q_dtype=self.qd, scale_fmt=self.sf,
                                         per_channel=self.channel)
        self.wl = bfq.BFQ_W_PACKED16 if w_layout == "packed" else bfq.BFQ_W_ROW_MAJOR
        if self.wl == bfq.BFQ_W_PACKED16:
            qw = bfq.pack_weights(qw)
        self.layout = bfq.BFQ_SCALES_COL_MAJOR if layout == "col" else bfq.BFQ_SCALES_ROW_MAJOR
        qa, sa = bfq.quant_tokens(x, q_dtype=self.qd, layout=self.layout, scale_fmt=self.sf,
                                  per_token=self.channel)
        del w, x
        foot = N * K + m_max * K
        if rotate is None:
            rotate = max(1, min(8, -(-(2 * MALL_BYTES) // max(foot, 1))))
        self.sets = [(qa, sa, qw, sw)]
        for _ in range(rotate - 1):
            self.sets.append((qa.clone(), sa.clone(), qw.clone(), sw.clone()))
        self.out = torch.empty((m_max, N), dtype=torch.bfloat16, device=dev)
        self.out32 = torch.empty((m_max, N), dtype=torch.float32, device=dev)
        self.ws = None
        self.ws_bytes = 0
        torch.cuda.synchronize()

    def workspace(self, nbytes):
        import torch
        if nbytes > self.ws_bytes:
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
            self.ws_bytes = nbytes
        return self.ws

    def launch(self, M, tile, i=0, out32=False):
        from . import bfq
        qa, sa, qw, sw = self.sets[i % len(self.sets)]
        need = bfq.bfq_gemm_workspace_bytes(M, self.N, self.K, tile)
        ws = self.workspace(need) if need else None
        out = self.out32 if out32 else self.out
        sa_m = sa if self.layout == bfq.BFQ_SCALES_COL_MAJOR else sa[:M]
        return bfq.bfq_block_gemm(qa[:M], sa_m, qw, sw, out[:M], a_layout=self.layout,
                                  a_scale_ld=sa.stride(0), tile=tile, workspace=ws,
                                  workspace_bytes=need, w_layout=self.wl, scale_fmt=self.sf,
                                  block_shape=self.bs)

    def time_us(self, M, tile, warmup=3, iters=20, reps=3):
        """Median over reps of the mean time of `iters` back-to-back launches, replayed from a
        captured graph (no host launch cost between kernels); rotation over the copies."""
        import torch
        for i in range(warmup):
            self.launch(M, tile, i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(iters):
                self.launch(M, tile, i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        res = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) * 1e3 / iters)
        del g
        res.sort()
        return res[len(res) // 2]


def candidates(qd, M, N, K, wl=0, sf=0, block_shape=(128, 128)):
    """Compiled kernels x split-K factors x tile orders worth timing at this shape: the
    streaming kernel only while it re-reads the weights at most 4 times, split-K only while
    the grid is short of 4 workgroups per CU, tile orders only for multi-tile grids."""
    from . import bfq
    out = []
    KB = K // 128
    for i in range(bfq.bfq_num_tile_candidates(qd, wl, sf, block_shape=block_shape)):
        t = bfq.bfq_get_tile_candidate(i, qd, wl, sf, block_shape=block_shape)
        if t.variant == 1 and M > 4 * t.bm:
            continue
        if t.variant in (0, 2) and M <= 16 and t.bm > 64:
            continue
        if t.variant == 1:
            ctas = -(-N // t.bn) * -(-M // t.bm)
            orders = [(1, 0)]
        else:
            ctas = -(-M // t.bm) * -(-N // t.bn)
            orders = [(8, 0), (2, 1)] if ctas >= 64 else [(8, 0)]
        for s in SPLITS:
            if s > KB or KB // s < 2 or (s > 1 and ctas * s > 4 * NUM_CUS):
                continue
            if t.variant == 2 and s > 1:        # stream-K splits K by itself
                continue
            for g, r in orders:
                d = t.as_dict()
                d["split_k"] = s
                d["group_m"], d["raster"] = g, r
                out.append(bfq.bfq_tile.from_dict(d))
    return out


def agrees(a, b) -> bool:
    """Parity gate between two fp32 outputs of the same inputs (different tiles): relative
    Frobenius <= 1e-3 and max |diff| <= 2^-7 rms + 1e-3. Used by the grouped (MoE) tuner."""
    import torch
    a64, b64 = a.double(), b.double()
    den = torch.linalg.norm(b64)
    rf = float(torch.linalg.norm(a64 - b64) / den) if den > 0 else float(torch.linalg.norm(a64))
    rms = float(torch.sqrt((b64 * b64).mean()))
    md = float((a64 - b64).abs().max())
    return rf <= 1e-3 and md <= 2.0 ** -7 * rms + 1e-3


def reference_key(N, K, dtype, scales, M) -> str:
    """Key of one (shape, code type, scale format, M) in the expected-value file that the
    oracle's sweep_reference script writes."""
    return f"{N}x{K}:{dtype}:{scales}:{M}"


def meets_bar(got, ref) -> bool:
    """The parity bar on sampled fp32 outputs against the expected values: relative
    Frobenius <= 1e-3 and max |diff| <= 2^-7 * rms(expected) + 1e-3."""
    import numpy as np
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape or not np.isfinite(g).all():
        return False
    den = np.linalg.norm(r)
    rf = np.linalg.norm(g - r) / den if den > 0 else np.linalg.norm(g)
    md = np.abs(g - r).max() if g.size else 0.0
    rms = np.sqrt((r * r).mean()) if r.size else 0.0
    return bool(rf <= 1e-3 and md <= 2.0 ** -7 * rms + 1e-3)


class Reference:
    """Expected sampled outputs (numpy .npz written by the oracle's sweep_reference script)."""

    def __init__(self, path):
        import numpy as np
        self.path = path
        self.data = np.load(path, allow_pickle=False)

    def get(self, N, K, dtype, scales, M):
        k = reference_key(N, K, dtype, scales, M)
        if k + ":ref" not in self.data.files:
            raise SystemExit(f"{self.path} has no expected values for {k}; write them with "
                             f"python -m oracle.sweep_reference --out {self.path} "
                             f"--shapes {N},{K} --dtype {dtype} --scales {scales}")
        return self.data[k + ":ms"], self.data[k + ":ns"], self.data[k + ":ref"]


def warm_up(prob, M, seconds=1.0):
    """About a second of sustained launches before anything is timed: the engine clock ramps
    up over the first fraction of a second under load, which would otherwise make the first
    candidates look slower than they are."""
    import torch

    from . import bfq
    _, tile = bfq.bfq_select_tile(M, prob.N, prob.K, prob.qd, bfq.BFQ_BF16, w_layout=prob.wl,
                                  scale_fmt=prob.sf, block_shape=prob.bs)
    t0, i = time.time(), 0
    while time.time() - t0 < seconds:
        for _ in range(8):
            prob.launch(M, tile, i)
            i += 1
        torch.cuda.synchronize()


def tune_shape(N, K, qname, grid, budget_s, reference, w_layout="row", scales="fp32"):
    """Every candidate of every M of the grid: launched, gated on the expected values (the
    oracle's, at sampled positions, from `reference`), then timed; the fastest passing one
    is kept."""
    import torch

    from . import bfq
    prob = Problem(N, K, max(grid), qname, w_layout=w_layout, scales=scales)
    warm_up(prob, max(grid))
    results = {}
    for M in grid:
        t0 = time.time()
        ms, ns, ref = reference.get(N, K, qname, scales, M)
        ms_d = torch.from_numpy(ms).to("cuda:0")
        ns_d = torch.from_numpy(ns).to("cuda:0")
        best = None
        trials = []
        for tile in candidates(prob.qd, M, N, K, prob.wl, prob.sf, prob.bs):
            if time.time() - t0 > budget_s:
                break
            try:
                prob.launch(M, tile, out32=True)
                torch.cuda.synchronize()
            except bfq.BfqError:
                continue                           # rejected: limits of this configuration
            if not meets_bar(prob.out32[ms_d, ns_d].cpu().numpy(), ref):
                log(f"  parity gate rejected {tile.as_dict()} at M={M}")
                continue
            us = prob.time_us(M, tile)
            trials.append((us, tile.as_dict()))
            if best is None or us < best[0]:
                best = (us, tile)
        trials.sort(key=lambda t: t[0])
        for us, d in trials[:4]:
            log(f"    {us:9.2f} us  {d}")
        if best is None:
            raise RuntimeError(f"no candidate passed the parity gate for N={N} K={K} {qname} "
                               f"M={M} within {budget_s} s")
        results[M] = (best[0], best[1].as_dict())
        d = best[1].as_dict()
        log(f"  N={N} K={K} M={M:5d}: {best[0]:9.2f} us  variant={d['variant']} bm={d['bm']} "
            f"bn={d['bn']} split={d['split_k']} ({time.time() - t0:.1f} s)")
    del prob
    torch.cuda.empty_cache()
    return results


class MoeProblem:
    """Device buffers of a grouped (MoE) layer: E experts of [N, K] (drawn and quantized on
    the device), t_max tokens with their routing, sorted per token count on demand."""

    def __init__(self, E, topk, N, K, t_max, w_layout="row", scales="fp32"):
        import torch

        from . import bfq, synth
        self.E, self.topk, self.N, self.K = E, topk, N, K
        dev = torch.device("cuda:0")
        self.sf = bfq.BFQ_SCALE_UE8M0 if scales == "ue8m0" else bfq.BFQ_SCALE_FP32
        self.wl = bfq.BFQ_W_PACKED16 if w_layout == "packed" else bfq.BFQ_W_ROW_MAJOR
        qw = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
        sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=dev)
        for e in range(E):
            q, s_ = bfq.quant_weight_blocks(synth.expert_weight_on(dev, e, N, K, seed=0),
                                            scale_fmt=self.sf)
            qw[e].copy_(q)
            sw[e].copy_(s_)
        self.qw = bfq.pack_weights(qw) if self.wl == bfq.BFQ_W_PACKED16 else qw
        self.sw = sw
        self.qa, self.sa = bfq.quant_tokens(synth.activations(t_max, K, seed=0).to(dev),
                                            layout=bfq.BFQ_SCALES_COL_MAJOR, scale_fmt=self.sf)
        self.ids = synth.routing(t_max, E, topk, seed=0).to(dev)
        self.out = torch.empty((t_max * topk, N), dtype=torch.float32, device=dev)
        self.ws = None
        self.ws_bytes = 0
        torch.cuda.synchronize()

    def route(self, T):
        from . import bfq
        self.off, self.srt = bfq.moe_align(self.ids[:T].contiguous(), self.E)

    def launch(self, T, tile):
        import torch

        from . import bfq
        need = bfq.bfq_moe_gemm_workspace_bytes(T, self.topk, self.N, tile)
        if need > self.ws_bytes:
            self.ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
            self.ws_bytes = need
        return bfq.bfq_moe_block_gemm(self.qa[:T], self.sa, self.srt, self.off, self.topk, self.qw,
                                      self.sw, self.out[:T * self.topk],
                                      a_layout=bfq.BFQ_SCALES_COL_MAJOR, a_scale_ld=self.sa.stride(0),
                                      tile=tile, workspace=self.ws if need else None,
                                      workspace_bytes=need, w_layout=self.wl, scale_fmt=self.sf)

    def time_us(self, T, tile, iters=20, reps=3):
        import torch
        self.launch(T, tile)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(iters):
                self.launch(T, tile)
        g.replay()
        torch.cuda.synchronize()
        res = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) * 1e3 / iters)
        del g
        return sorted(res)[len(res) // 2]


def moe_candidates(wl, sf, T, topk, E, K):
    """Grouped kernels x split-K {1, 2, 4} (split only while rows per expert are few)."""
    from . import bfq
    out = []
    pairs = T * topk
    rows = -(-pairs // min(E, pairs))
    for i in range(bfq.bfq_moe_num_tile_candidates(wl, sf)):
        t = bfq.bfq_moe_get_tile_candidate(i, wl, sf)
        if t.variant == 1 and rows > 4 * t.bm:
            continue
        if t.variant == 0 and rows <= 16:
            continue
        for s in (1, 2, 4):
            if s > 1 and (rows > 64 or K // 128 // s < 4):
                continue
            d = t.as_dict()
            d["split_k"] = s
            out.append(bfq.bfq_tile.from_dict(d))
    return out


def cmd_tune_moe(args):
    import torch

    from . import bfq
    N, K = (int(v) for v in args.shape.split(","))
    grid = args.grid or M_GRID
    prob = MoeProblem(args.E, args.topk, N, K, max(grid), args.w_layout, args.scales)
    results = {}
    for T in grid:
        t0 = time.time()
        prob.route(T)
        _, ref_tile = bfq.bfq_moe_select_tile(T, args.topk, args.E, N, K, bfq.BFQ_FP32, prob.wl, prob.sf)
        prob.launch(T, ref_tile)
        torch.cuda.synchronize()
        ref = prob.out[:T * args.topk].clone()
        best = None
        for tile in moe_candidates(prob.wl, prob.sf, T, args.topk, args.E, K):
            if time.time() - t0 > args.budget:
                break
            try:
                prob.launch(T, tile)
                torch.cuda.synchronize()
            except bfq.BfqError:
                continue
            if not agrees(prob.out[:T * args.topk], ref):
                log(f"  parity gate rejected {tile.as_dict()} at T={T}")
                continue
            us = prob.time_us(T, tile)
            if best is None or us < best[0]:
                best = (us, tile)
        if best is None:
            raise RuntimeError(f"no grouped candidate passed the parity gate for E={args.E} N={N} "
                               f"K={K} T={T} within {args.budget} s")
        results[T] = (best[0], best[1].as_dict())
        d = best[1].as_dict()
        log(f"  moe E={args.E} N={N} K={K} T={T:5d}: {best[0]:9.2f} us  variant={d['variant']} "
            f"bm={d['bm']} bn={d['bn']} sched={d['sched']} split={d['split_k']} ({time.time() - t0:.1f} s)")
    table = load_table(args.out)
    wname = "packed16" if args.w_layout == "packed" else "row_major"
    entry = {"N": N, "K": K, "dtype": "fp8_w8a8", "block_shape": [128, 128], "E": args.E,
             "configs": {str(T): {k: v for k, v in t.items() if k != "bk"} for T, (us, t) in results.items()},
             "us": {str(T): round(us, 3) for T, (us, t) in results.items()}}
    if wname != "row_major":
        entry["w_layout"] = wname
    if args.scales == "ue8m0":
        entry["scales"] = "ue8m0"

    def key(e):
        return (e.get("E", 0), e["N"], e["K"], e["dtype"], e.get("w_layout", "row_major"),
                e.get("scales", "fp32"), e.get("block_shape", [128, 128])[0])
    old = next((e for e in table["entries"] if key(e) == key(entry)), None)
    if args.merge and old is not None:
        merge_configs(old, entry)
    table["entries"] = [e for e in table["entries"] if key(e) != key(entry)] + [entry]
    save_table(args.out, table)
    print(json.dumps({"table": args.out, "entries": len(table["entries"])}))


def merge_configs(old, entry):
    """Retuned batch sizes of `entry` replace theirs in `old`; old's other sizes are kept."""
    for f in ("configs", "us"):
        merged = dict(old.get(f, {}), **entry[f])
        entry[f] = {m: merged[m] for m in sorted(merged, key=int)}


def load_table(path):
    if os.path.exists(path):
        with open(path) as f:
            return json.load(f)
    return {"device": "gfx950", "entries": []}


def save_table(path, table):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(table, f, indent=1)
    os.replace(tmp, path)


def cmd_tune(args):
    qname = args.dtype
    reference = Reference(args.reference)
    shapes = [tuple(int(v) for v in s.split(",")) for s in args.shapes] if args.shapes \
        else DEFAULT_SHAPES[qname]
    table = load_table(args.out)
    dname = "fp8_w8a8" if qname == "fp8" else "int8_w8a8"
    wname = "packed16" if args.w_layout == "packed" else "row_major"

    def key(e):   # grouped (E > 0) entries are other keys
        sc = "channel" if e.get("block_shape", [128, 128])[0] == 1 else e.get("scales", "fp32")
        return (e["N"], e["K"], e["dtype"], e.get("w_layout", "row_major"), sc, e.get("E", 0))

    done = {key(e) for e in table["entries"]}
    for (N, K) in shapes:
        k0 = (N, K, dname, wname, args.scales, 0)
        old = next((e for e in table["entries"] if key(e) == k0), None)
        if k0 in done and not (args.force or args.merge):
            log(f"[sweep] N={N} K={K} {dname} {wname} {args.scales}: already in {args.out}, skipped")
            continue
        log(f"[sweep] N={N} K={K} {dname} {wname} {args.scales}")
        res = tune_shape(N, K, qname, args.grid or M_GRID, args.budget, reference, args.w_layout,
                         args.scales)
        entry = {"N": N, "K": K, "dtype": dname,
                 "block_shape": [1, K] if args.scales == "channel" else [128, 128],
                 "configs": {str(M): {k: v for k, v in t.items() if k != "bk"}
                             for M, (us, t) in res.items()},
                 "us": {str(M): round(us, 3) for M, (us, t) in res.items()}}
        if wname != "row_major":
            entry["w_layout"] = wname
        if args.scales == "ue8m0":
            entry["scales"] = args.scales
        if args.merge and old is not None:
            merge_configs(old, entry)
        table["entries"] = [e for e in table["entries"] if key(e) != k0] + [entry]
        save_table(args.out, table)
    print(json.dumps({"table": args.out, "entries": len(table["entries"])}))


def cmd_run(args):
    import torch

    from . import bfq
    prob = Problem(args.N, args.K, args.M, args.dtype, rotate=args.rotate, layout=args.layout,
                   w_layout=args.w_layout, scales=args.scales)
    if args.tile:
        tile = bfq.bfq_tile.from_dict(json.loads(args.tile))
    else:
        _, tile = bfq.bfq_select_tile(args.M, args.N, args.K, prob.qd, bfq.BFQ_BF16,
                                      w_layout=prob.wl, scale_fmt=prob.sf, block_shape=prob.bs)
    if args.eager:
        # plain launches, no graph: for counter collection, which wants one dispatch per call
        for i in range(args.eager):
            prob.launch(args.M, tile, i)
        torch.cuda.synchronize()
        print(json.dumps({"M": args.M, "N": args.N, "K": args.K, "tile": tile.as_dict(),
                          "eager_launches": args.eager}), flush=True)
        return
    us = prob.time_us(args.M, tile, warmup=3, iters=args.iters, reps=1)
    from . import perf
    s = us * 1e-6
    print(json.dumps({"M": args.M, "N": args.N, "K": args.K, "tile": tile.as_dict(), "us": us,
                      "tflops": perf.tflops(args.M, args.N, args.K, s),
                      "gbs_all": perf.gbs_all(args.M, args.N, args.K, s)}), flush=True)
    torch.cuda.synchronize()


def cmd_copy(args):
    """A plain device-to-device copy of known size: the reference the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) are scaled against."""
    import torch
    n = args.bytes
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    for _ in range(args.iters):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "iters": args.iters}), flush=True)


def cmd_libref(args):
    """A reference point, not this library: the vendor library's fp8 GEMM with one scale per
    tensor (torch._scaled_mm, hipBLASLt on ROCm) on codes of the same shape, bf16 out. torch
    offers no 1x128 / 128x128 block-scaled form on ROCm, so this is the nearest library
    kernel. Times --iters launches (weights rotated like `run`) or, with --eager, only
    launches them (for a profiler)."""
    import torch

    from . import synth
    dev = "cuda:0"
    M, N, K = args.M, args.N, args.K
    a = synth.codes(M, K, seed=1, device=dev).view(torch.float8_e4m3fn)
    copies = [synth.codes(N, K, seed=2 + r, device=dev).view(torch.float8_e4m3fn)
              for r in range(args.rotate)]
    one = torch.ones((), device=dev)

    def f(i):
        return torch._scaled_mm(a, copies[i % len(copies)].t(), scale_a=one, scale_b=one,
                                out_dtype=torch.bfloat16)
    f(0)
    torch.cuda.synchronize()
    if args.eager:
        for i in range(args.eager):
            f(i)
        torch.cuda.synchronize()
        print(json.dumps({"M": M, "N": N, "K": K, "eager": args.eager}), flush=True)
        return
    t0 = time.time()
    while time.time() - t0 < 1.0:
        f(0)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.iters):
        f(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.iters
    print(json.dumps({"M": M, "N": N, "K": K, "us": round(us, 2),
                      "tflops": round(2 * M * N * K / us / 1e6, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("tune")
    t.add_argument("--shapes", nargs="*")
    t.add_argument("--dtype", default="fp8", choices=["fp8", "int8"])
    t.add_argument("--grid", type=int, nargs="*")
    t.add_argument("--out", default=DEFAULT_TABLE)
    t.add_argument("--budget", type=float, default=20.0, help="seconds per (shape, M)")
    t.add_argument("--force", action="store_true")
    t.add_argument("--merge", action="store_true",
                   help="retune only the --grid batch sizes of an existing entry, keep its other M")
    t.add_argument("--w-layout", default="row", choices=["row", "packed"])
    t.add_argument("--scales", default="fp32", choices=["fp32", "ue8m0", "channel"])
    t.add_argument("--reference", required=True,
                   help="expected sampled outputs (python -m oracle.sweep_reference --out PATH)")
    r = sub.add_parser("run")
    r.add_argument("--M", type=int, required=True)
    r.add_argument("--N", type=int, required=True)
    r.add_argument("--K", type=int, required=True)
    r.add_argument("--dtype", default="fp8", choices=["fp8", "int8"])
    r.add_argument("--tile")
    r.add_argument("--iters", type=int, default=50)
    r.add_argument("--rotate", type=int, default=None)
    r.add_argument("--eager", type=int, default=0, help="launch this many times without timing")
    r.add_argument("--layout", default="col", choices=["row", "col"], help="activation scales")
    r.add_argument("--w-layout", default="row", choices=["row", "packed"])
    r.add_argument("--scales", default="fp32", choices=["fp32", "ue8m0", "channel"])
    tm = sub.add_parser("tune-moe")
    tm.add_argument("--E", type=int, default=256)
    tm.add_argument("--topk", type=int, default=8)
    tm.add_argument("--shape", default="4096,7168", help="N,K of one expert")
    tm.add_argument("--grid", type=int, nargs="*")
    tm.add_argument("--out", default=DEFAULT_TABLE)
    tm.add_argument("--budget", type=float, default=20.0, help="seconds per token count")
    tm.add_argument("--w-layout", default="row", choices=["row", "packed"])
    tm.add_argument("--scales", default="fp32", choices=["fp32", "ue8m0"])
    tm.add_argument("--merge", action="store_true",
                    help="retune only the --grid token counts of an existing entry, keep the rest")
    c = sub.add_parser("copy")
    c.add_argument("--bytes", type=int, default=1 << 30)
    c.add_argument("--iters", type=int, default=3)
    lr = sub.add_parser("libref")
    lr.add_argument("--M", type=int, required=True)
    lr.add_argument("--N", type=int, required=True)
    lr.add_argument("--K", type=int, required=True)
    lr.add_argument("--iters", type=int, default=20)
    lr.add_argument("--rotate", type=int, default=3)
    lr.add_argument("--eager", type=int, default=0, help="launch this many times without timing")
    args = ap.parse_args()
    {"tune": cmd_tune, "tune-moe": cmd_tune_moe, "run": cmd_run, "copy": cmd_copy,
     "libref": cmd_libref}[args.cmd](args)


if __name__ == "__main__":
    main()
