"""Expected values for the parity gate of the on-device tile sweep -- TEST INFRASTRUCTURE.

The sweep (block_scaled_w8a8_amd/sweep.py, `tune --reference`) times every compiled kernel
configuration and keeps the fastest one whose output meets the parity bar. This script
writes what it is compared with: for each (N, K, code type, scale format) and each M of the
grid, the oracle's fp32 GEMM output at seeded sample positions, computed on the sweep's own
seeded inputs (block_scaled_w8a8_amd/synth.py: weights seed 0, activations seed 0 at the
grid's largest M, quantized here by the oracle, which the device quantizers match bit for
bit). The file is plain numpy data (no pickles); the sweep reads it and never imports this
package.

  python -m oracle.sweep_reference --out PATH [--shapes N,K ...] [--dtype fp8|int8]
                                   [--scales fp32|ue8m0|channel] [--grid M ...] [--samples S]

Sample positions of (N, K, M): numpy default_rng(N * 1_000_003 + K * 1009 + M) draws S rows
in [0, M) and S columns in [0, N); the first and last row and column are appended.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
M_GRID = (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512, 1024, 1536, 2048, 3072, 4096)


def key(N: int, K: int, dtype: str, scales: str, M: int) -> str:
    return f"{N}x{K}:{dtype}:{scales}:{M}"


def sample_positions(N: int, K: int, M: int, samples: int):
    rng = np.random.default_rng(N * 1_000_003 + K * 1009 + M)
    ms = np.concatenate([rng.integers(0, M, samples), [0, M - 1]]).astype(np.int64)
    ns = np.concatenate([rng.integers(0, N, samples), [0, N - 1]]).astype(np.int64)
    return ms, ns


def reference(N: int, K: int, dtype: str, scales: str, grid, samples: int) -> dict:
    if REPO not in sys.path:
        sys.path.insert(0, REPO)
    import oracle
    from block_scaled_w8a8_amd import synth
    qt = oracle.FP8 if dtype == "fp8" else oracle.INT8
    sf = oracle.SCALE_UE8M0 if scales == "ue8m0" else oracle.SCALE_FP32
    channel = scales == "channel"
    m_max = max(grid)
    x = synth.activations(m_max, K, seed=0)
    w = synth.weights(N, K, seed=0).numpy()
    qa, sa = oracle.quant_groups(synth.bf16_bits(x), group=K if channel else 128, qtype=qt,
                                 scale_fmt=sf)
    qw, sw = oracle.quant_blocks(w, block=(1, K) if channel else (128, 128), qtype=qt,
                                 scale_fmt=sf)
    out = {}
    for M in grid:
        ms, ns = sample_positions(N, K, M, samples)
        f = oracle.channel_gemm_sampled if channel else oracle.block_gemm_sampled
        ref = f(qa[:M], sa[:M], qw, sw, ms, ns, qtype=qt)
        k = key(N, K, dtype, scales, M)
        out[k + ":ms"], out[k + ":ns"] = ms, ns
        out[k + ":ref"] = np.asarray(ref, dtype=np.float32)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--shapes", nargs="*", default=None, help="N,K pairs")
    ap.add_argument("--dtype", default="fp8", choices=["fp8", "int8"])
    ap.add_argument("--scales", default="fp32", choices=["fp32", "ue8m0", "channel"])
    ap.add_argument("--grid", type=int, nargs="*", default=list(M_GRID))
    ap.add_argument("--samples", type=int, default=1024)
    args = ap.parse_args()
    shapes = ([tuple(int(v) for v in s.split(",")) for s in args.shapes] if args.shapes else
              ([(1536, 7168)] if args.dtype == "int8" else
               [(24576, 7168), (7168, 1536), (1536, 7168), (4096, 7168), (7168, 18432),
                (18432, 7168), (1536, 1536), (3072, 7168), (7168, 2304)]))
    data = {}
    if os.path.exists(args.out):
        with np.load(args.out, allow_pickle=False) as old:
            data.update({k: old[k] for k in old.files})
    for N, K in shapes:
        print(f"[sweep_reference] N={N} K={K} {args.dtype} {args.scales}", flush=True)
        data.update(reference(N, K, args.dtype, args.scales, args.grid, args.samples))
    np.savez(args.out, **data)


if __name__ == "__main__":
    main()
