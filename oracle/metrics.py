"""Accuracy metrics used by the tests -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

calc_diff follows the global similarity measure of the block GEMM benchmark page
("vLLM DeepGEMM FP8 Block GEMM 基准测试 ...", §4.4): both tensors in float64,
1 - 2*sum(x*y) / sum(x*x + y*y). The other helpers implement the element-wise tolerance
of the parity tests: relative Frobenius error and max |diff| against 2^-7 * rms(ref) + 1e-3.
"""
from __future__ import annotations

import numpy as np


def calc_diff(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    denom = (x * x + y * y).sum()
    return float(1.0 - 2.0 * (x * y).sum() / denom)


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt((x * x).mean())) if x.size else 0.0


def rel_frobenius(out, ref) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(out - ref) / den) if den > 0 else float(np.linalg.norm(out))


def max_abs_diff(out, ref) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(out - ref).max()) if out.size else 0.0


def max_diff_bound(ref) -> float:
    """Element-wise bound of the parity bar: 2^-7 * rms(ref) + 1e-3."""
    return 2.0 ** -7 * rms(ref) + 1e-3


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def gemm_fp32_report(out, ref) -> dict:
    """The parity bar for an fp32 GEMM output against the oracle's fp32 accumulator:
    relative Frobenius error <= 1e-3 and max |diff| <= 2^-7 * rms(ref) + 1e-3."""
    rf = rel_frobenius(out, ref)
    md = max_abs_diff(out, ref)
    bound = max_diff_bound(ref)
    return {"rel_frobenius": rf, "max_abs_diff": md, "max_diff_bound": bound,
            "ok": bool(rf <= 1e-3 and md <= bound)}


def bf16_straddle_report(out16_bits, ref16_bits, gpu32, ref32) -> dict:
    """The bf16-output reading of the parity bar. out16 vs the oracle's bf16 output:
    relative Frobenius <= 1e-3; every element beyond 2^-7*rms(ref)+1e-3 must be exactly one
    bf16 step from the oracle's value, with the rounding midpoint between the two lying
    between the oracle's fp32 accumulator and the GPU's own fp32 accumulator (same tile),
    i.e. the difference is the bf16 rounding of an fp32 difference the fp32 bar bounds."""
    o16 = np.asarray(out16_bits, dtype=np.uint16)
    r16 = np.asarray(ref16_bits, dtype=np.uint16)
    of = bf16_bits_to_f32(o16).astype(np.float64)
    rf = bf16_bits_to_f32(r16).astype(np.float64)
    ref32 = np.asarray(ref32, dtype=np.float64)
    gpu32 = np.asarray(gpu32, dtype=np.float64)
    rel = rel_frobenius(of, rf)
    bound = max_diff_bound(rf)
    bad = np.abs(of - rf) > bound
    unexplained = 0
    if bad.any():
        ob, rb = o16[bad].astype(np.int32), r16[bad].astype(np.int32)
        one_step = np.abs(ob - rb) == 1
        mid = (of[bad] + rf[bad]) / 2.0
        lo = np.minimum(ref32[bad], gpu32[bad])
        hi = np.maximum(ref32[bad], gpu32[bad])
        straddle = (mid >= lo) & (mid <= hi)
        unexplained = int((~(one_step & straddle)).sum())
    return {"rel_frobenius": rel, "beyond_bound": int(bad.sum()), "unexplained": unexplained,
            "ok": bool(rel <= 1e-3 and unexplained == 0)}
