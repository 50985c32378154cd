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
