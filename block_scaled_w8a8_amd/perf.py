"""Throughput formulas of the block GEMM and the quantizer, and the MI355X peaks they are
priced against.

The pages' formulas (block GEMM benchmark page, "vLLM DeepGEMM FP8 Block GEMM 基准测试 ...",
§4.3): TFLOPS = 2*m*n*k / t / 1e12 and GB/s = (m*k + k*n + 2*m*n) / t, i.e. fp8 inputs of one
byte per element, a bf16 output, and no scale bytes. ``gemm_bytes_all`` also counts the
fp32 scales and the real output width; it is the algorithmic byte count used for the
roofline. ``channel`` selects the per-token x per-channel format (Helion linear-backend page,
scope section): one fp32 scale per token and per output channel instead of per 1x128 group
and 128x128 block.
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA


def gemm_flops(m: int, n: int, k: int) -> float:
    return 2.0 * m * n * k


def gemm_bytes_page(m: int, n: int, k: int) -> float:
    """The pages' byte count: fp8 A and B, bf16 C; scales not counted."""
    return float(m * k + k * n + 2 * m * n)


def scale_bytes(m: int, n: int, k: int, channel: bool = False) -> float:
    if channel:
        return float(4 * m + 4 * n)
    return float(4 * m * (k // 128) + 4 * (n // 128) * (k // 128))


def gemm_bytes_all(m: int, n: int, k: int, out_bytes: int = 2, channel: bool = False) -> float:
    """Every byte the method must move once: codes, fp32 scales, output."""
    return float(m * k + n * k + out_bytes * m * n) + scale_bytes(m, n, k, channel)


def quant_bytes(m: int, k: int, channel: bool = False) -> float:
    """bf16 in, one code byte out, one fp32 scale per 128 elements (per token: per row)."""
    return float(2 * m * k + m * k) + (4.0 * m if channel else 4.0 * m * (k // 128))


def tflops(m: int, n: int, k: int, seconds: float) -> float:
    return gemm_flops(m, n, k) / seconds / 1e12


def gbs_page(m: int, n: int, k: int, seconds: float) -> float:
    return gemm_bytes_page(m, n, k) / seconds / 1e9


def gbs_all(m: int, n: int, k: int, seconds: float, out_bytes: int = 2,
            channel: bool = False) -> float:
    return gemm_bytes_all(m, n, k, out_bytes, channel) / seconds / 1e9


def roofline_time_s(m: int, n: int, k: int, out_bytes: int = 2, channel: bool = False) -> float:
    """Lower bound on the GEMM time on MI355X: max(bytes / HBM peak, flops / FP8 peak)."""
    return max(gemm_bytes_all(m, n, k, out_bytes, channel) / (HBM_PEAK_GBS * 1e9),
               gemm_flops(m, n, k) / (FP8_PEAK_TFLOPS * 1e12))


def bound(m: int, n: int, k: int, out_bytes: int = 2, channel: bool = False) -> str:
    t_mem = gemm_bytes_all(m, n, k, out_bytes, channel) / (HBM_PEAK_GBS * 1e9)
    t_mma = gemm_flops(m, n, k) / (FP8_PEAK_TFLOPS * 1e12)
    return "hbm" if t_mem >= t_mma else "mfma"


def moe_gemm_bytes(T: int, topk: int, active: int, N: int, K: int, out_bytes: int = 2) -> float:
    """Grouped (MoE) GEMM: each active expert's weight codes and block scales once, each
    token's codes and group scales once, one output row per (token, expert) pair."""
    return float(active * (N * K + 4 * (N // 128) * (K // 128)) + T * (K + 4 * (K // 128))
                 + out_bytes * T * topk * N)
