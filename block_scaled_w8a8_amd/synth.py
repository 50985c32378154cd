"""Seeded synthetic inputs shared by the tests, the on-device sweep and bench.py.

This module holds no step of the method: it only draws random numbers with
torch's CPU generator. The distributions stand in for the pages' workload (randn bf16
activations and weights of DeepSeek-V3 projection shapes, block GEMM benchmark page §4.1):
  W  = randn(N, K) * 0.02                       fp32, generator seed
  cols = randperm(K)[:round(0.02 K)]            generator seed + 1 (outlier channels)
  X  = randn(M_max, K); X[:, cols] *= 20; bf16  generator seed + 2
Each smaller M takes the first M rows of the M_max draw, so inputs nest across M.
MoE routing (the expert dimension of the config page's MoE tables, §5): each token picks
topk distinct experts of E, uniformly: the topk largest of E uniform draws (generator
seed + 3); expert weights are E independent weight draws (seed + 1000 + e).
GEMM inputs drawn directly, for cases too large to quantize on the host (a GEMM takes any
codes and positive scales): codes uniform over the code points (int8 -127..127; fp8 every
byte but the two NaN encodings 0x7F and 0xFF), scales 2^u with u uniform in [-10, -4).
"""
from __future__ import annotations

import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def weights(N: int, K: int, seed: int = 0) -> torch.Tensor:
    """fp32 [N, K] ~ N(0, 0.02^2)."""
    return torch.randn((N, K), generator=_gen(seed), dtype=torch.float32) * 0.02


def outlier_columns(K: int, seed: int = 0, frac: float = 0.02) -> torch.Tensor:
    n = int(round(frac * K))
    return torch.randperm(K, generator=_gen(seed + 1))[:n]


def activations(M: int, K: int, seed: int = 0, m_max: int | None = None) -> torch.Tensor:
    """bf16 [M, K] ~ N(0, 1) with 2% outlier columns scaled x20 (rows 0..M-1 of an
    m_max-row draw)."""
    m_max = max(M, m_max or M)
    x = torch.randn((m_max, K), generator=_gen(seed + 2), dtype=torch.float32)
    cols = outlier_columns(K, seed)
    x[:, cols] *= 20.0
    return x[:M].to(torch.bfloat16).contiguous()


def bf16_bits(x: torch.Tensor):
    """The uint16 bit patterns of a bf16 tensor, as a numpy array (for the CPU oracle)."""
    return x.contiguous().view(torch.int16).numpy().view("uint16")


def routing(T: int, E: int, topk: int, seed: int = 0, t_max: int | None = None) -> torch.Tensor:
    """int32 [T, topk]: distinct experts per token, uniform over the E experts (rows 0..T-1
    of a t_max-row draw, so routing nests across T like the activations)."""
    t_max = max(T, t_max or T)
    u = torch.rand((t_max, E), generator=_gen(seed + 3), dtype=torch.float32)
    return u.topk(topk, dim=1).indices[:T].to(torch.int32).contiguous()


def expert_weights(E: int, N: int, K: int, seed: int = 0) -> torch.Tensor:
    """fp32 [E, N, K]: one weights() draw per expert."""
    return torch.stack([weights(N, K, seed=seed + 1000 + e) for e in range(E)])


def expert_weight_on(device, e: int, N: int, K: int, seed: int = 0) -> torch.Tensor:
    """fp32 [N, K] weights of expert e drawn on `device` with its own seeded generator (the
    full expert stack of a large MoE layer is too big to draw on the host); the same call
    gives the same values again, so a checker can re-draw any expert it samples."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 1000 + int(e))
    return torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * 0.02


def codes(rows: int, cols: int, int8: bool = False, seed: int = 0, device="cpu") -> torch.Tensor:
    """[rows, cols] uniform random codes drawn on `device` (int8, or uint8 e4m3fn bytes)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    if int8:
        return torch.randint(-127, 128, (rows, cols), generator=g, device=device, dtype=torch.int8)
    r = torch.randint(0, 254, (rows, cols), generator=g, device=device, dtype=torch.uint8)
    return r + (r >= 0x7F).to(torch.uint8)      # 0..0xFE without 0x7F


def scales(rows: int, cols: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [rows, cols] = 2^u, u uniform in [-10, -4), drawn on `device`."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    u = torch.rand((rows, cols), generator=g, device=device, dtype=torch.float32)
    return torch.exp2(-10.0 + 6.0 * u)
