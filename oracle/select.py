"""Nearest-M bucket rule -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The config-mechanism page ("vLLM 量化 Kernel 配置机制 ...", §4.2) picks, for a runtime M,
the tuned entry whose key is closest to M; Python's min() over the ascending keys keeps
the first minimal key, so a tie goes to the smaller bucket. M beyond the grid maps to the
nearest end of the grid.
"""
from __future__ import annotations

M_GRID = (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512, 1024, 1536, 2048, 3072, 4096)


def nearest_bucket(M: int, keys=M_GRID) -> int:
    best = None
    for k in sorted(keys):
        if best is None or abs(k - M) < abs(best - M):
            best = k
    return best
