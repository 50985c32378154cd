"""CPU oracle for the block-scaled W8A8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. It shares no code with ``block_scaled_w8a8_amd`` (the HIP path)
and imports nothing from it; the HIP path never imports this package.

The arithmetic lives in ``oracle.c`` (plain C, fp64/int32-exact block sums, fp32
accumulation with contraction off). This module only marshals numpy arrays through ctypes
and builds the shared library with gcc. Metrics (``calc_diff`` and friends) and the
nearest-M rule are in ``metrics.py`` and ``select.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_DIR = os.path.join(HERE, "_build")
# ORACLE_LIBRARY names another build of oracle.c (the sanitizer build below); by default the
# gcc build.
LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(BUILD_DIR, "liboracle.so")
ASAN_LIB_PATH = os.path.join(BUILD_DIR, "liboracle_asan.so")

FP8 = 0
INT8 = 1
SCALE_FP32 = 0
SCALE_UE8M0 = 1
DEFAULT_EPS = np.float32(1e-10)


def build(force: bool = True) -> str:
    """Compile oracle.c into a shared library with gcc (-O2, OpenMP, no fp contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp,
           os.path.join(HERE, "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_sanitized(clang: str = "/opt/rocm/llvm/bin/clang") -> str:
    """oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer, built with the clang
    whose sanitizer runtime the process preloads (the same runtime as the library's
    sanitizer build). Same arithmetic flags as build(); OpenMP from clang's libomp."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = ASAN_LIB_PATH + ".tmp"
    cmd = [clang, "-std=c11", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared-libsan",
           "-o", tmp, os.path.join(HERE, "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, ASAN_LIB_PATH)
    return ASAN_LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [f32]
        L.orc_int8_encode.restype = ctypes.c_int8
        L.orc_int8_encode.argtypes = [f32]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [f32]
        L.orc_bf16_to_f32.restype = f32
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        for nm in ("orc_e4m3_encode_array", "orc_int8_encode_array", "orc_f32_to_bf16_array"):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = [p, i64, p]
        L.orc_quant_groups.restype = None
        L.orc_quant_groups.argtypes = [p, i64, i64, i64, i32, p, p, f32, i32]
        L.orc_quant_blocks.restype = None
        L.orc_quant_blocks.argtypes = [p, i64, i64, i64, i64, i32, p, p, f32, i32]
        L.orc_block_gemm.restype = None
        L.orc_block_gemm.argtypes = [p, p, p, p, i64, i64, i64, i32, p, p]
        L.orc_block_gemm_sampled.restype = None
        L.orc_block_gemm_sampled.argtypes = [p, p, p, p, i64, i64, i64, i32, p, p, i64, p]
        L.orc_pack_scales_ue8m0.restype = None
        L.orc_pack_scales_ue8m0.argtypes = [p, i64, i64, p, i64]
        L.orc_moe_align.restype = None
        L.orc_moe_align.argtypes = [p, i64, i64, p, p]
        L.orc_moe_gemm.restype = None
        L.orc_moe_gemm.argtypes = [p, p, p, i64, i64, p, p, i64, i64, i64, i32, p]
        L.orc_moe_gemm_sampled.restype = None
        L.orc_moe_gemm_sampled.argtypes = [p, p, p, i64, p, p, i64, i64, i32, p, p, i64, p]
        L.orc_channel_gemm.restype = None
        L.orc_channel_gemm.argtypes = [p, p, p, p, i64, i64, i64, i32, p, p]
        L.orc_channel_gemm_sampled.restype = None
        L.orc_channel_gemm_sampled.argtypes = [p, p, p, p, i64, i64, i64, i32, p, p, i64, p]
        L.orc_block_partials_i32.restype = None
        L.orc_block_partials_i32.argtypes = [p, p, i64, i64, i64, p]
        L.orc_dequant_gemm_f64.restype = None
        L.orc_dequant_gemm_f64.argtypes = [p, p, p, p, i64, i64, i64, i32, p]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _code_dtype(qtype: int):
    return np.uint8 if qtype == FP8 else np.int8


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ------------------------------------------------------------------ scalar codecs

def e4m3_decode(code: int) -> float:
    return float(lib().orc_e4m3_decode(int(code)))


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(np.float32(x))))


def int8_encode(x: float) -> int:
    return int(lib().orc_int8_encode(float(np.float32(x))))


def f32_to_bf16_bits(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(np.float32(x))))


def f32_to_bf16_bits_array(x: np.ndarray) -> np.ndarray:
    """Elementwise fp32 -> bf16 RNE bits."""
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    lib().orc_f32_to_bf16_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


def int8_encode_array(x: np.ndarray) -> np.ndarray:
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(flat.shape, dtype=np.int8)
    lib().orc_int8_encode_array(_ptr(flat), flat.size, _ptr(out))
    return out.reshape(np.shape(x))


# ------------------------------------------------------------------ quantizers

def quant_groups(x_bf16_bits: np.ndarray, group: int = 128, qtype: int = FP8,
                 eps: float = DEFAULT_EPS, scale_fmt: int = SCALE_FP32):
    """bf16 activations (uint16 bit patterns, [M, K]) -> (codes [M, K], scales [M, K/group]).
    scale_fmt SCALE_UE8M0: scales rounded up to a power of two (block GEMM benchmark page
    §4.1, use_ue8m0)."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    assert K % group == 0
    q = np.empty((M, K), dtype=_code_dtype(qtype))
    s = np.empty((M, K // group), dtype=np.float32)
    lib().orc_quant_groups(_ptr(x), M, K, group, qtype, _ptr(q), _ptr(s), float(eps),
                           int(scale_fmt))
    return q, s


def quant_blocks(w: np.ndarray, block=(128, 128), qtype: int = FP8, eps: float = DEFAULT_EPS,
                 scale_fmt: int = SCALE_FP32):
    """fp32 weights [N, K] -> (codes [N, K], scales [N/bn, K/bk]); scale_fmt as above."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    bn, bk = block
    assert N % bn == 0 and K % bk == 0
    q = np.empty((N, K), dtype=_code_dtype(qtype))
    s = np.empty((N // bn, K // bk), dtype=np.float32)
    lib().orc_quant_blocks(_ptr(w), N, K, bn, bk, qtype, _ptr(q), _ptr(s), float(eps),
                           int(scale_fmt))
    return q, s


# ------------------------------------------------------------------ GEMM

def pack_scales_ue8m0(s: np.ndarray, ld: int | None = None) -> np.ndarray:
    """UE8M0 scales [M, G] -> packed words [ceil(G/4), ld] (uint32), ld >= round_up(M, 4)
    (default round_up(M, 4)): the quantizer's packed scale output of the per-token-group
    kernel page (output_s_packed)."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    M, G = s.shape
    Mp = (M + 3) // 4 * 4
    ld = Mp if ld is None else ld
    assert ld >= Mp
    words = np.zeros(((G + 3) // 4, ld), dtype=np.uint32)
    lib().orc_pack_scales_ue8m0(_ptr(s), M, G, _ptr(words), ld)
    return words


def pack16(w: np.ndarray) -> np.ndarray:
    """The packed 16-row fragment layout of weight codes (a byte permutation; the layout is
    this library's own HBM format for the weights, not something the pages define, so the
    definition written out is the oracle). For every 16-row group f and 128-wide K block kb
    there are 2048 consecutive bytes at (f*(K/128) + kb)*2048; byte h*1024 + 16*l + b of
    them (h in {0,1}, l in [0,64), b in [0,16)) is w[16f + l%16, 128kb + 64h + 16*(l//16) + b].
    Works on any dtype (tests pack index arrays to check it is a permutation)."""
    N, K = w.shape
    assert N % 16 == 0 and K % 128 == 0
    # axes (f, r, kb, h, g, b): row 16f + r, column 128kb + 64h + 16g + b
    x = np.asarray(w).reshape(N // 16, 16, K // 128, 2, 4, 16)
    # fragment-major, then half, then lane l = 16g + r, then byte
    return np.ascontiguousarray(x.transpose(0, 2, 3, 4, 1, 5)).reshape(N, K)


def _gemm_args(qa, sa, qw, sw, qtype):
    qa = np.ascontiguousarray(qa, dtype=_code_dtype(qtype))
    qw = np.ascontiguousarray(qw, dtype=_code_dtype(qtype))
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and K % 128 == 0 and N % 128 == 0
    assert sa.shape == (M, K // 128) and sw.shape == (N // 128, K // 128)
    return qa, sa, qw, sw, M, N, K


def block_gemm(qa, sa, qw, sw, qtype: int = FP8):
    """Returns (c32 [M, N] float32, c16 [M, N] uint16 bf16 bits)."""
    qa, sa, qw, sw, M, N, K = _gemm_args(qa, sa, qw, sw, qtype)
    c32 = np.empty((M, N), dtype=np.float32)
    c16 = np.empty((M, N), dtype=np.uint16)
    lib().orc_block_gemm(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, qtype,
                         _ptr(c32), _ptr(c16))
    return c32, c16


def block_gemm_sampled(qa, sa, qw, sw, ms, ns, qtype: int = FP8):
    qa, sa, qw, sw, M, N, K = _gemm_args(qa, sa, qw, sw, qtype)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    assert ms.shape == ns.shape and ms.ndim == 1
    assert (ms >= 0).all() and (ms < M).all() and (ns >= 0).all() and (ns < N).all()
    out = np.empty(ms.shape, dtype=np.float32)
    lib().orc_block_gemm_sampled(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, qtype,
                                 _ptr(ms), _ptr(ns), ms.size, _ptr(out))
    return out


def _channel_args(qa, sa, qw, sw, qtype):
    qa = np.ascontiguousarray(qa, dtype=_code_dtype(qtype))
    qw = np.ascontiguousarray(qw, dtype=_code_dtype(qtype))
    sa = np.ascontiguousarray(np.asarray(sa, dtype=np.float32).reshape(-1))
    sw = np.ascontiguousarray(np.asarray(sw, dtype=np.float32).reshape(-1))
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and sa.shape == (M,) and sw.shape == (N,)
    return qa, sa, qw, sw, M, N, K


def channel_gemm(qa, sa, qw, sw, qtype: int = FP8):
    """Per-token x per-channel GEMM: sa [M] (or [M, 1]), sw [N] (or [N, 1]).
    Returns (c32 [M, N] float32, c16 [M, N] uint16 bf16 bits)."""
    qa, sa, qw, sw, M, N, K = _channel_args(qa, sa, qw, sw, qtype)
    c32 = np.empty((M, N), dtype=np.float32)
    c16 = np.empty((M, N), dtype=np.uint16)
    lib().orc_channel_gemm(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, qtype,
                           _ptr(c32), _ptr(c16))
    return c32, c16


def channel_gemm_sampled(qa, sa, qw, sw, ms, ns, qtype: int = FP8):
    qa, sa, qw, sw, M, N, K = _channel_args(qa, sa, qw, sw, qtype)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    assert ms.shape == ns.shape and ms.ndim == 1
    assert (ms >= 0).all() and (ms < M).all() and (ns >= 0).all() and (ns < N).all()
    out = np.empty(ms.shape, dtype=np.float32)
    lib().orc_channel_gemm_sampled(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, qtype,
                                   _ptr(ms), _ptr(ns), ms.size, _ptr(out))
    return out


def moe_align(topk_ids, E: int):
    """topk_ids int [T, topk] -> (offsets int32 [E+1], sorted int32 [T*topk]): pair ids
    q = t*topk + j grouped by expert, ascending within an expert."""
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32).reshape(-1)
    assert ids.size == 0 or (ids.min() >= 0 and ids.max() < E)
    offsets = np.empty(E + 1, dtype=np.int32)
    srt = np.empty(ids.size, dtype=np.int32)
    lib().orc_moe_align(_ptr(ids), ids.size, E, _ptr(offsets), _ptr(srt))
    return offsets, srt


def _moe_args(qa, sa, topk_ids, qw, sw, qtype):
    qa = np.ascontiguousarray(qa, dtype=_code_dtype(qtype))
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    qw = np.ascontiguousarray(qw, dtype=_code_dtype(qtype))
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    T, K = qa.shape
    E, N, K2 = qw.shape
    assert K == K2 and ids.shape[0] == T and sa.shape == (T, K // 128)
    assert sw.shape == (E, N // 128, K // 128) and (ids.size == 0 or ids.max() < E)
    return qa, sa, ids, qw, sw, T, ids.shape[1], E, N, K


def moe_gemm(qa, sa, topk_ids, qw, sw, qtype: int = FP8):
    """MoE grouped block GEMM: qa [T, K], sa [T, K/128], topk_ids [T, topk], qw [E, N, K],
    sw [E, N/128, K/128] -> c32 [T*topk, N] in pair order."""
    qa, sa, ids, qw, sw, T, topk, E, N, K = _moe_args(qa, sa, topk_ids, qw, sw, qtype)
    c32 = np.empty((T * topk, N), dtype=np.float32)
    lib().orc_moe_gemm(_ptr(qa), _ptr(sa), _ptr(ids), T, topk, _ptr(qw), _ptr(sw), E, N, K,
                       qtype, _ptr(c32))
    return c32


def moe_gemm_sampled(qa, sa, topk_ids, qw, sw, qs, ns, qtype: int = FP8):
    qa, sa, ids, qw, sw, T, topk, E, N, K = _moe_args(qa, sa, topk_ids, qw, sw, qtype)
    qs = np.ascontiguousarray(qs, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    assert (qs >= 0).all() and (qs < T * topk).all() and (ns >= 0).all() and (ns < N).all()
    out = np.empty(qs.shape, dtype=np.float32)
    lib().orc_moe_gemm_sampled(_ptr(qa), _ptr(sa), _ptr(ids), topk, _ptr(qw), _ptr(sw), N, K,
                               qtype, _ptr(qs), _ptr(ns), qs.size, _ptr(out))
    return out


def block_partials_i32(qa, qw):
    qa = np.ascontiguousarray(qa, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    M, K = qa.shape
    N, _ = qw.shape
    out = np.empty((K // 128, M, N), dtype=np.int32)
    lib().orc_block_partials_i32(_ptr(qa), _ptr(qw), M, N, K, _ptr(out))
    return out


def dequant_gemm_f64(qa, sa, qw, sw, qtype: int = FP8):
    qa, sa, qw, sw, M, N, K = _gemm_args(qa, sa, qw, sw, qtype)
    d = np.empty((M, N), dtype=np.float64)
    lib().orc_dequant_gemm_f64(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, qtype, _ptr(d))
    return d
