"""ctypes binding of libbfq (include/bfq.h): the same entry-point names, argument marshalling
only. Every step of the computation runs in the HIP kernels of libbfq.so; PyTorch supplies
device memory (tensor.data_ptr()) and the current HIP stream. There is no fallback: if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import warnings

HERE = os.path.dirname(os.path.abspath(__file__))
# BFQ_LIBRARY names another build of the same library (for example one whose host code is
# built with sanitizers); by default the in-tree libbfq.so.
LIB_PATH = os.environ.get("BFQ_LIBRARY") or os.path.join(HERE, "libbfq.so")

# status codes (bfq_status)
BFQ_OK = 0
BFQ_WARN_DEFAULT_TILE = 1
BFQ_ERR_NULL = -1
BFQ_ERR_SHAPE = -2
BFQ_ERR_DTYPE = -3
BFQ_ERR_ALIGN = -4
BFQ_ERR_WORKSPACE = -5
BFQ_ERR_TILE = -6
BFQ_ERR_TABLE = -7
BFQ_ERR_HIP = -8
BFQ_ERR_ARG = -9

# dtypes (bfq_dtype)
BFQ_BF16, BFQ_FP16, BFQ_FP32, BFQ_E4M3FN, BFQ_INT8, BFQ_INT32 = range(6)
# scale layouts (bfq_scale_layout)
BFQ_SCALES_ROW_MAJOR = 0
BFQ_SCALES_COL_MAJOR = 1
BFQ_SCALES_PACKED_UE8M0 = 2   # uint32 words of four E8M0 codes (UE8M0 scales only)
# weight-code layouts (bfq_weight_layout)
BFQ_W_ROW_MAJOR = 0
BFQ_W_PACKED16 = 1
# scale formats (bfq_scale_format)
BFQ_SCALE_FP32 = 0
BFQ_SCALE_UE8M0 = 1

DEFAULT_EPS = 1e-10
BLOCK_SHAPE = (128, 128)
# Maximum K of the per-token x per-channel format (block_shape (1, K)).
CHANNEL_MAX_K = 32768


def channel_block_shape(K: int):
    """block_shape of the per-token x per-channel format (one scale per token and per output
    channel; Helion linear-backend page, scope section)."""
    return (1, int(K))

EXPORTED = (
    "bfq_quant_tokens", "bfq_quant_weight_blocks", "bfq_pack_weights", "bfq_select_tile",
    "bfq_gemm_workspace_bytes", "bfq_block_gemm", "bfq_load_tile_table",
    "bfq_num_tile_candidates", "bfq_get_tile_candidate", "bfq_status_string",
    "bfq_last_error", "bfq_debug_block_partials_i32", "bfq_debug_encode",
    "bfq_set_batch_invariant", "bfq_get_batch_invariant",
    "bfq_moe_align_workspace_bytes", "bfq_moe_align", "bfq_moe_select_tile",
    "bfq_moe_gemm_workspace_bytes", "bfq_moe_block_gemm", "bfq_moe_num_tile_candidates",
    "bfq_moe_get_tile_candidate", "bfq_block_gemm_noalloc", "bfq_noalloc_scratch_bytes",
    "bfq_probe_mfma_peak", "bfq_probe_mfma_flops",
)


class bfq_tile(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("bk", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("sched", ctypes.c_int32), ("raster", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    FIELDS = ("variant", "bm", "bn", "bk", "split_k", "waves_m", "waves_n", "stages", "group_m",
              "sched", "raster")

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f in self.FIELDS}

    @classmethod
    def from_dict(cls, d: dict) -> "bfq_tile":
        t = cls()
        t.bk = 128
        t.split_k = 1
        t.waves_m = 1
        t.stages = 2
        t.group_m = 1
        for k, v in d.items():
            if k in cls.FIELDS:
                setattr(t, k, int(v))
        return t


class BfqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {last_error()}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libbfq.so not found at {LIB_PATH}; build it with "
            "`python -m block_scaled_w8a8_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                            ctypes.c_size_t)
    tp = ctypes.POINTER(bfq_tile)
    bs = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "bfq_quant_tokens": (i32, [p, i64, i64, i32, i32, p, p, i32, i64, f32, i32, p]),
        "bfq_quant_weight_blocks": (i32, [p, i64, i64, bs, i32, p, p, f32, i32, p]),
        "bfq_pack_weights": (i32, [p, i64, i64, i32, p, p]),
        "bfq_select_tile": (i32, [i64, i64, i64, bs, i32, i32, i32, i32, tp]),
        "bfq_gemm_workspace_bytes": (sz, [i64, i64, i64, tp]),
        "bfq_block_gemm": (i32, [p, p, i32, i64, p, p, i32, i32, p, i64, i64, i64, bs, i32, i32,
                                 tp, p, sz, p]),
        "bfq_load_tile_table": (i32, [ctypes.c_char_p]),
        "bfq_num_tile_candidates": (i32, [bs, i32, i32, i32]),
        "bfq_get_tile_candidate": (i32, [bs, i32, i32, i32, i32, tp]),
        "bfq_status_string": (ctypes.c_char_p, [i32]),
        "bfq_last_error": (ctypes.c_char_p, []),
        "bfq_debug_block_partials_i32": (i32, [p, p, p, i64, i64, i64, p]),
        "bfq_debug_encode": (i32, [p, i64, i32, p, p]),
        "bfq_set_batch_invariant": (None, [i32]),
        "bfq_moe_align_workspace_bytes": (sz, [i64, i32, i32]),
        "bfq_moe_align": (i32, [p, i64, i32, i32, p, p, p, sz, p]),
        "bfq_moe_select_tile": (i32, [i64, i32, i32, i64, i64, bs, i32, i32, i32, i32, tp]),
        "bfq_moe_gemm_workspace_bytes": (sz, [i64, i32, i64, tp]),
        "bfq_moe_block_gemm": (i32, [p, p, i32, i64, p, p, i32, p, p, i32, i32, p, i64, i64, i64,
                                     i32, bs, i32, i32, tp, p, sz, p]),
        "bfq_moe_num_tile_candidates": (i32, [i32, i32]),
        "bfq_moe_get_tile_candidate": (i32, [i32, i32, i32, tp]),
        "bfq_get_batch_invariant": (i32, []),
        "bfq_block_gemm_noalloc": (i32, [p, p, i32, i64, p, p, i32, i32, p, i64, i64, i64, bs,
                                         i32, i32, tp, p]),
        "bfq_noalloc_scratch_bytes": (sz, []),
        "bfq_probe_mfma_peak": (i32, [i64, i64, p, p]),
        "bfq_probe_mfma_flops": (ctypes.c_double, [i64, i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load()

_warned: set = set()


def status_string(s: int) -> str:
    return lib.bfq_status_string(int(s)).decode()


def last_error() -> str:
    return lib.bfq_last_error().decode()


def _check(status: int, where: str, warn_key=None) -> int:
    if status < 0:
        raise BfqError(status, where)
    if status > 0 and warn_key not in _warned:
        _warned.add(warn_key)
        warnings.warn(f"{where}: {status_string(status)} (no tuned tile for {warn_key}; "
                      "using the default tile)", RuntimeWarning, stacklevel=3)
    return status


def _block_shape(block_shape=BLOCK_SHAPE):
    return (ctypes.c_int32 * 2)(*block_shape)


def _ptr(t) -> int:
    """Device address of a tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ------------------------------------------------------------------ argument checks
# The kernels take raw device addresses and assume the layouts stated in include/bfq.h (rows
# of codes and outputs packed at stride K or N, scales at the stated leading dimension). The
# wrappers below check every tensor against those assumptions before the C call, so that a
# host tensor, a strided view or a buffer of the wrong size raises here instead of handing a
# kernel an address it would read or write past. Order: type, dtype, shape, strides, device
# (a tensor that passes all but the device check is a host tensor). Plain int addresses are
# passed through unchecked: the caller vouches for them.

class BfqArgumentError(ValueError):
    """A tensor argument does not match what the kernel will read or write."""


U8_CODES = ("uint8", "float8_e4m3fn")


def _dt(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _tensor(t, name, dtypes):
    if isinstance(t, int):
        return False
    import torch
    if not isinstance(t, torch.Tensor):
        raise BfqArgumentError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if _dt(t) not in dtypes:
        raise BfqArgumentError(f"{name} has dtype {_dt(t)}; expected one of {', '.join(dtypes)}")
    return True


def _devices(**tensors):
    """Last check of a wrapper: every tensor argument is on the current GPU."""
    for name, t in tensors.items():
        if t is not None and not isinstance(t, int):
            _on_device(t, name)


def _on_device(t, name):
    import torch
    if not t.is_cuda:
        raise BfqArgumentError(f"{name} is on device {t.device}; the kernels need a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise BfqArgumentError(f"{name} is on {t.device}, not the current device "
                               f"cuda:{torch.cuda.current_device()}")


def _rows(t, name, dtypes, rows, cols):
    """A [rows, cols] matrix whose rows are packed at stride cols (what the kernels index)."""
    if not _tensor(t, name, dtypes):
        return
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise BfqArgumentError(f"{name} has shape {tuple(t.shape)}; expected ({rows}, {cols})")
    if rows > 0 and cols > 0 and (t.stride(1) != 1 or (rows > 1 and t.stride(0) != cols)):
        raise BfqArgumentError(f"{name} has strides {t.stride()}; its rows must be contiguous "
                               f"at stride {cols} (call .contiguous())")


def _flat(t, name, dtypes, numel, exact=True):
    """A contiguous buffer of exactly (or at least) numel elements, any shape."""
    if not _tensor(t, name, dtypes):
        return
    if (t.numel() != numel) if exact else (t.numel() < numel):
        raise BfqArgumentError(f"{name} holds {t.numel()} elements; expected "
                               f"{'' if exact else 'at least '}{numel}")
    if not t.is_contiguous():
        raise BfqArgumentError(f"{name} must be contiguous")


def _scales(t, name, layout, ld, m, groups, write):
    """Activation scales in `layout` with leading dimension ld over m tokens and `groups`
    scales per token: the 2-D view must cover every element the kernel touches, at stride
    (ld, 1). Packed words: int32, ceil(groups/4) word rows of ld words, ld >= m rounded up to
    4 when the quantizer writes them (>= m when the GEMM reads them)."""
    if layout == BFQ_SCALES_PACKED_UE8M0:
        if not _tensor(t, name, ("int32", "uint32")):
            return
        need = ((groups + 3) // 4, (m + 3) // 4 * 4 if write else m)
    else:
        if not _tensor(t, name, ("float32",)):
            return
        need = (m, groups) if layout == BFQ_SCALES_ROW_MAJOR else (groups, m)
    if t.dim() != 2:
        raise BfqArgumentError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[0] < need[0] or t.shape[1] < need[1]:
        raise BfqArgumentError(f"{name} has shape {tuple(t.shape)}; the layout needs at least "
                               f"{need}")
    if t.shape[0] > 1 and t.stride(0) != ld:
        raise BfqArgumentError(f"{name} has row stride {t.stride(0)} but scale_ld is {ld}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise BfqArgumentError(f"{name} must have unit stride along its second dimension")


def _workspace(t, nbytes):
    if t is None or isinstance(t, int):
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise BfqArgumentError("workspace must be a torch.Tensor")
    if t.numel() * t.element_size() < nbytes or not t.is_contiguous():
        raise BfqArgumentError(f"workspace holds {t.numel() * t.element_size()} bytes "
                               f"(contiguous: {t.is_contiguous()}); {nbytes} are declared")


CODE_DTYPES = U8_CODES + ("int8",)
OUT_DTYPES = ("bfloat16", "float16", "float32")


def _shape2(t, name):
    if not hasattr(t, "dim") or t.dim() != 2:
        raise BfqArgumentError(f"{name} must be a 2-D tensor")
    return int(t.shape[0]), int(t.shape[1])


def _same_codes(a, w):
    """Token and weight codes must be the same code type (e4m3fn bytes or int8)."""
    if isinstance(a, int) or isinstance(w, int):
        return
    if (_dt(a) == "int8") != (_dt(w) == "int8"):
        raise BfqArgumentError(f"a_q ({_dt(a)}) and w_q ({_dt(w)}) hold different code types")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _qdtype(t) -> int:
    import torch
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return BFQ_E4M3FN
    if t.dtype == torch.int8:
        return BFQ_INT8
    raise BfqArgumentError(f"code tensor dtype {t.dtype} is neither e4m3fn/uint8 nor int8")


def _odtype(t) -> int:
    import torch
    return {torch.bfloat16: BFQ_BF16, torch.float16: BFQ_FP16, torch.float32: BFQ_FP32}[t.dtype]


# ----------------------------------------------------------------------- entry points

def bfq_quant_tokens(x, q, scales, layout=BFQ_SCALES_ROW_MAJOR, scale_ld=None,
                     eps=DEFAULT_EPS, group_size=128, stream=None,
                     scale_fmt=BFQ_SCALE_FP32) -> int:
    """x: bf16 [M, K]; q: uint8/float8_e4m3fn (e4m3fn codes) or int8 [M, K];
    scales: fp32, [M, ld] (row-major) or [K/group_size, ld] (column-major). group_size 128,
    or K for one scale per token."""
    M, K = _shape2(x, "x")
    if scale_ld is None:
        scale_ld = scales.stride(0)
    _rows(x, "x", ("bfloat16",), M, K)
    _rows(q, "q", CODE_DTYPES, M, K)
    if group_size > 0 and K % group_size == 0:
        _scales(scales, "scales", layout, scale_ld, M, K // group_size, write=True)
    _devices(x=x, q=q, scales=scales)
    st = lib.bfq_quant_tokens(_ptr(x), M, K, group_size, _qdtype(q), _ptr(q), _ptr(scales),
                              layout, scale_ld, eps, scale_fmt, _stream(stream))
    return _check(st, "bfq_quant_tokens")


def bfq_quant_weight_blocks(w, q, scales, eps=DEFAULT_EPS, block_shape=BLOCK_SHAPE,
                            stream=None, scale_fmt=BFQ_SCALE_FP32) -> int:
    """w: fp32 [N, K]; q: codes [N, K]; scales: fp32 [N/128, K/128], or [N] (any shape of N
    contiguous floats) with block_shape (1, K)."""
    N, K = _shape2(w, "w")
    _rows(w, "w", ("float32",), N, K)
    _rows(q, "q", CODE_DTYPES, N, K)
    per_channel = tuple(block_shape)[0] == 1
    _flat(scales, "scales", ("float32",), N if per_channel else (N // 128) * (K // 128))
    _devices(w=w, q=q, scales=scales)
    st = lib.bfq_quant_weight_blocks(_ptr(w), N, K, _block_shape(block_shape), _qdtype(q),
                                     _ptr(q), _ptr(scales), eps, scale_fmt, _stream(stream))
    return _check(st, "bfq_quant_weight_blocks")


def bfq_pack_weights(w_q, w_packed, stream=None) -> int:
    """w_q: row-major codes [N, K]; w_packed: a separate N*K-byte buffer (any shape with that
    many bytes, e.g. [N, K] uint8) that receives the BFQ_W_PACKED16 layout."""
    N, K = _shape2(w_q, "w_q")
    _rows(w_q, "w_q", CODE_DTYPES, N, K)
    if _tensor(w_packed, "w_packed", CODE_DTYPES):
        if w_packed.numel() * w_packed.element_size() != N * K or not w_packed.is_contiguous():
            raise BfqArgumentError("w_packed must be a contiguous buffer of exactly N*K bytes")
    _devices(w_q=w_q, w_packed=w_packed)
    st = lib.bfq_pack_weights(_ptr(w_q), N, K, _qdtype(w_q), _ptr(w_packed), _stream(stream))
    return _check(st, "bfq_pack_weights")


def bfq_select_tile(M, N, K, in_dtype=BFQ_E4M3FN, out_dtype=BFQ_BF16,
                    block_shape=BLOCK_SHAPE, w_layout=BFQ_W_ROW_MAJOR, scale_fmt=BFQ_SCALE_FP32):
    """Returns (status, bfq_tile)."""
    t = bfq_tile()
    st = lib.bfq_select_tile(M, N, K, _block_shape(block_shape), in_dtype, out_dtype,
                             w_layout, scale_fmt, ctypes.byref(t))
    if st < 0:
        raise BfqError(st, "bfq_select_tile")
    return st, t


def bfq_gemm_workspace_bytes(M, N, K, tile=None) -> int:
    return int(lib.bfq_gemm_workspace_bytes(M, N, K, ctypes.byref(tile) if tile else None))


def bfq_block_gemm(a_q, a_scales, w_q, w_scales, out, a_layout=BFQ_SCALES_ROW_MAJOR,
                   a_scale_ld=None, tile=None, workspace=None, workspace_bytes=None,
                   block_shape=BLOCK_SHAPE, stream=None, w_layout=BFQ_W_ROW_MAJOR,
                   scale_fmt=BFQ_SCALE_FP32) -> int:
    """a_q [M, K] codes, w_q [N, K] codes in w_layout (row-major, or packed by
    bfq_pack_weights and still shaped [N, K]), a_scales per layout, w_scales [N/128, K/128],
    out [M, N] (bf16 / fp16 / fp32). scale_fmt BFQ_SCALE_UE8M0 declares every scale a power
    of two. block_shape (1, K): per-token a_scales ([M, 1] or [1, M]) and per-channel
    w_scales [N]. Returns the status (>= 0)."""
    M, K = _shape2(a_q, "a_q")
    N = _shape2(w_q, "w_q")[0]
    if a_scale_ld is None:
        a_scale_ld = a_scales.stride(0)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _rows(a_q, "a_q", CODE_DTYPES, M, K)
    _rows(w_q, "w_q", CODE_DTYPES, N, K)
    _same_codes(a_q, w_q)
    per_channel = tuple(block_shape)[0] == 1
    _scales(a_scales, "a_scales", a_layout, a_scale_ld, M, 1 if per_channel else K // 128,
            write=False)
    _flat(w_scales, "w_scales", ("float32",), N if per_channel else (N // 128) * (K // 128))
    _rows(out, "out", OUT_DTYPES, M, N)
    _workspace(workspace, workspace_bytes)
    _devices(a_q=a_q, a_scales=a_scales, w_q=w_q, w_scales=w_scales, out=out, workspace=workspace)
    st = lib.bfq_block_gemm(_ptr(a_q), _ptr(a_scales), a_layout, a_scale_ld, _ptr(w_q),
                            _ptr(w_scales), w_layout, scale_fmt, _ptr(out), M, N, K,
                            _block_shape(block_shape),
                            _qdtype(a_q), _odtype(out), ctypes.byref(tile) if tile else None,
                            _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(st, "bfq_block_gemm", warn_key=(N, K))


def bfq_block_gemm_noalloc(a_q, a_scales, w_q, w_scales, out, a_layout=BFQ_SCALES_ROW_MAJOR,
                           a_scale_ld=None, tile=None, block_shape=BLOCK_SHAPE, stream=None,
                           w_layout=BFQ_W_ROW_MAJOR, scale_fmt=BFQ_SCALE_FP32) -> int:
    """bfq_block_gemm without a workspace argument: split-K partials and stream-K slots use the
    library's static device buffer (bfq_noalloc_scratch_bytes()). No allocation anywhere on
    this path; calls that overlap on one GPU race."""
    M, K = _shape2(a_q, "a_q")
    N = _shape2(w_q, "w_q")[0]
    if a_scale_ld is None:
        a_scale_ld = a_scales.stride(0)
    _rows(a_q, "a_q", CODE_DTYPES, M, K)
    _rows(w_q, "w_q", CODE_DTYPES, N, K)
    _same_codes(a_q, w_q)
    per_channel = tuple(block_shape)[0] == 1
    _scales(a_scales, "a_scales", a_layout, a_scale_ld, M, 1 if per_channel else K // 128,
            write=False)
    _flat(w_scales, "w_scales", ("float32",), N if per_channel else (N // 128) * (K // 128))
    _rows(out, "out", OUT_DTYPES, M, N)
    _devices(a_q=a_q, a_scales=a_scales, w_q=w_q, w_scales=w_scales, out=out)
    st = lib.bfq_block_gemm_noalloc(_ptr(a_q), _ptr(a_scales), a_layout, a_scale_ld, _ptr(w_q),
                                    _ptr(w_scales), w_layout, scale_fmt, _ptr(out), M, N, K,
                                    _block_shape(block_shape), _qdtype(a_q), _odtype(out),
                                    ctypes.byref(tile) if tile else None, _stream(stream))
    return _check(st, "bfq_block_gemm_noalloc", warn_key=(N, K))


def bfq_noalloc_scratch_bytes() -> int:
    return int(lib.bfq_noalloc_scratch_bytes())


def bfq_load_tile_table(path=None) -> int:
    st = lib.bfq_load_tile_table(path.encode() if path else None)
    return _check(st, "bfq_load_tile_table")


def bfq_num_tile_candidates(in_dtype=BFQ_E4M3FN, w_layout=BFQ_W_ROW_MAJOR,
                            scale_fmt=BFQ_SCALE_FP32, block_shape=BLOCK_SHAPE) -> int:
    return int(lib.bfq_num_tile_candidates(_block_shape(block_shape), in_dtype, w_layout,
                                           scale_fmt))


def bfq_get_tile_candidate(index, in_dtype=BFQ_E4M3FN, w_layout=BFQ_W_ROW_MAJOR,
                           scale_fmt=BFQ_SCALE_FP32, block_shape=BLOCK_SHAPE) -> bfq_tile:
    t = bfq_tile()
    _check(lib.bfq_get_tile_candidate(_block_shape(block_shape), in_dtype, w_layout, scale_fmt,
                                      index, ctypes.byref(t)),
           "bfq_get_tile_candidate")
    return t


def bfq_moe_align(topk_ids, E, expert_offsets, sorted_pairs, workspace=None, stream=None) -> int:
    """topk_ids int32 [T, topk]; expert_offsets int32 [E+1]; sorted_pairs int32 [T*topk]."""
    T, topk = _shape2(topk_ids, "topk_ids")
    need = int(lib.bfq_moe_align_workspace_bytes(T, topk, E))
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _rows(topk_ids, "topk_ids", ("int32",), T, topk)
    _flat(expert_offsets, "expert_offsets", ("int32",), E + 1)
    _flat(sorted_pairs, "sorted_pairs", ("int32",), T * topk, exact=False)
    _workspace(workspace, need)
    _devices(topk_ids=topk_ids, expert_offsets=expert_offsets, sorted_pairs=sorted_pairs,
             workspace=workspace)
    st = lib.bfq_moe_align(_ptr(topk_ids), T, topk, E, _ptr(expert_offsets), _ptr(sorted_pairs),
                           _ptr(workspace), wb if workspace is not None else need, _stream(stream))
    return _check(st, "bfq_moe_align")


def bfq_moe_select_tile(T, topk, E, N, K, out_dtype=BFQ_BF16, w_layout=BFQ_W_ROW_MAJOR,
                        scale_fmt=BFQ_SCALE_FP32):
    """Returns (status, bfq_tile)."""
    t = bfq_tile()
    st = lib.bfq_moe_select_tile(T, topk, E, N, K, _block_shape(BLOCK_SHAPE), BFQ_E4M3FN,
                                 out_dtype, w_layout, scale_fmt, ctypes.byref(t))
    if st < 0:
        raise BfqError(st, "bfq_moe_select_tile")
    return st, t


def bfq_moe_gemm_workspace_bytes(T, topk, N, tile) -> int:
    return int(lib.bfq_moe_gemm_workspace_bytes(T, topk, N, ctypes.byref(tile)))


def bfq_moe_block_gemm(a_q, a_scales, sorted_pairs, expert_offsets, topk, w_q, w_scales, out,
                       a_layout=BFQ_SCALES_ROW_MAJOR, a_scale_ld=None, tile=None, workspace=None,
                       workspace_bytes=None, stream=None, w_layout=BFQ_W_ROW_MAJOR,
                       scale_fmt=BFQ_SCALE_FP32) -> int:
    """a_q [T, K]; w_q [E, N, K] (row-major, or each expert packed); w_scales
    [E, N/128, K/128]; out [T*topk, N] in pair order."""
    T, K = _shape2(a_q, "a_q")
    if not hasattr(w_q, "dim") or w_q.dim() != 3:
        raise BfqArgumentError("w_q must be a 3-D [E, N, K] tensor")
    E, N = w_q.shape[0], w_q.shape[1]
    if a_scale_ld is None:
        a_scale_ld = a_scales.stride(0)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _rows(a_q, "a_q", U8_CODES, T, K)
    if w_q.shape[2] != K:
        raise BfqArgumentError(f"w_q has shape {tuple(w_q.shape)}; its last dimension must be K={K}")
    _flat(w_q, "w_q", U8_CODES, E * N * K)
    _scales(a_scales, "a_scales", a_layout, a_scale_ld, T, K // 128, write=False)
    _flat(w_scales, "w_scales", ("float32",), E * (N // 128) * (K // 128))
    _flat(sorted_pairs, "sorted_pairs", ("int32",), T * topk, exact=False)
    _flat(expert_offsets, "expert_offsets", ("int32",), E + 1)
    _rows(out, "out", OUT_DTYPES, T * topk, N)
    _workspace(workspace, workspace_bytes)
    _devices(a_q=a_q, a_scales=a_scales, sorted_pairs=sorted_pairs,
             expert_offsets=expert_offsets, w_q=w_q, w_scales=w_scales, out=out,
             workspace=workspace)
    st = lib.bfq_moe_block_gemm(_ptr(a_q), _ptr(a_scales), a_layout, a_scale_ld, _ptr(sorted_pairs),
                                _ptr(expert_offsets), topk, _ptr(w_q), _ptr(w_scales), w_layout,
                                scale_fmt, _ptr(out), T, N, K, E, _block_shape(BLOCK_SHAPE),
                                BFQ_E4M3FN, _odtype(out), ctypes.byref(tile) if tile else None,
                                _ptr(workspace), workspace_bytes, _stream(stream))
    return _check(st, "bfq_moe_block_gemm", warn_key=("moe", E, N, K))


def bfq_moe_num_tile_candidates(w_layout=BFQ_W_ROW_MAJOR, scale_fmt=BFQ_SCALE_FP32) -> int:
    return int(lib.bfq_moe_num_tile_candidates(w_layout, scale_fmt))


def bfq_moe_get_tile_candidate(index, w_layout=BFQ_W_ROW_MAJOR, scale_fmt=BFQ_SCALE_FP32) -> bfq_tile:
    t = bfq_tile()
    _check(lib.bfq_moe_get_tile_candidate(w_layout, scale_fmt, index, ctypes.byref(t)),
           "bfq_moe_get_tile_candidate")
    return t


def bfq_status_string(s: int) -> str:
    return status_string(s)


def bfq_set_batch_invariant(enable: bool) -> None:
    lib.bfq_set_batch_invariant(1 if enable else 0)


def bfq_get_batch_invariant() -> bool:
    return bool(lib.bfq_get_batch_invariant())


def bfq_last_error() -> str:
    return last_error()


def bfq_debug_block_partials_i32(a_q, w_q, partials, stream=None) -> int:
    M, K = _shape2(a_q, "a_q")
    N = _shape2(w_q, "w_q")[0]
    _rows(a_q, "a_q", ("int8",), M, K)
    _rows(w_q, "w_q", ("int8",), N, K)
    _flat(partials, "partials", ("int32",), (K // 128) * M * N)
    _devices(a_q=a_q, w_q=w_q, partials=partials)
    st = lib.bfq_debug_block_partials_i32(_ptr(a_q), _ptr(w_q), _ptr(partials), M, N, K,
                                          _stream(stream))
    return _check(st, "bfq_debug_block_partials_i32")


def bfq_probe_mfma_peak(blocks, iters, out, stream=None) -> float:
    """Launch the MFMA-only probe (out: >= blocks * 512 fp32 on the device); returns the
    flops of the launch."""
    _flat(out, "out", ("float32",), blocks * 512, exact=False)
    _devices(out=out)
    _check(lib.bfq_probe_mfma_peak(blocks, iters, _ptr(out), _stream(stream)),
           "bfq_probe_mfma_peak")
    return float(lib.bfq_probe_mfma_flops(blocks, iters))


def bfq_debug_encode(x, codes, q_dtype=BFQ_E4M3FN, stream=None) -> int:
    _flat(x, "x", ("float32",), x.numel())
    _flat(codes, "codes", CODE_DTYPES, x.numel())
    _devices(x=x, codes=codes)
    st = lib.bfq_debug_encode(_ptr(x), x.numel(), q_dtype, _ptr(codes), _stream(stream))
    return _check(st, "bfq_debug_encode")


# ------------------------------------------------------------ allocating conveniences

def quant_tokens(x, q_dtype=BFQ_E4M3FN, layout=BFQ_SCALES_ROW_MAJOR, eps=DEFAULT_EPS,
                 stream=None, scale_fmt=BFQ_SCALE_FP32, per_token=False):
    """Allocate (q, scales) with torch and run bfq_quant_tokens. Returns (q, scales); with
    per_token the scales are [M, 1] (row-major) or [1, M] (column-major); with
    BFQ_SCALES_PACKED_UE8M0 they are int32 words [ceil(K/512), round_up(M, 4)]."""
    import torch
    M, K = x.shape
    group = K if per_token else 128
    q = torch.empty((M, K), dtype=torch.uint8 if q_dtype == BFQ_E4M3FN else torch.int8,
                    device=x.device)
    if layout == BFQ_SCALES_ROW_MAJOR:
        s = torch.empty((M, K // group), dtype=torch.float32, device=x.device)
    elif layout == BFQ_SCALES_PACKED_UE8M0:     # int32 words [ceil(G/4), round_up(M, 4)]
        s = torch.empty(((K // 128 + 3) // 4, (M + 3) // 4 * 4), dtype=torch.int32,
                        device=x.device)
    else:
        s = torch.empty((K // group, M), dtype=torch.float32, device=x.device)
    bfq_quant_tokens(x, q, s, layout=layout, scale_ld=s.stride(0), eps=eps, stream=stream,
                     scale_fmt=scale_fmt, group_size=group)
    return q, s


def quant_weight_blocks(w, q_dtype=BFQ_E4M3FN, eps=DEFAULT_EPS, stream=None,
                        scale_fmt=BFQ_SCALE_FP32, per_channel=False):
    """Allocate (q, scales) with torch and run bfq_quant_weight_blocks; per_channel gives one
    scale per output channel (scales [N])."""
    import torch
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8 if q_dtype == BFQ_E4M3FN else torch.int8,
                    device=w.device)
    if per_channel:
        s = torch.empty((N,), dtype=torch.float32, device=w.device)
        bs = channel_block_shape(K)
    else:
        s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
        bs = BLOCK_SHAPE
    bfq_quant_weight_blocks(w, q, s, eps=eps, stream=stream, scale_fmt=scale_fmt, block_shape=bs)
    return q, s


def moe_align(topk_ids, E, stream=None):
    """Allocate and run bfq_moe_align. Returns (expert_offsets int32 [E+1], sorted_pairs
    int32 [T*topk])."""
    import torch
    T, topk = topk_ids.shape
    dev = topk_ids.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    srt = torch.empty(T * topk, dtype=torch.int32, device=dev)
    need = int(lib.bfq_moe_align_workspace_bytes(T, topk, E))
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    bfq_moe_align(topk_ids, E, off, srt, workspace=ws, stream=stream)
    return off, srt


def moe_block_gemm(a_q, a_scales, sorted_pairs, expert_offsets, topk, w_q, w_scales,
                   out_dtype=None, a_layout=BFQ_SCALES_ROW_MAJOR, tile=None, stream=None,
                   w_layout=BFQ_W_ROW_MAJOR, scale_fmt=BFQ_SCALE_FP32):
    """Allocate out [T*topk, N] (and split-K workspace) with torch and run bfq_moe_block_gemm."""
    import torch
    out_dtype = out_dtype or torch.bfloat16
    T, K = a_q.shape
    E, N = w_q.shape[0], w_q.shape[1]
    out = torch.empty((T * topk, N), dtype=out_dtype, device=a_q.device)
    if tile is None:
        st, tile = bfq_moe_select_tile(T, topk, E, N, K, _odtype(out), w_layout, scale_fmt)
        _check(st, "bfq_moe_select_tile", warn_key=("moe", E, N, K))
    ws_bytes = bfq_moe_gemm_workspace_bytes(T, topk, N, tile)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=a_q.device) if ws_bytes else None
    bfq_moe_block_gemm(a_q, a_scales, sorted_pairs, expert_offsets, topk, w_q, w_scales, out,
                       a_layout=a_layout, tile=tile, workspace=ws, workspace_bytes=ws_bytes,
                       stream=stream, w_layout=w_layout, scale_fmt=scale_fmt)
    return out


def pack_weights(w_q, stream=None):
    """Allocate a packed copy of row-major weight codes (same dtype and shape) with torch and
    run bfq_pack_weights. [E, N, K] expert weights pack as one [E*N, K] matrix, which is each
    expert packed in turn (16-row fragments never straddle experts, N being a multiple of
    128)."""
    import torch
    p = torch.empty_like(w_q, memory_format=torch.contiguous_format)
    bfq_pack_weights(w_q.reshape(-1, w_q.shape[-1]), p.view(-1, w_q.shape[-1]), stream=stream)
    return p


def block_gemm(a_q, a_scales, w_q, w_scales, out_dtype=None, a_layout=BFQ_SCALES_ROW_MAJOR,
               tile=None, stream=None, w_layout=BFQ_W_ROW_MAJOR, scale_fmt=BFQ_SCALE_FP32,
               per_channel=False):
    """Allocate out (and split-K workspace) with torch and run bfq_block_gemm; per_channel
    selects the per-token x per-channel format (block_shape (1, K))."""
    import torch
    out_dtype = out_dtype or torch.bfloat16
    M, K = a_q.shape
    N = w_q.shape[0]
    bs = channel_block_shape(K) if per_channel else BLOCK_SHAPE
    out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    if tile is None:
        st, tile = bfq_select_tile(M, N, K, _qdtype(a_q), _odtype(out), w_layout=w_layout,
                                   scale_fmt=scale_fmt, block_shape=bs)
        _check(st, "bfq_select_tile", warn_key=(N, K))
    ws_bytes = bfq_gemm_workspace_bytes(M, N, K, tile)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=a_q.device) if ws_bytes else None
    bfq_block_gemm(a_q, a_scales, w_q, w_scales, out, a_layout=a_layout, tile=tile,
                   workspace=ws, workspace_bytes=ws_bytes, stream=stream, w_layout=w_layout,
                   scale_fmt=scale_fmt, block_shape=bs)
    return out
