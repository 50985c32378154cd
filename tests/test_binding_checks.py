"""CPU tests of the Python binding's argument checks: every wrapper rejects a tensor that does
not match what its kernel reads or writes (wrong dtype, shape, strides, size, or a host
tensor) with BfqArgumentError before the C call, so nothing is launched. Host tensors are
used throughout: a tensor that passes every other check fails the device check last."""
import pytest
import torch


def _err(bfq, match, fn, *a, **kw):
    with pytest.raises(bfq.BfqArgumentError, match=match):
        fn(*a, **kw)


def test_quant_tokens_checks(bfq):
    M, K = 4, 256
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    q = torch.zeros((M, K), dtype=torch.uint8)
    s = torch.zeros((M, K // 128), dtype=torch.float32)
    _err(bfq, "dtype float32", bfq.bfq_quant_tokens, x.float(), q, s)
    wide = torch.zeros((M, 2 * K), dtype=torch.bfloat16)
    _err(bfq, "strides", bfq.bfq_quant_tokens, wide[:, :K], q, s)    # a column slice
    _err(bfq, "shape", bfq.bfq_quant_tokens, x, q[:, :128], s)
    _err(bfq, "needs at least", bfq.bfq_quant_tokens, x, q, s[:, :1])
    _err(bfq, "row stride", bfq.bfq_quant_tokens, x, q, s, scale_ld=5)
    _err(bfq, "needs at least", bfq.bfq_quant_tokens, x, q, s.t().contiguous()[:, :3],
         layout=bfq.BFQ_SCALES_COL_MAJOR)
    # packed words: int32, rows rounded up to 4 tokens when written
    words = torch.zeros((1, M), dtype=torch.int32)
    _err(bfq, "dtype", bfq.bfq_quant_tokens, x, q, words.float(),
         layout=bfq.BFQ_SCALES_PACKED_UE8M0, scale_fmt=bfq.BFQ_SCALE_UE8M0)
    _err(bfq, "device", bfq.bfq_quant_tokens, x, q, words,
         layout=bfq.BFQ_SCALES_PACKED_UE8M0, scale_fmt=bfq.BFQ_SCALE_UE8M0)
    _err(bfq, "needs at least", bfq.bfq_quant_tokens, x[:3], q[:3], words[:, :2],
         layout=bfq.BFQ_SCALES_PACKED_UE8M0, scale_fmt=bfq.BFQ_SCALE_UE8M0)
    _err(bfq, "2-D", bfq.bfq_quant_tokens, x.reshape(-1), q, s)
    _err(bfq, "device", bfq.bfq_quant_tokens, x, q, s)   # everything else is right


def test_weight_quant_and_pack_checks(bfq):
    N, K = 256, 256
    w = torch.zeros((N, K), dtype=torch.float32)
    q = torch.zeros((N, K), dtype=torch.uint8)
    s = torch.zeros((N // 128, K // 128), dtype=torch.float32)
    _err(bfq, "dtype bfloat16", bfq.bfq_quant_weight_blocks, w.bfloat16(), q, s)
    _err(bfq, "elements", bfq.bfq_quant_weight_blocks, w, q, s[:1])
    _err(bfq, "elements", bfq.bfq_quant_weight_blocks, w, q, s, block_shape=(1, K))
    _err(bfq, "strides", bfq.bfq_quant_weight_blocks, w.t(), q, s)
    _err(bfq, "device", bfq.bfq_quant_weight_blocks, w, q, s)
    _err(bfq, "exactly N\\*K bytes", bfq.bfq_pack_weights, q, torch.zeros(N * K - 16, dtype=torch.uint8))
    _err(bfq, "dtype float32", bfq.bfq_pack_weights, w, q)
    _err(bfq, "device", bfq.bfq_pack_weights, q, torch.zeros_like(q))


def test_block_gemm_checks(bfq):
    M, N, K = 8, 256, 512
    a = torch.zeros((M, K), dtype=torch.uint8)
    sa = torch.zeros((M, K // 128), dtype=torch.float32)
    w = torch.zeros((N, K), dtype=torch.uint8)
    sw = torch.zeros((N // 128, K // 128), dtype=torch.float32)
    out = torch.zeros((M, N), dtype=torch.bfloat16)
    g = bfq.bfq_block_gemm
    _err(bfq, "dtype float32", g, a.float(), sa, w, sw, out)
    _err(bfq, "different code types", g, a, sa, w.view(torch.int8), sw, out)
    _err(bfq, "shape", g, a, sa, w[:, :256], sw, out)
    _err(bfq, "strides", g, a, sa, torch.zeros((N, 2 * K), dtype=torch.uint8)[:, K:], sw, out)
    _err(bfq, "needs at least", g, a, sa[:, :2], w, sw, out)
    _err(bfq, "needs at least", g, a, sa.t().contiguous()[:, :4], w, sw, out,
         a_layout=bfq.BFQ_SCALES_COL_MAJOR)
    _err(bfq, "elements", g, a, sa, w, sw[:1], out)
    _err(bfq, "shape", g, a, sa, w, sw, out[:, :128])
    _err(bfq, "dtype int32", g, a, sa, w, sw, out.int())
    _err(bfq, "strides", g, a, sa, w, sw, torch.zeros((N, M), dtype=torch.bfloat16).t())
    _err(bfq, "bytes", g, a, sa, w, sw, out, workspace=torch.zeros(64, dtype=torch.uint8),
         workspace_bytes=4096)
    # per-token x per-channel: [M, 1] token scales, N channel scales
    _err(bfq, "elements", g, a, sa[:, :1], w, sw, out, block_shape=(1, K))
    _err(bfq, "device", g, a, sa[:, :1].contiguous(), w, torch.zeros(N), out, block_shape=(1, K))
    _err(bfq, "device", g, a, sa, w, sw, out)


def test_moe_and_debug_checks(bfq):
    T, topk, E, N, K = 4, 2, 3, 256, 256
    a = torch.zeros((T, K), dtype=torch.uint8)
    sa = torch.zeros((T, K // 128), dtype=torch.float32)
    w = torch.zeros((E, N, K), dtype=torch.uint8)
    sw = torch.zeros((E, N // 128, K // 128), dtype=torch.float32)
    srt = torch.zeros(T * topk, dtype=torch.int32)
    off = torch.zeros(E + 1, dtype=torch.int32)
    out = torch.zeros((T * topk, N), dtype=torch.bfloat16)
    g = bfq.bfq_moe_block_gemm
    _err(bfq, "3-D", g, a, sa, srt, off, topk, w[0], sw, out)
    _err(bfq, "dtype int8", g, a.view(torch.int8), sa, srt, off, topk, w, sw, out)
    _err(bfq, "last dimension", g, a, sa, srt, off, topk, w[:, :, :128], sw, out)
    _err(bfq, "at least", g, a, sa, srt[:3], off, topk, w, sw, out)
    _err(bfq, "elements", g, a, sa, srt, off[:E], topk, w, sw, out)
    _err(bfq, "dtype int64", g, a, sa, srt.long(), off, topk, w, sw, out)
    _err(bfq, "shape", g, a, sa, srt, off, topk, w, sw, out[:T])
    _err(bfq, "device", g, a, sa, srt, off, topk, w, sw, out)
    # a pair list preallocated for more tokens is fine (only the first T*topk entries are read)
    big = torch.zeros(16 * T * topk, dtype=torch.int32)
    _err(bfq, "device", g, a, sa, big, off, topk, w, sw, out)
    ids = torch.zeros((T, topk), dtype=torch.int32)
    _err(bfq, "dtype int64", bfq.bfq_moe_align, ids.long(), E, off, srt)
    _err(bfq, "elements", bfq.bfq_moe_align, ids, E, off[:2], srt)
    _err(bfq, "at least", bfq.bfq_moe_align, ids, E, off, srt[:T * topk - 1])
    _err(bfq, "device", bfq.bfq_moe_align, ids, E, off, big)
    _err(bfq, "device", bfq.bfq_moe_align, ids, E, off, srt)
    ai = torch.zeros((T, K), dtype=torch.int8)
    _err(bfq, "elements", bfq.bfq_debug_block_partials_i32, ai, torch.zeros((N, K), dtype=torch.int8),
         torch.zeros((K // 128, T, N - 1), dtype=torch.int32))
    _err(bfq, "elements", bfq.bfq_debug_encode, torch.zeros(64), torch.zeros(32, dtype=torch.uint8))
