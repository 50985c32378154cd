"""HIP-graph capture of the library's calls: a captured sequence (quantize, GEMM with split-K
workspace and reduction, stream-K fixup, MoE routing sort + grouped GEMM) is replayed several
times with eager work and synchronizations in between, and every replay must equal the eager
result bit for bit (the kernels hold no state between calls and enqueue no memset)."""
import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _tile(bfq, **kw):
    d = {"variant": 0, "bm": 128, "bn": 128, "waves_m": 2, "waves_n": 2, "stages": 2,
         "group_m": 8, "sched": 0, "raster": 0, "split_k": 1}
    d.update(kw)
    return bfq.bfq_tile.from_dict(d)


def _replay_check(step, outs, reps=4):
    """Eager reference, then capture and replay `reps` times with eager work in between."""
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        torch.ones(1 << 20, device=DEV).sum()        # unrelated eager work between replays
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.int8) if o.element_size() == 1 else o.view(torch.int16)
                               if o.element_size() == 2 else o.view(torch.int32),
                               e.view(torch.int8) if e.element_size() == 1 else e.view(torch.int16)
                               if e.element_size() == 2 else e.view(torch.int32)), r


@pytest.mark.parametrize("case", ["split", "streamk", "swapab", "channel", "packed"])
def test_graph_replay_dense(bfq, case):
    M, N, K = 300, 1536, 2048
    x = synth.activations(M, K, seed=81).to(DEV)
    w = synth.weights(N, K, seed=82).to(DEV)
    sf = bfq.BFQ_SCALE_UE8M0 if case == "packed" else bfq.BFQ_SCALE_FP32
    per_channel = case == "channel"
    qw, sw = bfq.quant_weight_blocks(w, scale_fmt=sf, per_channel=per_channel)
    qwp = bfq.pack_weights(qw)
    if case == "packed":
        lay = bfq.BFQ_SCALES_PACKED_UE8M0
        sa = torch.empty(((K // 128 + 3) // 4, (M + 3) // 4 * 4), dtype=torch.int32, device=DEV)
        group = 128
    else:
        lay = bfq.BFQ_SCALES_COL_MAJOR
        sa = torch.empty((1 if per_channel else K // 128, M), dtype=torch.float32, device=DEV)
        group = K if per_channel else 128
    qa = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    bs = bfq.channel_block_shape(K) if per_channel else bfq.BLOCK_SHAPE
    tile = {"split": _tile(bfq, split_k=4),
            "streamk": _tile(bfq, variant=2, bm=256, bn=256, waves_m=4, waves_n=2),
            "swapab": _tile(bfq, variant=1, bm=64, bn=96, waves_m=2, waves_n=6, stages=4, sched=1,
                            group_m=1, split_k=2),
            "channel": _tile(bfq, sched=4, split_k=2),
            "packed": _tile(bfq, bm=256, bn=256, waves_m=4, waves_n=2, sched=3)}[case]
    ws_bytes = bfq.bfq_gemm_workspace_bytes(M, N, K, tile)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)

    def step():
        bfq.bfq_quant_tokens(x, qa, sa, layout=lay, scale_ld=sa.stride(0), scale_fmt=sf,
                             group_size=group)
        bfq.bfq_block_gemm(qa, sa, qwp, sw, out, a_layout=lay, a_scale_ld=sa.stride(0), tile=tile,
                           workspace=ws, workspace_bytes=ws_bytes, w_layout=bfq.BFQ_W_PACKED16,
                           scale_fmt=sf, block_shape=bs)

    _replay_check(step, [qa, out])


def test_graph_replay_moe(bfq):
    T, E, topk, N, K = 200, 16, 4, 512, 1024
    x = synth.activations(T, K, seed=83).to(DEV)
    ids = synth.routing(T, E, topk, seed=83).to(DEV)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=DEV)
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=DEV)
    for e in range(E):
        q, s = bfq.quant_weight_blocks(synth.expert_weight_on(DEV, e, N, K, seed=83))
        qw[e].copy_(q)
        sw[e].copy_(s)
    qa, sa = bfq.quant_tokens(x, layout=bfq.BFQ_SCALES_COL_MAJOR)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    srt = torch.empty(T * topk, dtype=torch.int32, device=DEV)
    aws = torch.empty(max(int(bfq.lib.bfq_moe_align_workspace_bytes(T, topk, E)), 16),
                      dtype=torch.uint8, device=DEV)
    out = torch.empty((T * topk, N), dtype=torch.bfloat16, device=DEV)
    tiles = [_tile(bfq, variant=1, bm=32, bn=128, waves_m=1, waves_n=8, stages=4, sched=1,
                   group_m=1, split_k=2), _tile(bfq, group_m=1)]
    for tile in tiles:
        ws_bytes = bfq.bfq_moe_gemm_workspace_bytes(T, topk, N, tile)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)

        def step():
            bfq.bfq_quant_tokens(x, qa, sa, layout=bfq.BFQ_SCALES_COL_MAJOR, scale_ld=sa.stride(0))
            bfq.bfq_moe_align(ids, E, off, srt, workspace=aws)
            bfq.bfq_moe_block_gemm(qa, sa, srt, off, topk, qw, sw, out,
                                   a_layout=bfq.BFQ_SCALES_COL_MAJOR, a_scale_ld=sa.stride(0),
                                   tile=tile, workspace=ws, workspace_bytes=ws_bytes)

        _replay_check(step, [qa, off, srt, out])
