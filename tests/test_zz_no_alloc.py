"""The allocation-free block GEMM (bfq_block_gemm_noalloc) against bfq_block_gemm: same tile,
same inputs -> bitwise the same output, on two calls in a row whose second is smaller (the
static scratch keeps the first call's partials, which the second must not read), and both
within the parity bar of the oracle. With no tile given, a selected stream-K tile runs as the
plain grid of the same tile inside the buffer; explicit tiles that need more workspace than
the buffer holds are rejected without a launch."""
import ctypes

import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(orc, M, N, K, seed, qtype):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed + 1).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), qtype=qtype)
    qw, sw = orc.quant_blocks(w, qtype=qtype)
    return qa, sa, qw, sw


def _dev(*arrs):
    return [torch.from_numpy(a).to(DEV) for a in arrs]


def _with(t, **kw):
    d = t.as_dict()
    d.update(kw)
    return type(t).from_dict(d)


def _both(bfq, qa, sa, qw, sw, tile, odt, w_layout):
    """(allocating entry point with a torch workspace, allocation-free entry point)."""
    M, N = qa.shape[0], qw.shape[0]
    ref = torch.full((M, N), float("nan"), dtype=odt, device=DEV)
    got = torch.full((M, N), float("nan"), dtype=odt, device=DEV)
    need = bfq.bfq_gemm_workspace_bytes(M, N, qa.shape[1], tile)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    bfq.bfq_block_gemm(qa, sa, qw, sw, ref, tile=tile, workspace=ws, workspace_bytes=need,
                       w_layout=w_layout)
    st = bfq.bfq_block_gemm_noalloc(qa, sa, qw, sw, got, tile=tile, w_layout=w_layout)
    torch.cuda.synchronize()
    return ref, got, st


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_noalloc_matches_allocating_entry_point(bfq, orc, qname):
    from oracle import metrics
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    N, K = 1536, 7168
    cands = [bfq.bfq_get_tile_candidate(i, qd) for i in range(bfq.bfq_num_tile_candidates(qd))]
    std = next(t for t in cands if t.variant == 0 and t.bm == 128 and t.bn == 128)
    sab = next(t for t in cands if t.variant == 1)
    big = _inputs(orc, 300, N, K, 5, qt)
    ref32_big, _ = orc.block_gemm(*big, qtype=qt)
    small = _inputs(orc, 40, N, K, 7, qt)
    ref32_small, _ = orc.block_gemm(*small, qtype=qt)
    for tile in (_with(std, split_k=4), _with(sab, split_k=2), _with(std, split_k=1)):
        # two calls in a row, the second smaller: M = 300 (7.4 MB of split-K partials), then 40
        for (host, ref32) in ((big, ref32_big), (small, ref32_small)):
            qa, sa, qw, sw = _dev(*host)
            M = qa.shape[0]
            print("noalloc", qname, M, tile.as_dict(), flush=True)
            for odt in (torch.float32, torch.bfloat16):
                ref, got, st = _both(bfq, qa, sa, qw, sw, tile, odt, bfq.BFQ_W_ROW_MAJOR)
                assert st == bfq.BFQ_OK
                assert torch.equal(_bits(got), _bits(ref)), (qname, M, tile.as_dict(), odt)
                if odt == torch.float32:
                    r = metrics.gemm_fp32_report(got.cpu().numpy(), ref32)
                    assert r["ok"], (qname, M, tile.as_dict(), r)


def test_noalloc_selected_stream_k_tile_runs_in_the_buffer(bfq, orc):
    """M = 1024 on the wide up-projection: the tuned tile is stream-K (128 MiB of slots); the
    allocation-free call runs the same tile on the plain grid and matches bfq_block_gemm with
    that tile given explicitly, bit for bit, and the oracle on sampled outputs."""
    from oracle import metrics
    M, N, K = 1024, 24576, 7168
    wl = bfq.BFQ_W_PACKED16
    _, sel = bfq.bfq_select_tile(M, N, K, w_layout=wl)
    print("selected", sel.as_dict(), flush=True)
    x = synth.activations(M, K, seed=0)
    w = synth.weights(N, K, seed=0)
    qw, sw = bfq.quant_weight_blocks(w.to(DEV))
    qwp = bfq.pack_weights(qw)
    qa, sa = bfq.quant_tokens(x.to(DEV))
    # the tile the allocation-free call should run: stream-K on the plain grid, K split
    # reduced until the partials fit the buffer
    want = _with(sel, variant=0, split_k=1) if sel.variant == 2 else sel
    cap = bfq.bfq_noalloc_scratch_bytes()
    while want.split_k > 1 and bfq.bfq_gemm_workspace_bytes(M, N, K, want) > cap:
        want = _with(want, split_k=want.split_k - 1)
    ref, got, st = _both(bfq, qa, sa, qwp, sw, want, torch.float32, wl)
    assert torch.equal(_bits(got), _bits(ref))
    got2 = torch.full_like(got, float("nan"))
    st2 = bfq.bfq_block_gemm_noalloc(qa, sa, qwp, sw, got2, w_layout=wl)      # tile NULL
    torch.cuda.synchronize()
    assert st2 >= 0
    assert torch.equal(_bits(got2), _bits(ref)), (sel.as_dict(), want.as_dict())
    rng = np.random.default_rng(3)
    ms = np.concatenate([rng.integers(0, M, 2048), [0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 2048), [N - 1, 0]])
    qa_o, sa_o = orc.quant_groups(synth.bf16_bits(x))
    qw_o, sw_o = orc.quant_blocks(w.numpy())
    r = metrics.gemm_fp32_report(got2.cpu().numpy()[ms, ns],
                                 orc.block_gemm_sampled(qa_o, sa_o, qw_o, sw_o, ms, ns))
    assert r["ok"], r


def test_noalloc_rejects_tiles_beyond_the_buffer(bfq):
    """Explicit tiles needing more than the buffer: BFQ_ERR_WORKSPACE, output untouched."""
    M, N, K = 1024, 24576, 7168
    qa = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    sa = torch.ones((M, K // 128), dtype=torch.float32, device=DEV)
    qw = torch.zeros((N, K), dtype=torch.uint8, device=DEV)
    sw = torch.ones((N // 128, K // 128), dtype=torch.float32, device=DEV)
    out = torch.full((M, N), 7.0, dtype=torch.float32, device=DEV)
    cands = [bfq.bfq_get_tile_candidate(i) for i in range(bfq.bfq_num_tile_candidates())]
    sk = next(t for t in cands if t.variant == 2)
    split = _with(next(t for t in cands if t.variant == 0), split_k=4)   # 4*1024*24576*4 B
    for t in (sk, split):
        assert bfq.bfq_gemm_workspace_bytes(M, N, K, t) > bfq.bfq_noalloc_scratch_bytes()
        with pytest.raises(bfq.BfqError, match="allocation-free"):
            bfq.bfq_block_gemm_noalloc(qa, sa, qw, sw, out, tile=t)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    bs = (ctypes.c_int32 * 2)(128, 128)
    assert bfq.lib.bfq_block_gemm_noalloc(None, None, 0, 56, None, None, 0, 0, None, 0, N, K, bs,
                                          bfq.BFQ_E4M3FN, bfq.BFQ_BF16, None, None) == bfq.BFQ_ERR_NULL
