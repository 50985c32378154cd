"""GPU parity at the library's size limits, through the C-ABI, against the CPU oracle.

  * K = 2^23, the largest K the block GEMM and the quantizer take: a 128-row weight tile
    spans 2^30 bytes behind one buffer resource, the scale tables hold 65536 K blocks, and
    a whole-K workgroup runs 65536 block steps.
  * M x N above 2^31 output elements: output, partial and activation offsets need 64 bits.

The GEMM inputs are drawn directly as codes and scales (synth.codes / synth.scales: a GEMM
takes any codes and positive scales), so no gigabyte array is quantized on the host; the
oracle is evaluated on sampled outputs (block_gemm_sampled), which it computes one by one.
Bar: the fp32 parity bar of oracle/metrics.py on the samples; quantizer codes and scales
bit-exact on sampled rows.
"""
import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
K_MAX = 1 << 23


def _gemm(bfq, qa, sa, qw, sw, layout, tile=None, out_dtype=torch.float32):
    wl = bfq.BFQ_W_PACKED16 if layout == "packed" else bfq.BFQ_W_ROW_MAJOR
    M, K = qa.shape
    N = qw.shape[0]
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    if tile is None:
        st, tile = bfq.bfq_select_tile(M, N, K, bfq._qdtype(qa), bfq._odtype(out), w_layout=wl)
    need = bfq.bfq_gemm_workspace_bytes(M, N, K, tile)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    bfq.bfq_block_gemm(qa, sa, qw, sw, out, a_layout=bfq.BFQ_SCALES_ROW_MAJOR,
                       a_scale_ld=sa.stride(0), tile=tile, workspace=ws, workspace_bytes=need,
                       w_layout=wl)
    torch.cuda.synchronize()
    return out, tile


def _with_split(t, s):
    d = t.as_dict()
    d["split_k"] = s
    return type(t).from_dict(d)


def _samples(rng, M, N, n=32):
    ms = np.concatenate([[0, M - 1, M - 1, 0], rng.integers(0, M, n)]).astype(np.int64)
    ns = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, n)]).astype(np.int64)
    return ms, ns


@pytest.mark.parametrize("layout", ["row", "packed"])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_maximum_k_gemm(bfq, orc, qname, layout):
    """K = 2^23, N = 128: the selected tile at M = 1, 40 and 160 (the swap-AB and standard
    families), and at M = 160 every compiled candidate with split_k 1 and 7 (stream-K:
    1), sampled against the oracle."""
    from oracle import metrics
    int8 = qname == "int8"
    qd = bfq.BFQ_INT8 if int8 else bfq.BFQ_E4M3FN
    qt = orc.INT8 if int8 else orc.FP8
    N, M_MAX = 128, 160
    print(f"maximum K: {qname} {layout} K={K_MAX}", flush=True)
    qa_all = synth.codes(M_MAX, K_MAX, int8, seed=401, device=DEV)
    sa_all = synth.scales(M_MAX, K_MAX // 128, seed=402, device=DEV)
    qw = synth.codes(N, K_MAX, int8, seed=403, device=DEV)
    sw = synth.scales(N // 128, K_MAX // 128, seed=404, device=DEV)
    host = [t.cpu().numpy() for t in (qa_all, sa_all, qw, sw)]
    if layout == "packed":
        qw = bfq.pack_weights(qw)
    wl = bfq.BFQ_W_PACKED16 if layout == "packed" else bfq.BFQ_W_ROW_MAJOR
    cands = [bfq.bfq_get_tile_candidate(i, qd, wl, 0)
             for i in range(bfq.bfq_num_tile_candidates(qd, wl, 0))]
    assert cands
    rng = np.random.default_rng(405)
    for M in (1, 40, M_MAX):
        qa, sa = qa_all[:M], sa_all[:M]
        ms, ns = _samples(rng, M, N)
        ref = orc.block_gemm_sampled(host[0][:M], host[1][:M], host[2], host[3], ms, ns,
                                     qtype=qt)
        tiles = [None]
        if M == M_MAX:
            tiles += [_with_split(t, s) for t in cands for s in (1, 7)
                      if not (t.variant == 2 and s > 1)]
        for t in tiles:
            out, used = _gemm(bfq, qa, sa, qw, sw, layout, tile=t)
            what = (qname, layout, M, used.as_dict(), "selected" if t is None else "candidate")
            print("  ", what, flush=True)
            got = out[torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)].cpu().numpy()
            r = metrics.gemm_fp32_report(got, ref)
            assert r["ok"], (what, r)


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_maximum_k_quant_tokens(bfq, orc, qname, layout):
    """Token-group quantization of 3 rows of K = 2^23 (65536 groups per row), both scale
    layouts: codes and scales bit-exact against the oracle."""
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    lay = bfq.BFQ_SCALES_ROW_MAJOR if layout == "row" else bfq.BFQ_SCALES_COL_MAJOR
    M, G = 3, K_MAX // 128
    x = synth.activations(M, K_MAX, seed=406)
    q = torch.full((M, K_MAX), 0x55, dtype=torch.uint8 if qname == "fp8" else torch.int8,
                   device=DEV)
    shape = (M, G) if layout == "row" else (G, M)
    s = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    bfq.bfq_quant_tokens(x.to(DEV), q, s, layout=lay, scale_ld=s.stride(0))
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(synth.bf16_bits(x), qtype=qt)
    sg = s.cpu().numpy()
    sg = sg if layout == "row" else sg.T.copy()
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))


def test_output_offsets_beyond_2_31(bfq, orc):
    """M = 2^20 + 19 tokens, N = 2304, K = 256: M*N = 2.4e9 output elements. The tokens are
    quantized on the device (sampled rows bit-exact against the oracle, including rows past
    2^20), then the selected tile's fp32 and bf16 outputs are sampled against the oracle,
    with samples in the last rows, whose offsets exceed 2^31, and the bf16 samples must be
    the rounding of the fp32 run's."""
    from oracle import metrics
    M, N, K = (1 << 20) + 19, 2304, 256
    print(f"large M: M={M} N={N} K={K}", flush=True)
    x = synth.activations(M, K, seed=407)
    xd = x.to(DEV)
    qa, sa = bfq.quant_tokens(xd, q_dtype=bfq.BFQ_E4M3FN, layout=bfq.BFQ_SCALES_ROW_MAJOR)
    rng = np.random.default_rng(408)
    rows = np.unique(np.concatenate([[0, 1, M // 2, (1 << 20) - 1, 1 << 20, M - 2, M - 1],
                                     rng.integers(0, M, 25)])).astype(np.int64)
    qo, so = orc.quant_groups(synth.bf16_bits(x[torch.from_numpy(rows)]))
    ri = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(qa[ri].cpu().numpy(), qo)
    assert np.array_equal(sa[ri].cpu().numpy().view(np.uint32), so.view(np.uint32))
    qw, sw = orc.quant_blocks(synth.weights(N, K, seed=409).numpy())
    # samples: every sampled row against a spread of columns, corners included
    ms_local = np.repeat(np.arange(rows.size), 6)
    ns = np.concatenate([[0, N - 1], rng.integers(0, N, ms_local.size - 2)]).astype(np.int64)
    ref = orc.block_gemm_sampled(qo, so, qw, sw, ms_local, ns)
    ms = rows[ms_local]
    mi, ni = torch.from_numpy(ms).to(DEV), torch.from_numpy(ns).to(DEV)
    for layout in ("row", "packed"):
        qw_d = torch.from_numpy(qw).to(DEV)
        if layout == "packed":
            qw_d = bfq.pack_weights(qw_d)
        sw_d = torch.from_numpy(sw).to(DEV)
        out32, used = _gemm(bfq, qa, sa, qw_d, sw_d, layout)
        got32 = out32[mi, ni].cpu().numpy()
        del out32
        r = metrics.gemm_fp32_report(got32, ref)
        assert r["ok"], (layout, used.as_dict(), r)
        out16, used16 = _gemm(bfq, qa, sa, qw_d, sw_d, layout, tile=used,
                              out_dtype=torch.bfloat16)
        got16 = out16[mi, ni].view(torch.int16).cpu().numpy().view(np.uint16)
        del out16
        assert np.array_equal(got16, orc.f32_to_bf16_bits_array(got32)), (layout, used.as_dict())
        torch.cuda.empty_cache()
