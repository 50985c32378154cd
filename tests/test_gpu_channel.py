"""GPU parity of the per-token x per-channel format (FP8_Dynamic / W8A8_INT8 of the Helion
linear-backend page, scope section), through the C-ABI, against the CPU oracle.

Bar: quantizer codes and scales bit-exact; GEMM fp32 output against the oracle's
channel_gemm within rel. Frobenius <= 1e-3 and max |diff| <= 2^-7 * rms(ref) + 1e-3 (the
GPU accumulates the whole-K dot product in fp32 in the MFMA, the oracle exactly and rounds
once); bf16 / fp16 output bit-exact roundings of the same tile's fp32 output;
integer-valued codes with power-of-two scales bit-exact (every step is exact).
"""
import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LAYOUTS = ["row", "packed"]


def _wl(bfq, layout):
    return bfq.BFQ_W_PACKED16 if layout == "packed" else bfq.BFQ_W_ROW_MAJOR


def _host_case(orc, M, N, K, seed, qt):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed + 1).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), group=K, qtype=qt)
    qw, sw = orc.quant_blocks(w, block=(1, K), qtype=qt)
    return qa, sa[:, 0].copy(), qw, sw[:, 0].copy()


def _to_dev(bfq, qa, sa, qw, sw, layout):
    qw_d = torch.from_numpy(qw).to(DEV)
    if layout == "packed":
        qw_d = bfq.pack_weights(qw_d)
    return (torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).reshape(-1, 1).to(DEV), qw_d,
            torch.from_numpy(sw).to(DEV), layout)


def _run(bfq, dq, out_dtype, tile=None, a_layout=None, sa_override=None):
    qa, sa, qw, sw, layout = dq
    wl = _wl(bfq, layout)
    M, K = qa.shape
    N = qw.shape[0]
    bs = bfq.channel_block_shape(K)
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    if tile is None:
        _, tile = bfq.bfq_select_tile(M, N, K, bfq._qdtype(qa), bfq._odtype(out), w_layout=wl,
                                      block_shape=bs)
    ws_bytes = bfq.bfq_gemm_workspace_bytes(M, N, K, tile)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    sa_arg = sa if sa_override is None else sa_override
    layout_arg = bfq.BFQ_SCALES_ROW_MAJOR if a_layout is None else a_layout
    bfq.bfq_block_gemm(qa, sa_arg, qw, sw, out, a_layout=layout_arg, a_scale_ld=sa_arg.stride(0),
                       tile=tile, workspace=ws, workspace_bytes=ws_bytes, w_layout=wl,
                       block_shape=bs)
    torch.cuda.synchronize()
    return out


def _candidates(bfq, qd, layout, K):
    wl = _wl(bfq, layout)
    bs = bfq.channel_block_shape(K)
    return [bfq.bfq_get_tile_candidate(i, qd, wl, 0, block_shape=bs)
            for i in range(bfq.bfq_num_tile_candidates(qd, wl, 0, block_shape=bs))]


def _with_split(t, s):
    d = t.as_dict()
    d["split_k"] = s
    return type(t).from_dict(d)


# ------------------------------------------------------------------------ quantizers

@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("M,K", [(1, 7168), (37, 1536), (128, 7168), (300, 768), (64, 18432),
                                 (4096, 7168), (5, 32768), (3, 256)])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_per_token_bit_exact(bfq, orc, M, K, qname, sfmt):
    print(f"quant per-token M={M} K={K} {qname} sfmt={sfmt}", flush=True)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    x = synth.activations(M, K, seed=M + 3 * K)
    q, s = bfq.quant_tokens(x.to(DEV), q_dtype=qd, scale_fmt=sfmt, per_token=True)
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(synth.bf16_bits(x), group=K, qtype=qt, scale_fmt=sfmt)
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("layout", ["row", "col"])
def test_quant_per_token_scale_layouts(bfq, orc, layout):
    """Per-token scales land at s[m * ld] (row-major, padded ld) or s[m] (column-major)."""
    M, K = 45, 1536
    x = synth.activations(M, K, seed=8)
    lay = bfq.BFQ_SCALES_ROW_MAJOR if layout == "row" else bfq.BFQ_SCALES_COL_MAJOR
    q = torch.full((M, K), 0x55, dtype=torch.uint8, device=DEV)
    if layout == "row":
        s = torch.full((M, 3), float("nan"), device=DEV)
    else:
        s = torch.full((1, M + 5), float("nan"), device=DEV)
    bfq.bfq_quant_tokens(x.to(DEV), q, s, layout=lay, scale_ld=s.stride(0), group_size=K)
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(synth.bf16_bits(x), group=K)
    got = s[:, 0] if layout == "row" else s[0, :M]
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), so[:, 0].view(np.uint32))
    rest = s[:, 1:] if layout == "row" else s[0, M:]
    assert torch.isnan(rest).all()          # nothing written past the scales


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_per_token_special_values(bfq, orc, qname, sfmt):
    """Rows with zeros, NaN, +-Inf, bf16 subnormals, max-finite and sub-eps values."""
    from test_gpu_quant import _special_input
    bits = _special_input()
    M, K = bits.shape
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    q, s = bfq.quant_tokens(x.to(DEV), q_dtype=qd, scale_fmt=sfmt, per_token=True)
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(bits, group=K, qtype=qt, scale_fmt=sfmt)
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))
    sg = s.cpu().numpy()
    assert np.array_equal(np.isnan(sg), np.isnan(so))
    assert np.array_equal(sg[~np.isnan(sg)].view(np.uint32), so[~np.isnan(so)].view(np.uint32))


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("N,K", [(256, 384), (1536, 7168), (7168, 18432), (24576, 7168),
                                 (128, 32768)])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_per_channel_bit_exact(bfq, orc, N, K, qname, sfmt):
    if N * K > 50_000_000 and qname == "int8":
        pytest.skip("the large shapes are covered by the fp8 case")
    print(f"quant per-channel N={N} K={K} {qname} sfmt={sfmt}", flush=True)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    w = synth.weights(N, K, seed=N + K)
    q, s = bfq.quant_weight_blocks(w.to(DEV), q_dtype=qd, scale_fmt=sfmt, per_channel=True)
    torch.cuda.synchronize()
    qo, so = orc.quant_blocks(w.numpy(), block=(1, K), qtype=qt, scale_fmt=sfmt)
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so[:, 0].view(np.uint32))


def test_quant_per_channel_special_values(bfq, orc):
    w = synth.weights(256, 512, seed=2).numpy().copy()
    w[0] = 0.0
    w[5, 130] = np.nan
    w[200, 7] = np.inf
    w[201, 8] = -np.inf
    w[130] *= 1e-30
    q, s = bfq.quant_weight_blocks(torch.from_numpy(w).to(DEV), per_channel=True)
    torch.cuda.synchronize()
    qo, so = orc.quant_blocks(w, block=(1, 512))
    assert np.array_equal(q.cpu().numpy(), qo)
    sg, so = s.cpu().numpy(), so[:, 0]
    assert np.array_equal(np.isnan(sg), np.isnan(so))
    assert np.array_equal(sg[~np.isnan(sg)].view(np.uint32), so[~np.isnan(so)].view(np.uint32))


# ------------------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_every_channel_candidate_and_split(bfq, orc, qname, layout):
    """Every per-channel kernel x split_k {1, 2, 3} x out dtype, on a shape spanning several
    tiles with ragged M."""
    from oracle import metrics
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    M, N, K = 83, 640, 768
    host = _host_case(orc, M, N, K, 91, qt)
    ref32, _ = orc.channel_gemm(*host, qtype=qt)
    dq = _to_dev(bfq, *host, layout)
    cands = _candidates(bfq, qd, layout, K)
    assert cands
    for t in cands:
        for s in (1, 2, 3):
            if t.variant == 2 and s > 1:
                continue
            tile = _with_split(t, s)
            what = (qname, layout, tile.as_dict())
            print("candidate", what, flush=True)
            o32 = _run(bfq, dq, torch.float32, tile=tile).cpu().numpy()
            r = metrics.gemm_fp32_report(o32, ref32)
            assert r["ok"], (what, r)
            o16 = _run(bfq, dq, torch.bfloat16, tile=tile).view(torch.int16).cpu().numpy()
            assert np.array_equal(o16.view(np.uint16), orc.f32_to_bf16_bits_array(o32)), what
            oh = _run(bfq, dq, torch.float16, tile=tile).float().cpu().numpy()
            assert np.array_equal(oh, torch.from_numpy(o32).half().float().numpy()), what


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_channel_exact_integer_case(bfq, orc, qname, layout):
    """Integer codes |v| <= 8, token scales 2^-(m mod 3), channel scales 2^-(n mod 4): every
    kernel and split must give the integer matmul times the two powers of two bit for bit
    (scales differing per row and per column pin their indexing)."""
    rng = np.random.default_rng(92)
    M, N, K = 45, 384, 1024
    ia = rng.integers(-8, 9, size=(M, K))
    iw = rng.integers(-8, 9, size=(N, K))
    if qname == "fp8":
        qd = bfq.BFQ_E4M3FN
        enc = {int(v): torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
               for v in range(-8, 9)}
        qa = np.vectorize(enc.get)(ia).astype(np.uint8)
        qw = np.vectorize(enc.get)(iw).astype(np.uint8)
    else:
        qd = bfq.BFQ_INT8
        qa, qw = ia.astype(np.int8), iw.astype(np.int8)
    ea, ew = -(np.arange(M) % 3), -(np.arange(N) % 4)
    sa = (2.0 ** ea).astype(np.float32)
    sw = (2.0 ** ew).astype(np.float32)
    exact = (ia.astype(np.int64) @ iw.T.astype(np.int64)).astype(np.float64)
    exact *= (2.0 ** ea)[:, None] * (2.0 ** ew)[None, :]
    assert np.array_equal(orc.channel_gemm(qa, sa, qw, sw, qtype=orc.FP8 if qname == "fp8"
                                           else orc.INT8)[0].astype(np.float64), exact)
    dq = _to_dev(bfq, qa, sa, qw, sw, layout)
    for t in _candidates(bfq, qd, layout, K):
        for s in (1, 4):
            if t.variant == 2 and s > 1:
                continue
            tile = _with_split(t, s)
            o32 = _run(bfq, dq, torch.float32, tile=tile).cpu().numpy().astype(np.float64)
            assert np.array_equal(o32, exact), (qname, layout, tile.as_dict())


@pytest.mark.parametrize("layout", LAYOUTS)
def test_channel_column_major_token_scales(bfq, orc, layout):
    """Per-token scales given column-major ([1][ld >= M], padded) select the same values."""
    from oracle import metrics
    M, N, K = 50, 512, 1024
    host = _host_case(orc, M, N, K, 93, orc.FP8)
    ref32, _ = orc.channel_gemm(*host)
    dq = _to_dev(bfq, *host, layout)
    sa_col = torch.full((1, M + 3), float("nan"), device=DEV)
    sa_col[0, :M] = dq[1][:, 0]
    sa_row = torch.full((M, 4), float("nan"), device=DEV)
    sa_row[:, 0] = dq[1][:, 0]
    for t in [None] + _candidates(bfq, bfq.BFQ_E4M3FN, layout, K):
        what = (layout, None if t is None else t.as_dict())
        o = _run(bfq, dq, torch.float32, tile=t, a_layout=bfq.BFQ_SCALES_COL_MAJOR,
                 sa_override=sa_col)
        assert metrics.gemm_fp32_report(o.cpu().numpy(), ref32)["ok"], what
        o = _run(bfq, dq, torch.float32, tile=t, sa_override=sa_row)
        assert metrics.gemm_fp32_report(o.cpu().numpy(), ref32)["ok"], what


@pytest.mark.parametrize("layout", LAYOUTS)
def test_channel_int8_large_sums(bfq, orc, layout):
    """int8 codes of one sign make whole-K sums beyond 2^24 (K = 7168): the kernels keep the
    sum exact in int32 and round once, like the oracle (fp32 bar, expected ~1e-7)."""
    from oracle import metrics
    rng = np.random.default_rng(94)
    M, N, K = 40, 256, 7168
    qa = rng.integers(60, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(60, 128, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.5, 2.0, M).astype(np.float32)
    sw = rng.uniform(0.5, 2.0, N).astype(np.float32)
    ref32, _ = orc.channel_gemm(qa, sa, qw, sw, qtype=orc.INT8)
    dq = _to_dev(bfq, qa, sa, qw, sw, layout)
    for t in _candidates(bfq, bfq.BFQ_INT8, layout, K):
        o = _run(bfq, dq, torch.float32, tile=t).cpu().numpy()
        r = metrics.gemm_fp32_report(o, ref32)
        assert r["ok"] and r["rel_frobenius"] < 1e-6, (layout, t.as_dict(), r)


# ------------------------------------------------------------- full-size workloads

CHANNEL_CONFIGS = ([("fp8", m, 24576, 7168) for m in (1, 16, 64, 256, 1024, 4096)]
                   + [("fp8", 4096, 7168, 18432), ("fp8", 64, 18432, 7168), ("fp8", 8, 1536, 1536)]
                   + [("int8", m, 1536, 7168) for m in (1, 16, 128, 1024, 4096)])


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname,M,N,K", CHANNEL_CONFIGS)
def test_channel_config_sampled(bfq, orc, qname, M, N, K, layout):
    """The workloads in the per-token x per-channel format at their real sizes: quantized on
    the device (checked bit-exact against the oracle), the GEMM through the tile the library
    selects, sampled outputs against the oracle, bf16 the rounding of the same fp32."""
    from oracle import metrics
    print(f"channel config {qname} M={M} N={N} K={K} {layout}", flush=True)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    x = synth.activations(M, K, seed=0)
    w = synth.weights(N, K, seed=0)
    qa, sa = bfq.quant_tokens(x.to(DEV), q_dtype=qd, per_token=True)
    qw, sw = bfq.quant_weight_blocks(w.to(DEV), q_dtype=qd, per_channel=True)
    torch.cuda.synchronize()
    qa_h, sa_h, qw_h, sw_h = qa.cpu().numpy(), sa.cpu().numpy()[:, 0], qw.cpu().numpy(), sw.cpu().numpy()
    qo, so = orc.quant_groups(synth.bf16_bits(x), group=K, qtype=qt)
    assert np.array_equal(qa_h.view(np.uint8), qo.view(np.uint8))
    assert np.array_equal(sa_h.view(np.uint32), so[:, 0].view(np.uint32))
    if layout == "packed":
        qw = bfq.pack_weights(qw)
    dq = (qa, sa, qw, sw, layout)
    o32 = _run(bfq, dq, torch.float32).cpu().numpy()
    o16 = _run(bfq, dq, torch.bfloat16).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o16, orc.f32_to_bf16_bits_array(o32))
    rng = np.random.default_rng(M * 5 + N)
    ms = np.concatenate([rng.integers(0, M, 4096), [0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 4096), [N - 1, 0]])
    ref = orc.channel_gemm_sampled(qa_h, sa_h, qw_h, sw_h, ms, ns, qtype=qt)
    r = metrics.gemm_fp32_report(o32[ms, ns], ref)
    assert r["ok"], (qname, M, N, K, layout, r)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_channel_batch_invariant_rows_bitwise(bfq, orc, qname, layout):
    """Batch-invariant mode with per-channel scales: rows of the first M tokens bitwise equal
    to those of the 600-token run, across every tile bracket the mode selects."""
    from oracle import metrics
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    M_all, N, K = 600, 1536, 3072
    host = _host_case(orc, M_all, N, K, 95, qt)
    dq = _to_dev(bfq, *host, layout)
    bfq.bfq_set_batch_invariant(True)
    try:
        for odt in (torch.float32, torch.bfloat16):
            full = _run(bfq, dq, odt)
            for M in (1, 9, 16, 17, 40, 64, 65, 100, 128, 129, 300, 512, 513):
                sub = (dq[0][:M], dq[1][:M], dq[2], dq[3], layout)
                got = _run(bfq, sub, odt)
                assert torch.equal(got.view(torch.int16) if odt == torch.bfloat16 else got.view(torch.int32),
                                   (full[:M].view(torch.int16) if odt == torch.bfloat16
                                    else full[:M].view(torch.int32))), (qname, layout, odt, M)
        ref32, _ = orc.channel_gemm(*host, qtype=qt)
        o = _run(bfq, dq, torch.float32).cpu().numpy()
        assert metrics.gemm_fp32_report(o, ref32)["ok"]
    finally:
        bfq.bfq_set_batch_invariant(False)
