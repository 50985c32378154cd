"""GPU parity of the block-scaled GEMM (through the C-ABI) against the CPU oracle.

Bar (see oracle/metrics.py):
  fp32 output vs the oracle's fp32 accumulator: rel. Frobenius <= 1e-3 and
  max |diff| <= 2^-7 * rms(ref) + 1e-3;
  bf16 output: bit-exact bf16 rounding of the GPU's own fp32 output for the same tile,
  plus the straddle reading against the oracle's bf16 output;
  exact-integer inputs: fp32 output bit-exact; int8 block partials bit-exact.
Kernels are checked with the weights row-major and packed (the packing done on the device
by bfq_pack_weights, itself checked byte for byte against the oracle's pack16), and with
UE8M0 (power-of-two) scales, where the block-scaled-MFMA tiles (sched 3) also run.
"""
import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LAYOUTS = ["row", "packed"]


def _case(orc, M, N, K, seed, qtype, sfmt=0):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed + 1).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), qtype=qtype, scale_fmt=sfmt)
    qw, sw = orc.quant_blocks(w, qtype=qtype, scale_fmt=sfmt)
    return qa, sa, qw, sw


def _to_dev(qa, sa, qw, sw, layout="row", sfmt=0):
    """Device copies; with layout "packed" the weight codes are packed on the device. sfmt is
    the scale format the GEMM is told (1: every scale a power of two)."""
    from block_scaled_w8a8_amd import bfq
    qw_d = torch.from_numpy(qw).to(DEV)
    if layout == "packed":
        qw_d = bfq.pack_weights(qw_d)
    return (torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV), qw_d,
            torch.from_numpy(sw).to(DEV), layout, sfmt)


def _wl(bfq, layout):
    return bfq.BFQ_W_PACKED16 if layout == "packed" else bfq.BFQ_W_ROW_MAJOR


def _run(bfq, dq, out_dtype, tile=None, a_layout=None, sa_override=None):
    qa, sa, qw, sw, wlay, sf = dq
    wl = _wl(bfq, wlay)
    M, N = qa.shape[0], qw.shape[0]
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    layout = bfq.BFQ_SCALES_ROW_MAJOR if a_layout is None else a_layout
    sa_arg = sa if sa_override is None else sa_override
    ws_bytes = bfq.bfq_gemm_workspace_bytes(M, N, qa.shape[1], tile) if tile is not None else 0
    if tile is None:
        st, t = bfq.bfq_select_tile(M, N, qa.shape[1], bfq._qdtype(qa), bfq._odtype(out),
                                    w_layout=wl, scale_fmt=sf)
        ws_bytes = bfq.bfq_gemm_workspace_bytes(M, N, qa.shape[1], t)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    bfq.bfq_block_gemm(qa, sa_arg, qw, sw, out, a_layout=layout, a_scale_ld=sa_arg.stride(0),
                       tile=tile, workspace=ws, workspace_bytes=ws_bytes, w_layout=wl,
                       scale_fmt=sf)
    torch.cuda.synchronize()
    return out


def _candidates(bfq, qd, layout="row", sfmt=0):
    wl = _wl(bfq, layout)
    return [bfq.bfq_get_tile_candidate(i, qd, wl, sfmt)
            for i in range(bfq.bfq_num_tile_candidates(qd, wl, sfmt))]


@pytest.mark.parametrize("N,K", [(128, 128), (640, 768), (1536, 7168), (24576, 7168)])
def test_pack_weights_bit_exact(bfq, orc, N, K):
    """bfq_pack_weights equals the oracle's pack16 byte for byte (the full-size shape is the
    wide up-projection's weight matrix)."""
    g = torch.Generator().manual_seed(N + K)
    w = torch.randint(0, 256, (N, K), dtype=torch.uint8, generator=g)
    got = bfq.pack_weights(w.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), orc.pack16(w.numpy()))


def _with_split(t, s):
    d = t.as_dict()
    d["split_k"] = s
    return type(t).from_dict(d)


def _check_fp32(orc_metrics, out, ref, what):
    r = orc_metrics.gemm_fp32_report(out, ref)
    assert r["ok"], (what, r)


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_sampled(bfq, orc, seed):
    """Seeded random shapes (M in [1, 700), N and K random multiples of 128, so M and N end in
    ragged tiles of every kernel family), both weight layouts, both scale formats and both
    code types: the library's own tile choice and a random compiled candidate with a random
    split, fp32 out, sampled against the oracle."""
    from oracle import metrics
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.integers(1, 700))
    N = 128 * int(rng.integers(1, 25))
    K = 128 * int(rng.integers(1, 33))
    layout, sfmt = LAYOUTS[seed % 2], (seed // 2) % 2
    qname = "int8" if seed >= 6 else "fp8"
    qd = bfq.BFQ_INT8 if qname == "int8" else bfq.BFQ_E4M3FN
    qt = orc.INT8 if qname == "int8" else orc.FP8
    print(f"random shape M={M} N={N} K={K} {layout} sfmt={sfmt} {qname}", flush=True)
    host = _case(orc, M, N, K, 31 + seed, qt, sfmt)
    dq = _to_dev(*host, layout=layout, sfmt=sfmt)
    ms = np.concatenate([rng.integers(0, M, 400), [0, M - 1, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 400), [0, N - 1, 0]])
    ref = orc.block_gemm_sampled(*host, ms, ns, qtype=qt)
    cands = _candidates(bfq, qd, layout, sfmt)
    t = cands[int(rng.integers(0, len(cands)))]
    split = 1 if t.variant == 2 else int(rng.integers(1, min(4, K // 128) + 1))
    for tile in (None, _with_split(t, split)):
        what = (M, N, K, layout, sfmt, qname, tile.as_dict() if tile is not None else "selected")
        o = _run(bfq, dq, torch.float32, tile=tile).cpu().numpy()
        r = metrics.gemm_fp32_report(o[ms, ns], ref)
        assert r["ok"], (what, r)


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_every_candidate_and_split_parity(bfq, orc, qname, layout, sfmt):
    """Every compiled kernel x split_k {1, 2, 3} x out dtype on a shape spanning several
    tiles with ragged M (multiple tiles in N, K = 6 blocks so 3 splits are uneven-free),
    for plain fp32 scales and for UE8M0 scales (every kernel that serves them)."""
    from oracle import metrics
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    M, N, K = 83, 640, 768
    host = _case(orc, M, N, K, 21, qt, sfmt)
    ref32, ref16 = orc.block_gemm(*host, qtype=qt)
    dq = _to_dev(*host, layout=layout, sfmt=sfmt)
    cands = _candidates(bfq, qd, layout, sfmt)
    assert cands, (qname, layout)
    for t in cands:
        for s in (1, 2, 3):
            if t.variant == 2 and s > 1:        # stream-K splits K by itself
                continue
            tile = _with_split(t, s)
            what = (qname, layout, sfmt, tile.as_dict())
            print("candidate", what, flush=True)
            o32 = _run(bfq, dq, torch.float32, tile=tile).cpu().numpy()
            _check_fp32(metrics, o32, ref32, what)
            o16 = _run(bfq, dq, torch.bfloat16, tile=tile)
            o16b = o16.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(o16b, orc.f32_to_bf16_bits_array(o32)), what
            r = metrics.bf16_straddle_report(o16b, ref16, o32, ref32)
            assert r["ok"], (what, r)
            oh = _run(bfq, dq, torch.float16, tile=tile).float().cpu().numpy()
            ref_h = torch.from_numpy(o32).half().float().numpy()
            assert np.array_equal(oh, ref_h), what


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_streamk_segments_and_determinism(bfq, orc, qname, layout, sfmt):
    """Stream-K (variant 2) with few tiles and many K blocks: at M=300, N=640, K=896 a 256x256
    tile grid has 6 tiles of 7 blocks, so 42 one-block segments land on 42 workgroups and
    every tile is summed from 7 parked partials; fp32 within the bar of the oracle, bf16 the
    rounding of the same run's fp32, and two runs bit-identical (the segment sum order does
    not depend on which workgroup arrives last)."""
    from oracle import metrics
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    M, N, K = 300, 640, 896
    host = _case(orc, M, N, K, 25, qt, sfmt)
    ref32, _ = orc.block_gemm(*host, qtype=qt)
    dq = _to_dev(*host, layout=layout, sfmt=sfmt)
    sk = [t for t in _candidates(bfq, qd, layout, sfmt) if t.variant == 2]
    assert sk, "no stream-K kernel compiled for " + qname
    for t in sk:
        what = (qname, layout, t.as_dict())
        print("stream-K", what, flush=True)
        o32a = _run(bfq, dq, torch.float32, tile=t).cpu().numpy()
        _check_fp32(metrics, o32a, ref32, what)
        o32b = _run(bfq, dq, torch.float32, tile=t).cpu().numpy()
        assert np.array_equal(o32a.view(np.uint32), o32b.view(np.uint32)), what
        o16 = _run(bfq, dq, torch.bfloat16, tile=t).view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(o16, orc.f32_to_bf16_bits_array(o32a)), what


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(2304, 7680, 1024), (5120, 7680, 512)])
def test_streamk_large_sampled(bfq, orc, M, N, K, layout):
    """Stream-K at grid-filling sizes, sampled against the oracle: 270 tiles of 256x256 (all
    split over the grid) and 600 tiles (256 taken whole, 344 split)."""
    for t in [t for t in _candidates(bfq, bfq.BFQ_E4M3FN, layout) if t.variant == 2]:
        print("stream-K", M, N, K, layout, t.as_dict(), flush=True)
        _sampled_check(bfq, orc, M, N, K, M, "fp8", n_samples=2048, tile=t, layout=layout)


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_exact_integer_case_every_candidate(bfq, orc, qname, layout, sfmt):
    """P6 on the device: integer-valued codes with |v| <= 8 and power-of-two scales make
    every partial exact, so the fp32 output must equal the integer matmul bit for bit for
    every kernel and split."""
    rng = np.random.default_rng(4)
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
    sa = np.full((M, K // 128), 2.0 ** -3, dtype=np.float32)
    sw = np.full((N // 128, K // 128), 2.0 ** -5, dtype=np.float32)
    exact = (ia.astype(np.int64) @ iw.T.astype(np.int64)).astype(np.float64) * 2.0 ** -8
    dq = _to_dev(qa, sa, qw, sw, layout=layout, sfmt=sfmt)   # the scales are powers of two
    for t in _candidates(bfq, qd, layout, sfmt):
        for s in (1, 4):
            if t.variant == 2 and s > 1:
                continue
            tile = _with_split(t, s)
            o32 = _run(bfq, dq, torch.float32, tile=tile).cpu().numpy().astype(np.float64)
            assert np.array_equal(o32, exact), (qname, layout, sfmt, tile.as_dict())


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_one_hot_rows_pin_layout(bfq, orc, layout, sfmt):
    """A token row holding code 1.0 at one column reproduces that weight column times its
    block scale (fp32 product) on every kernel: pins the row/column/K index mapping."""
    M, N, K = 20, 256, 512
    host = _case(orc, 1, N, K, 31, orc.FP8, sfmt)
    qw, sw = host[2], host[3]
    ks = [(m * 37 + 5) % K for m in range(M)]
    qa = np.zeros((M, K), dtype=np.uint8)
    for m, k in enumerate(ks):
        qa[m, k] = 0x38
    sa = np.ones((M, K // 128), dtype=np.float32)
    deq = torch.from_numpy(qw).view(torch.float8_e4m3fn).float().numpy()
    want = np.stack([deq[:, k] * np.repeat(sw[:, k // 128], 128) for k in ks]).astype(np.float32)
    dq = _to_dev(qa, sa, qw, sw, layout=layout, sfmt=sfmt)
    for t in _candidates(bfq, bfq.BFQ_E4M3FN, layout, sfmt):
        o32 = _run(bfq, dq, torch.float32, tile=t).cpu().numpy()
        assert np.array_equal(o32, want), (layout, sfmt, t.as_dict())


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 1536, 7168), (130, 1536, 7168),
                                   (1024, 1536, 7168), (4096, 1536, 7168)])
def test_int8_block_partials_bit_exact(bfq, orc, M, N, K):
    """P7 on the device: per-K-block int32 partials equal the oracle's exactly."""
    host = _case(orc, M, N, K, 41, orc.INT8)
    qa, qw = host[0], host[2]
    if M * N * (K // 128) > 60_000_000:
        qa = qa[:256]
        M = 256
    part = torch.empty((K // 128, M, N), dtype=torch.int32, device=DEV)
    bfq.bfq_debug_block_partials_i32(torch.from_numpy(qa).to(DEV), torch.from_numpy(qw).to(DEV), part)
    torch.cuda.synchronize()
    assert np.array_equal(part.cpu().numpy(), orc.block_partials_i32(qa, qw))


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_column_major_scales_and_padded_ld(bfq, orc, layout, sfmt):
    from oracle import metrics
    M, N, K = 50, 512, 1024
    host = _case(orc, M, N, K, 51, orc.FP8, sfmt)
    ref32, _ = orc.block_gemm(*host)
    dq = _to_dev(*host, layout=layout, sfmt=sfmt)
    sa = dq[1]
    sa_col = torch.full((K // 128, M + 3), float("nan"), device=DEV)
    sa_col[:, :M] = sa.t()
    for t in _candidates(bfq, bfq.BFQ_E4M3FN, layout, sfmt):
        o = _run(bfq, dq, torch.float32, tile=t, a_layout=bfq.BFQ_SCALES_COL_MAJOR,
                 sa_override=sa_col)
        _check_fp32(metrics, o.cpu().numpy(), ref32, (layout, t.as_dict()))
    sa_pad = torch.full((M, K // 128 + 4), float("nan"), device=DEV)
    sa_pad[:, :K // 128] = sa
    o = _run(bfq, dq, torch.float32, sa_override=sa_pad)
    _check_fp32(metrics, o.cpu().numpy(), ref32, "padded ld")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_nan_input_propagates_to_its_row(bfq, orc, layout):
    """A NaN activation gives its group a NaN scale; the whole output row is NaN, other
    rows are unaffected (oracle and GPU agree on which outputs are NaN)."""
    M, N, K = 8, 256, 512
    x = synth.activations(M, K, seed=61)
    bits = synth.bf16_bits(x).copy()
    bits[3, 300] = 0x7FC0
    qa, sa = orc.quant_groups(bits)
    qw, sw = orc.quant_blocks(synth.weights(N, K, seed=62).numpy())
    ref32, _ = orc.block_gemm(qa, sa, qw, sw)
    dq = _to_dev(qa, sa, qw, sw, layout=layout)
    for t in [None] + _candidates(bfq, bfq.BFQ_E4M3FN, layout):
        o = _run(bfq, dq, torch.float32, tile=t).cpu().numpy()
        what = (layout, None if t is None else t.as_dict())
        assert np.array_equal(np.isnan(o), np.isnan(ref32)), what
        assert np.isnan(o[3]).all() and not np.isnan(np.delete(o, 3, 0)).any(), what


def test_m0_no_launch(bfq):
    qw = torch.zeros((256, 256), dtype=torch.uint8, device=DEV)
    sw = torch.ones((2, 2), dtype=torch.float32, device=DEV)
    qa = torch.empty((0, 256), dtype=torch.uint8, device=DEV)
    sa = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    out = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    st = bfq.bfq_block_gemm(qa, sa, qw, sw, out, a_scale_ld=2)
    assert st >= 0


@pytest.mark.parametrize("layout", LAYOUTS)
def test_deterministic_run_twice(bfq, orc, layout):
    M, N, K = 64, 1536, 7168
    dq = _to_dev(*_case(orc, M, N, K, 71, orc.FP8), layout=layout)
    for t in _candidates(bfq, bfq.BFQ_E4M3FN, layout):
        tile = _with_split(t, 1 if t.variant == 2 else 4)
        a = _run(bfq, dq, torch.float32, tile=tile)
        b = _run(bfq, dq, torch.float32, tile=tile)
        assert torch.equal(a, b), t.as_dict()


# ------------------------------------------------------------- full-size configs
# The five workloads at their real sizes, through the product path (tile selected by the
# library), on sampled outputs the oracle computes one by one.

CONFIGS = {
    "tiny": [(8, 1536, 1536)],
    "decode": [(m, n, k) for (n, k) in [(7168, 1536), (1536, 7168)]
               for m in (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128)],
    "mgrid": [(m, 24576, 7168) for m in (1, 2, 4, 8, 16, 24, 32, 48, 64, 96, 128, 256, 512,
                                         1024, 1536, 2048, 3072, 4096)],
    "dense": [(m, n, k) for (n, k) in [(4096, 7168), (7168, 18432), (18432, 7168)]
              for m in (8, 64, 128, 4096)],
}

_cache = {}


def _full_inputs(bfq, N, K, m_max, qname, sfmt=0):
    key = (N, K, m_max, qname, sfmt)
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
        x = synth.activations(m_max, K, seed=0)
        w = synth.weights(N, K, seed=0)
        xd, wd = x.to(DEV), w.to(DEV)
        qw, sw = bfq.quant_weight_blocks(wd, q_dtype=qd, scale_fmt=sfmt)
        qa, sa = bfq.quant_tokens(xd, q_dtype=qd, scale_fmt=sfmt)
        # the timed layout: the quantizer writes the scales column-major, ld = m_max
        qa_c, sa_col = bfq.quant_tokens(xd, q_dtype=qd, scale_fmt=sfmt,
                                        layout=bfq.BFQ_SCALES_COL_MAJOR)
        qwp = bfq.pack_weights(qw)
        torch.cuda.synchronize()
        assert torch.equal(qa_c, qa) and torch.equal(sa_col.t().view(torch.int32),
                                                     sa.view(torch.int32))
        del wd, qa_c
        _cache[key] = (qa, sa, qw, sw, qa.cpu().numpy(), sa.cpu().numpy(), qw.cpu().numpy(),
                       sw.cpu().numpy(), qwp, sa_col)
    return _cache[key]


def _sampled_check(bfq, orc, M, N, K, m_max, qname, n_samples=4096, tile=None, layout="row",
                   sfmt=0, scale_layout="row"):
    """scale_layout "col": the activation scales column-major with ld = m_max, as the
    benchmark lays them out (every M reads the first M columns of one [K/128, m_max] array)."""
    from oracle import metrics
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    qa, sa, qw, sw, qa_h, sa_h, qw_h, sw_h, qwp, sa_col = _full_inputs(bfq, N, K, m_max, qname,
                                                                       sfmt)
    wl = _wl(bfq, layout)
    if scale_layout == "col":
        a_lay, sa_arg = bfq.BFQ_SCALES_COL_MAJOR, sa_col
    else:
        a_lay, sa_arg = bfq.BFQ_SCALES_ROW_MAJOR, sa[:M]
    qw_arg = qwp if layout == "packed" else qw
    # NaN-prefilled, so an element a tile fails to write cannot pass on stale memory
    out32 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    out16 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    if tile is None:
        st, tile = bfq.bfq_select_tile(M, N, K, bfq._qdtype(qa), bfq.BFQ_FP32, w_layout=wl,
                                       scale_fmt=sfmt)
    ws_bytes = bfq.bfq_gemm_workspace_bytes(M, N, K, tile)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    bfq.bfq_block_gemm(qa[:M], sa_arg, qw_arg, sw, out32, tile=tile, workspace=ws,
                       workspace_bytes=ws_bytes, w_layout=wl, scale_fmt=sfmt, a_layout=a_lay)
    bfq.bfq_block_gemm(qa[:M], sa_arg, qw_arg, sw, out16, tile=tile, workspace=ws,
                       workspace_bytes=ws_bytes, w_layout=wl, scale_fmt=sfmt, a_layout=a_lay)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M * 7 + N)
    ms = np.concatenate([rng.integers(0, M, n_samples), [0, M - 1, M - 1]])
    ns = np.concatenate([rng.integers(0, N, n_samples), [0, N - 1, 0]])
    ref = orc.block_gemm_sampled(qa_h[:M], sa_h[:M], qw_h, sw_h, ms, ns, qtype=qt)
    o32 = out32.cpu().numpy()
    got = o32[ms, ns]
    r = metrics.gemm_fp32_report(got, ref)
    assert r["ok"], (M, N, K, layout, sfmt, scale_layout, tile.as_dict(), r)
    o16 = out16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o16, orc.f32_to_bf16_bits_array(o32)), (M, N, K)
    # quantized inputs were produced on the device: they must equal the oracle's
    if M == m_max:
        x = synth.activations(m_max, K, seed=0)
        qo, so = orc.quant_groups(synth.bf16_bits(x), qtype=qt, scale_fmt=sfmt)
        assert np.array_equal(qa_h.view(np.uint8), qo.view(np.uint8))
        assert np.array_equal(sa_h.view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", CONFIGS["tiny"] + CONFIGS["decode"])
def test_config_tiny_and_decode(bfq, orc, M, N, K, layout):
    print(f"config M={M} N={N} K={K} {layout}", flush=True)
    _sampled_check(bfq, orc, M, N, K, 128 if M > 8 or N != 1536 or K != 1536 else 8, "fp8",
                   layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", CONFIGS["mgrid"])
def test_config_mgrid(bfq, orc, M, N, K, layout):
    print(f"config M={M} N={N} K={K} {layout}", flush=True)
    _sampled_check(bfq, orc, M, N, K, 4096, "fp8", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", CONFIGS["dense"])
def test_config_dense(bfq, orc, M, N, K, layout):
    print(f"config M={M} N={N} K={K} {layout}", flush=True)
    _sampled_check(bfq, orc, M, N, K, 4096, "fp8", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M", [1, 16, 128, 1024, 4096])
def test_config_int8(bfq, orc, M, layout):
    print(f"config int8 M={M} {layout}", flush=True)
    _sampled_check(bfq, orc, M, 1536, 7168, 4096, "int8", layout=layout)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(m, 24576, 7168) for m in (1, 64, 256, 1024, 2048, 4096)]
                         + [(4096, 7168, 18432), (4096, 18432, 7168), (8, 1536, 1536)])
def test_config_ue8m0(bfq, orc, M, N, K, layout):
    """The workloads with UE8M0 scales (quantized on the device in that format, the GEMM told
    so), through the tile the library selects: block-scaled-MFMA tiles at large M."""
    print(f"config ue8m0 M={M} N={N} K={K} {layout}", flush=True)
    _sampled_check(bfq, orc, M, N, K, 4096 if M > 8 else 8, "fp8", layout=layout, sfmt=1)


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_batch_invariant_mode_rows_bitwise(bfq, orc, qname, layout, sfmt):
    """Batch-invariant mode (config page §5): the output rows of the first M tokens are
    bitwise the same whatever M is — across every tile bracket the mode selects (swap-AB,
    LDS-shared tokens, 64x128, 128x128, 256x256) — and within the parity bar of the oracle."""
    from oracle import metrics
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    M_all, N, K = 600, 1536, 3072
    host = _case(orc, M_all, N, K, 91, qt, sfmt)
    ref32, _ = orc.block_gemm(*host, qtype=qt)
    qa, sa, qw, sw, wlay, sf = _to_dev(*host, layout=layout, sfmt=sfmt)
    bfq.bfq_set_batch_invariant(True)
    try:
        full = _run(bfq, (qa, sa, qw, sw, wlay, sf), torch.float32).cpu().numpy()
        _check_fp32(metrics, full, ref32, (qname, layout, sfmt, "M=600"))
        full16 = _run(bfq, (qa, sa, qw, sw, wlay, sf), torch.bfloat16).view(torch.int16).cpu().numpy()
        for M in (1, 9, 16, 17, 40, 64, 65, 100, 128, 129, 300, 512, 513):
            st, t = bfq.bfq_select_tile(M, N, K, qd, bfq.BFQ_FP32, w_layout=_wl(bfq, layout),
                                        scale_fmt=sfmt)
            print("batch-invariant", qname, layout, sfmt, M, t.as_dict(), flush=True)
            dq = (qa[:M], sa[:M], qw, sw, wlay, sf)
            o = _run(bfq, dq, torch.float32).cpu().numpy()
            assert np.array_equal(o.view(np.uint32), full[:M].view(np.uint32)), (M, t.as_dict())
            o16 = _run(bfq, dq, torch.bfloat16).view(torch.int16).cpu().numpy()
            assert np.array_equal(o16, full16[:M]), (M, t.as_dict())
    finally:
        bfq.bfq_set_batch_invariant(False)


# ------------------------------------------------ packed UE8M0 activation-scale words

def _to_packed_words(bfq, sa_dev, M, ld=None):
    """Device words [ceil(G/4), ld] from device UE8M0 scales [M, G] (the oracle's packing)."""
    import oracle
    ld = ld or (M + 3) // 4 * 4
    w = oracle.pack_scales_ue8m0(sa_dev.cpu().numpy(), ld=ld)
    return torch.from_numpy(w.view(np.int32)).to(DEV)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_packed_scale_words_every_candidate(bfq, orc, layout):
    """Every fp8 kernel that serves UE8M0 scales, and every split, gives bitwise the same
    output with the activation scales as packed words as with the same scales column-major
    in fp32 (the decoded values are identical), and meets the bar against the oracle."""
    from oracle import metrics
    M, N, K = 83, 640, 768
    host = _case(orc, M, N, K, 23, orc.FP8, 1)
    ref32, _ = orc.block_gemm(*host)
    dq = _to_dev(*host, layout=layout, sfmt=1)
    words = _to_packed_words(bfq, dq[1], M, ld=M + 5)
    sa_col = dq[1].t().contiguous()
    for t in _candidates(bfq, bfq.BFQ_E4M3FN, layout, 1):
        for s in (1, 3):
            if t.variant == 2 and s > 1:
                continue
            tile = _with_split(t, s)
            what = (layout, tile.as_dict())
            print("packed", what, flush=True)
            for odt in (torch.float32, torch.bfloat16):
                col = _run(bfq, dq, odt, tile=tile, a_layout=bfq.BFQ_SCALES_COL_MAJOR,
                           sa_override=sa_col)
                pk = _run(bfq, dq, odt, tile=tile, a_layout=bfq.BFQ_SCALES_PACKED_UE8M0,
                          sa_override=words)
                assert torch.equal(pk.view(torch.int16) if odt == torch.bfloat16 else pk.view(torch.int32),
                                   col.view(torch.int16) if odt == torch.bfloat16 else col.view(torch.int32)), (what, odt)
                if odt == torch.float32:
                    _check_fp32(metrics, pk.cpu().numpy(), ref32, what)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(m, 24576, 7168) for m in (1, 16, 64, 256, 2048, 4096)]
                         + [(8, 1536, 1536), (4096, 7168, 18432)])
def test_packed_scale_words_configs(bfq, orc, M, N, K, layout):
    """The workloads with the quantizer writing packed words and the GEMM reading them
    (tile selected by the library), sampled against the oracle."""
    from oracle import metrics
    print(f"packed config M={M} N={N} K={K} {layout}", flush=True)
    x = synth.activations(M, K, seed=0)
    w = synth.weights(N, K, seed=0)
    qw, sw = bfq.quant_weight_blocks(w.to(DEV), scale_fmt=bfq.BFQ_SCALE_UE8M0)
    if layout == "packed":
        qw = bfq.pack_weights(qw)
    qa, words = bfq.quant_tokens(x.to(DEV), layout=bfq.BFQ_SCALES_PACKED_UE8M0,
                                 scale_fmt=bfq.BFQ_SCALE_UE8M0)
    out = bfq.block_gemm(qa, words, qw, sw, out_dtype=torch.float32,
                         a_layout=bfq.BFQ_SCALES_PACKED_UE8M0, w_layout=_wl(bfq, layout),
                         scale_fmt=bfq.BFQ_SCALE_UE8M0)
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(synth.bf16_bits(x), scale_fmt=orc.SCALE_UE8M0)
    qwo, swo = orc.quant_blocks(w.numpy(), scale_fmt=orc.SCALE_UE8M0)
    assert np.array_equal(qa.cpu().numpy(), qo)
    rng = np.random.default_rng(M + N)
    ms = np.concatenate([rng.integers(0, M, 2048), [0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 2048), [N - 1, 0]])
    ref = orc.block_gemm_sampled(qo, so, qwo, swo, ms, ns)
    r = metrics.gemm_fp32_report(out.cpu().numpy()[ms, ns], ref)
    assert r["ok"], (M, N, K, layout, r)


# ------------------------------------------------ the configuration the benchmark times
# The benchmark runs packed weights, activation scales written column-major by the quantizer
# with ld = M_max (the layout of the block GEMM benchmark page's §4.1 for CUTLASS/DeepGEMM),
# and the tuned tile of each M. These tests run exactly that, at full size, through the tile
# the library selects, sampled against the oracle.

TIMED_MGRID = [1, 64, 128, 256, 512, 1024, 1536, 2048, 3072, 4096]


@pytest.mark.parametrize("M", TIMED_MGRID)
def test_timed_config_mgrid(bfq, orc, M):
    print(f"timed config M={M} N=24576 K=7168 packed col-major ld=4096", flush=True)
    _sampled_check(bfq, orc, M, 24576, 7168, 4096, "fp8", layout="packed", scale_layout="col")


@pytest.mark.parametrize("N,K", [(7168, 18432), (18432, 7168)])
def test_timed_config_dense_4096(bfq, orc, N, K):
    print(f"timed config M=4096 N={N} K={K} packed col-major", flush=True)
    _sampled_check(bfq, orc, 4096, N, K, 4096, "fp8", layout="packed", scale_layout="col")


@pytest.mark.parametrize("N,K", [(3072, 7168), (7168, 2304)])
@pytest.mark.parametrize("M", [1, 64, 512, 4096])
def test_timed_config_tp8_shards(bfq, orc, M, N, K):
    """The per-GPU shard shapes of 8-way tensor parallelism the benchmark also times."""
    print(f"timed config M={M} N={N} K={K} packed col-major", flush=True)
    _sampled_check(bfq, orc, M, N, K, 4096, "fp8", layout="packed", scale_layout="col")


@pytest.mark.parametrize("M", [1, 128, 4096])
def test_timed_config_int8(bfq, orc, M):
    print(f"timed config int8 M={M} N=1536 K=7168 packed col-major", flush=True)
    _sampled_check(bfq, orc, M, 1536, 7168, 4096, "int8", layout="packed", scale_layout="col")


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_every_candidate_col_major_full_tiles(bfq, orc, qname, layout, sfmt):
    """Column-major activation scales with a padded ld at M = 600, which fills whole 256-row
    tiles (and ends in a ragged one): every compiled kernel and split {1, 2} against the
    oracle, so each row range of the scale staging (rows 0-255 of a tile and beyond) is read
    in the layout the benchmark uses."""
    from oracle import metrics
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    M, N, K = 600, 640, 768
    host = _case(orc, M, N, K, 27, qt, sfmt)
    ref32, _ = orc.block_gemm(*host, qtype=qt)
    dq = _to_dev(*host, layout=layout, sfmt=sfmt)
    sa_col = torch.full((K // 128, M + 7), float("nan"), device=DEV)
    sa_col[:, :M] = dq[1].t()
    for t in _candidates(bfq, qd, layout, sfmt):
        for s in (1, 2):
            if t.variant == 2 and s > 1:
                continue
            tile = _with_split(t, s)
            what = (qname, layout, sfmt, tile.as_dict())
            print("col-major candidate", what, flush=True)
            o = _run(bfq, dq, torch.float32, tile=tile, a_layout=bfq.BFQ_SCALES_COL_MAJOR,
                     sa_override=sa_col).cpu().numpy()
            _check_fp32(metrics, o, ref32, what)


# ------------------------------------------------ int8: exact partials in the product tiles

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("K", [128, 1024])
def test_int8_full_range_partials_exact_every_candidate(bfq, orc, K, layout):
    """The product int8 tiles keep each 128-wide block partial as an exact int32 (the int8
    block variant of the config page, §1): codes over the full range [-127, 127] (rows and
    columns of all +127 / -127 reach the extreme partial 128 * 127^2 = 2,064,512) with one
    power-of-two scale for every block. Every partial, every scaled partial and every running
    sum of up to 8 blocks is then an integer multiple of 2^-8 below 2^16, exact in fp32, so
    the fp32 output of every int8 kernel and split (split partials and their fixed-order sum
    included) must equal the int64 matmul times 2^-8 bit for bit."""
    rng = np.random.default_rng(K + 17)
    M, N = 83, 640
    ia = rng.integers(-127, 128, size=(M, K))
    iw = rng.integers(-127, 128, size=(N, K))
    ia[0], ia[1], iw[0], iw[1] = 127, -127, 127, -127
    exact = (ia.astype(np.int64) @ iw.T.astype(np.int64))
    assert np.abs(exact).max() == 127 * 127 * K
    exact = exact.astype(np.float64) * 2.0 ** -8
    sa = np.full((M, K // 128), 2.0 ** -3, dtype=np.float32)
    sw = np.full((N // 128, K // 128), 2.0 ** -5, dtype=np.float32)
    dq = _to_dev(ia.astype(np.int8), sa, iw.astype(np.int8), sw, layout=layout)
    cands = _candidates(bfq, bfq.BFQ_INT8, layout)
    assert cands
    for t in cands:
        for s in (1, 2, 4):
            if (t.variant == 2 and s > 1) or s > K // 128:
                continue
            tile = _with_split(t, s)
            o32 = _run(bfq, dq, torch.float32, tile=tile).cpu().numpy().astype(np.float64)
            assert np.array_equal(o32, exact), (K, layout, tile.as_dict())


# ------------------------------------------------ guard bands around outputs and workspace

SENTINEL = 0xA5


def _guarded(n_bytes, front, back):
    """A device byte buffer of front + n_bytes + back sentinel bytes; returns (buf, view)."""
    buf = torch.full((front + n_bytes + back,), SENTINEL, dtype=torch.uint8, device=DEV)
    return buf, buf[front:front + n_bytes]


def _untouched(buf, front, n_bytes):
    h = buf.cpu().numpy()
    return bool((h[:front] == SENTINEL).all() and (h[front + n_bytes:] == SENTINEL).all())


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_guard_bands_every_candidate(bfq, orc, qname, layout, odt):
    """Ragged M (83) and N (640: 2.5 tiles of 256, 3.3 of 192) for every compiled kernel with
    split {1, 3}: the output [M, N] sits inside a larger sentinel-filled buffer and the split-K
    / stream-K workspace inside one too. No byte before or after either is written, and the
    output still meets the bar against the oracle."""
    from oracle import metrics
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    M, N, K = 83, 640, 768
    host = _case(orc, M, N, K, 29, qt)
    ref32, _ = orc.block_gemm(*host, qtype=qt)
    qa, sa, qw, sw, _, _ = _to_dev(*host, layout=layout)
    esz = torch.tensor([], dtype=odt).element_size()
    front, back = 4096, 64 * 1024
    for t in _candidates(bfq, qd, layout):
        for s in (1, 3):
            if t.variant == 2 and s > 1:
                continue
            tile = _with_split(t, s)
            what = (qname, layout, str(odt), tile.as_dict())
            obuf, oview = _guarded(M * N * esz, front, back)
            out = oview.view(odt).view(M, N)
            need = bfq.bfq_gemm_workspace_bytes(M, N, K, tile)
            wbuf, wview = _guarded(max(need, 16), front, back)
            bfq.bfq_block_gemm(qa, sa, qw, sw, out, tile=tile, workspace=wview,
                               workspace_bytes=need, w_layout=_wl(bfq, layout))
            torch.cuda.synchronize()
            assert _untouched(obuf, front, M * N * esz), ("output guard", what)
            assert _untouched(wbuf, front, max(need, 16)), ("workspace guard", what)
            if odt == torch.float32:
                _check_fp32(metrics, out.cpu().numpy(), ref32, what)
