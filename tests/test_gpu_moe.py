"""GPU parity of the MoE grouped block GEMM and its routing sort (through the C-ABI) against
the CPU oracle (config page §5: MoE kernels keyed by an expert count E).

Bar: routing offsets and pair order bit-exact; grouped GEMM fp32 output within the block
GEMM's bar (rel. Frobenius <= 1e-3, max |diff| <= 2^-7 rms + 1e-3) of orc_moe_gemm, bf16 the
RNE rounding of the same tile's fp32; integer-valued inputs bit-exact.
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


def _expected_align(ids, E):
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    srt = np.argsort(key, kind="stable").astype(np.int32)
    off = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=E + 1))[:E]]).astype(np.int32)
    return off, srt


@pytest.mark.parametrize("T,E,topk", [(1, 256, 8), (37, 16, 4), (4096, 256, 8), (5000, 1023, 6),
                                      (3, 3, 1), (1500, 64, 2), (0, 8, 2)])
def test_moe_align_bit_exact(bfq, orc, T, E, topk):
    print(f"moe_align T={T} E={E} topk={topk}", flush=True)
    ids = synth.routing(max(T, 1), E, topk, seed=T + E)[:T].contiguous()
    off, srt = bfq.moe_align(ids.to(DEV), E)
    torch.cuda.synchronize()
    if T > 0:
        o_off, o_srt = orc.moe_align(ids.numpy(), E)
        assert np.array_equal(off.cpu().numpy(), o_off)
        assert np.array_equal(srt.cpu().numpy(), o_srt)
    else:
        assert (off.cpu() == 0).all()


def test_moe_align_out_of_range_ids(bfq):
    """Ids outside [0, E) go after every expert; offsets[E] counts the valid pairs."""
    ids = synth.routing(300, 32, 4, seed=5).clone()
    ids[7, 1] = -1
    ids[100, 3] = 32
    ids[299, 0] = 1 << 20
    off, srt = bfq.moe_align(ids.to(DEV), 32)
    torch.cuda.synchronize()
    e_off, e_srt = _expected_align(ids.numpy(), 32)
    assert e_off[32] == 1200 - 3
    assert np.array_equal(off.cpu().numpy(), e_off)
    assert np.array_equal(srt.cpu().numpy(), e_srt)


def _moe_host(orc, T, E, topk, N, K, seed, sfmt=0):
    x = synth.activations(T, K, seed=seed)
    ids = synth.routing(T, E, topk, seed=seed)
    w = synth.expert_weights(E, N, K, seed=seed).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), scale_fmt=sfmt)
    qs = [orc.quant_blocks(w[e], scale_fmt=sfmt) for e in range(E)]
    return qa, sa, ids.numpy(), np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def _moe_dev(bfq, qa, sa, ids, qw, sw, layout, E):
    qw_d = torch.from_numpy(qw).to(DEV)
    if layout == "packed":
        qw_d = bfq.pack_weights(qw_d)
    off, srt = bfq.moe_align(torch.from_numpy(ids).to(DEV), E)
    return (torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV), srt, off, ids.shape[1],
            qw_d, torch.from_numpy(sw).to(DEV))


def _moe_run(bfq, d, out_dtype, tile, layout, sfmt=0, a_layout=None, sa=None, fill=float("nan")):
    qa, sa0, srt, off, topk, qw, sw = d
    sa = sa0 if sa is None else sa
    T, N = qa.shape[0], qw.shape[1]
    out = torch.full((T * topk, N), fill, dtype=out_dtype, device=DEV)
    ws_bytes = bfq.bfq_moe_gemm_workspace_bytes(T, topk, N, tile) if tile is not None else 0
    if tile is None:
        _, t = bfq.bfq_moe_select_tile(T, topk, qw.shape[0], N, qa.shape[1], bfq._odtype(out),
                                       _wl(bfq, layout), sfmt)
        ws_bytes = bfq.bfq_moe_gemm_workspace_bytes(T, topk, N, t)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
    bfq.bfq_moe_block_gemm(qa, sa, srt, off, topk, qw, sw, out,
                           a_layout=bfq.BFQ_SCALES_ROW_MAJOR if a_layout is None else a_layout,
                           a_scale_ld=sa.stride(0), tile=tile, workspace=ws, workspace_bytes=ws_bytes,
                           w_layout=_wl(bfq, layout), scale_fmt=sfmt)
    torch.cuda.synchronize()
    return out


def _with_split(t, s):
    d = t.as_dict()
    d["split_k"] = s
    return type(t).from_dict(d)


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_moe_every_candidate_and_split(bfq, orc, layout, sfmt):
    """Every grouped kernel x split {1, 2} x out dtype; experts with 0, few and many rows
    (T=37 tokens, top-4 of 8 experts, N=256, K=768)."""
    from oracle import metrics
    T, E, topk, N, K = 37, 8, 4, 256, 768
    host = _moe_host(orc, T, E, topk, N, K, 51, sfmt)
    ref = orc.moe_gemm(*host)
    d = _moe_dev(bfq, *host, layout, E)
    wl = _wl(bfq, layout)
    cands = [bfq.bfq_moe_get_tile_candidate(i, wl, sfmt)
             for i in range(bfq.bfq_moe_num_tile_candidates(wl, sfmt))]
    assert cands
    for t in cands:
        for s in (1, 2):
            tile = _with_split(t, s)
            what = (layout, sfmt, tile.as_dict())
            print("moe candidate", what, flush=True)
            o32 = _moe_run(bfq, d, torch.float32, tile, layout, sfmt).cpu().numpy()
            r = metrics.gemm_fp32_report(o32, ref)
            assert r["ok"], (what, r)
            o16 = _moe_run(bfq, d, torch.bfloat16, tile, layout, sfmt)
            o16 = o16.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(o16, orc.f32_to_bf16_bits_array(o32)), what


@pytest.mark.parametrize("seed", range(6))
def test_moe_random_shapes_sampled(bfq, orc, seed):
    """Seeded random grouped problems (T in [1, 600), E in [2, 64], top-k up to 8, N and K
    random multiples of 128), both weight layouts and scale formats: the library's own tile
    choice and a random grouped candidate with a random split, sampled against the oracle."""
    from oracle import metrics
    rng = np.random.default_rng(2000 + seed)
    T = int(rng.integers(1, 600))
    E = int(rng.integers(2, 65))
    topk = int(rng.integers(1, min(8, E) + 1))
    N = 128 * int(rng.integers(1, 13))
    K = 128 * int(rng.integers(1, 17))
    layout, sfmt = LAYOUTS[seed % 2], (seed // 2) % 2
    print(f"moe random T={T} E={E} topk={topk} N={N} K={K} {layout} sfmt={sfmt}", flush=True)
    host = _moe_host(orc, T, E, topk, N, K, 61 + seed, sfmt)
    d = _moe_dev(bfq, *host, layout, E)
    qs = np.concatenate([rng.integers(0, T * topk, 400), [0, T * topk - 1]])
    ns = np.concatenate([rng.integers(0, N, 400), [N - 1, 0]])
    ref = orc.moe_gemm_sampled(*host, qs, ns)
    wl = _wl(bfq, layout)
    cands = [bfq.bfq_moe_get_tile_candidate(i, wl, sfmt)
             for i in range(bfq.bfq_moe_num_tile_candidates(wl, sfmt))]
    t = cands[int(rng.integers(0, len(cands)))]
    for tile in (None, _with_split(t, int(rng.integers(1, min(2, K // 128) + 1)))):
        what = (T, E, topk, N, K, layout, sfmt, tile.as_dict() if tile is not None else "selected")
        o = _moe_run(bfq, d, torch.float32, tile, layout, sfmt).cpu().numpy()
        r = metrics.gemm_fp32_report(o[qs, ns], ref)
        assert r["ok"], (what, r)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_moe_scale_layouts(bfq, orc, layout):
    """Column-major (padded ld) and packed UE8M0 activation scales give bitwise the result of
    row-major ones, on every grouped kernel."""
    T, E, topk, N, K = 45, 6, 2, 256, 1024
    host = _moe_host(orc, T, E, topk, N, K, 52, 1)
    d = _moe_dev(bfq, *host, layout, E)
    sa = d[1]
    sa_col = torch.full((K // 128, T + 3), float("nan"), device=DEV)
    sa_col[:, :T] = sa.t()
    words = torch.from_numpy(orc.pack_scales_ue8m0(host[1]).view(np.int32)).to(DEV)
    wl = _wl(bfq, layout)
    for t in [bfq.bfq_moe_get_tile_candidate(i, wl, 1) for i in range(bfq.bfq_moe_num_tile_candidates(wl, 1))]:
        base = _moe_run(bfq, d, torch.float32, t, layout, 1)
        col = _moe_run(bfq, d, torch.float32, t, layout, 1, a_layout=bfq.BFQ_SCALES_COL_MAJOR, sa=sa_col)
        pk = _moe_run(bfq, d, torch.float32, t, layout, 1, a_layout=bfq.BFQ_SCALES_PACKED_UE8M0, sa=words)
        assert torch.equal(base.view(torch.int32), col.view(torch.int32)), t.as_dict()
        assert torch.equal(base.view(torch.int32), pk.view(torch.int32)), t.as_dict()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_moe_exact_integer_case(bfq, orc, layout):
    """Integer codes |v| <= 8, power-of-two scales differing per expert: every grouped kernel
    gives each pair's integer product with its expert exactly."""
    rng = np.random.default_rng(53)
    T, E, topk, N, K = 29, 5, 2, 128, 512
    enc = {int(v): torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
           for v in range(-8, 9)}
    ia = rng.integers(-8, 9, size=(T, K))
    iw = rng.integers(-8, 9, size=(E, N, K))
    qa = np.vectorize(enc.get)(ia).astype(np.uint8)
    qw = np.vectorize(enc.get)(iw).astype(np.uint8)
    sa = np.full((T, K // 128), 2.0 ** -3, dtype=np.float32)
    sw = np.stack([np.full((N // 128, K // 128), 2.0 ** -(e + 1), dtype=np.float32) for e in range(E)])
    ids = synth.routing(T, E, topk, seed=53).numpy()
    exact = np.empty((T * topk, N))
    for q in range(T * topk):
        e = ids[q // topk, q % topk]
        exact[q] = (iw[e].astype(np.int64) @ ia[q // topk].astype(np.int64)) * 2.0 ** -3 * 2.0 ** -(e + 1)
    d = _moe_dev(bfq, qa, sa, ids, qw, sw, layout, E)
    wl = _wl(bfq, layout)
    for t in [bfq.bfq_moe_get_tile_candidate(i, wl, 0) for i in range(bfq.bfq_moe_num_tile_candidates(wl, 0))]:
        for s in (1, 4):
            tile = _with_split(t, s)
            o = _moe_run(bfq, d, torch.float32, tile, layout).cpu().numpy().astype(np.float64)
            assert np.array_equal(o, exact), (layout, tile.as_dict())


def test_moe_invalid_expert_rows_untouched(bfq, orc):
    """A pair routed outside [0, E) gets no row (split 1): its output row keeps its old
    contents; every other row matches the oracle with those pairs' rows ignored."""
    from oracle import metrics
    T, E, topk, N, K = 20, 4, 2, 128, 256
    qa, sa, ids, qw, sw = _moe_host(orc, T, E, topk, N, K, 54)
    ref = orc.moe_gemm(qa, sa, ids, qw, sw)
    bad = ids.copy()
    bad[3, 1] = E
    bad[11, 0] = -5
    d = _moe_dev(bfq, qa, sa, bad, qw, sw, "row", E)
    for t in [None] + [bfq.bfq_moe_get_tile_candidate(i) for i in range(bfq.bfq_moe_num_tile_candidates())]:
        o = _moe_run(bfq, d, torch.float32, t, "row", fill=7.0).cpu().numpy()
        dead = [3 * topk + 1, 11 * topk + 0]
        assert (o[dead] == 7.0).all()
        keep = np.setdiff1d(np.arange(T * topk), dead)
        assert metrics.gemm_fp32_report(o[keep], ref[keep])["ok"]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("T,N,K", [(1, 4096, 7168), (16, 4096, 7168), (128, 4096, 7168),
                                   (1024, 4096, 7168), (4096, 4096, 7168),
                                   (16, 7168, 2048), (1024, 7168, 2048)])
def test_moe_deepseek_config_sampled(bfq, orc, T, N, K, layout):
    """DeepSeek-V3 routed experts at full size (E=256, top-8; gate+up N=4096, K=7168 and the
    down projection N=7168, K=2048): tokens quantized and routed on the device, weights drawn
    and quantized on the device; outputs of pairs of three sampled experts checked against the
    oracle, which re-draws and quantizes those experts itself."""
    from oracle import metrics
    print(f"moe config T={T} N={N} K={K} {layout}", flush=True)
    E, topk = 256, 8
    x = synth.activations(T, K, seed=0)
    ids = synth.routing(T, E, topk, seed=0)
    qw = torch.empty((E, N, K), dtype=torch.uint8, device=DEV)
    sw = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=DEV)
    for e in range(E):
        q, s = bfq.quant_weight_blocks(synth.expert_weight_on(DEV, e, N, K, seed=0))
        qw[e].copy_(q)
        sw[e].copy_(s)
    if layout == "packed":
        qw = bfq.pack_weights(qw)
    qa, sa = bfq.quant_tokens(x.to(DEV))
    off, srt = bfq.moe_align(ids.to(DEV), E)
    out = bfq.moe_block_gemm(qa, sa, srt, off, topk, qw, sw, out_dtype=torch.float32,
                             w_layout=_wl(bfq, layout))
    torch.cuda.synchronize()
    flat = ids.numpy().reshape(-1)
    chosen = list(dict.fromkeys(flat[[0, len(flat) // 2, len(flat) - 1]].tolist()))
    qo, so = orc.quant_groups(synth.bf16_bits(x))
    assert np.array_equal(qa.cpu().numpy(), qo)
    sub = [orc.quant_blocks(synth.expert_weight_on(DEV, e, N, K, seed=0).cpu().numpy()) for e in chosen]
    qw_sub = np.stack([q for q, _ in sub])
    sw_sub = np.stack([s for _, s in sub])
    remap = {e: i for i, e in enumerate(chosen)}
    ids_sub = np.vectorize(lambda v: remap.get(v, 0))(ids.numpy()).astype(np.int32)
    pairs = np.nonzero(np.isin(flat, chosen))[0]
    rng = np.random.default_rng(T)
    qs = rng.choice(pairs, size=1024)
    ns = rng.integers(0, N, size=1024)
    ref = orc.moe_gemm_sampled(qo, so, ids_sub, qw_sub, sw_sub, qs, ns)
    got = out.cpu().numpy()[qs, ns]
    r = metrics.gemm_fp32_report(got, ref)
    assert r["ok"], (T, layout, r)
