"""CPU tests of the C-ABI library: it loads, exports every entry point include/bfq.h
declares, validates arguments before any launch, and selects tiles per the tile table and
the default rule. No compute call is made (no GPU here)."""
import ctypes
import json
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)


def _declared_entry_points():
    text = open(os.path.join(REPO, "include", "bfq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bfq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(bfq):
    names = _declared_entry_points()
    assert len(names) >= 12
    for n in names:
        assert hasattr(bfq.lib, n), n
    assert set(names) == set(bfq.EXPORTED)


def test_status_strings(bfq):
    for code in range(-9, 2):
        assert bfq.status_string(code).startswith("BFQ_")


BS = (ctypes.c_int32 * 2)(128, 128)
FAKE = 1 << 20          # a 16-byte aligned non-NULL address; never dereferenced here


def _gemm(bfq, **kw):
    a = dict(a_q=FAKE, a_scales=FAKE, a_layout=0, a_scale_ld=56, w_q=FAKE, w_scales=FAKE,
             w_layout=0, scale_fmt=0, out=FAKE, M=0, N=1536, K=7168, block_shape=BS,
             in_dtype=bfq.BFQ_E4M3FN,
             out_dtype=bfq.BFQ_BF16, tile=None, workspace=None, workspace_bytes=0, stream=None)
    a.update(kw)
    return bfq.lib.bfq_block_gemm(*a.values())


def test_gemm_validation_errors_without_launch(bfq):
    assert _gemm(bfq, w_q=None) == bfq.BFQ_ERR_NULL
    assert _gemm(bfq, M=5, a_q=None) == bfq.BFQ_ERR_NULL
    assert _gemm(bfq, K=7000) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, N=1000) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, M=-1) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, block_shape=(ctypes.c_int32 * 2)(128, 64)) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, in_dtype=bfq.BFQ_BF16) == bfq.BFQ_ERR_DTYPE
    assert _gemm(bfq, out_dtype=bfq.BFQ_INT8) == bfq.BFQ_ERR_DTYPE
    assert _gemm(bfq, w_q=FAKE + 8) == bfq.BFQ_ERR_ALIGN
    assert _gemm(bfq, a_scales=FAKE + 2) == bfq.BFQ_ERR_ALIGN
    assert _gemm(bfq, a_scale_ld=10) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, M=64, a_layout=1, a_scale_ld=63) == bfq.BFQ_ERR_SHAPE
    # at most 2^40 outputs: 2^21 x 2^19 is rejected, one row fewer passes the shape checks
    big = dict(N=1 << 19, K=128, a_scale_ld=1)
    assert _gemm(bfq, M=1 << 21, **big) == bfq.BFQ_ERR_SHAPE
    assert "2^40" in bfq.last_error()
    # the size queries answer SIZE_MAX for such shapes (never a wrapped product)
    size_max = ctypes.c_size_t(-1).value
    t = bfq.bfq_tile(variant=0, bm=256, bn=256, bk=128, split_k=256, waves_m=4, waves_n=2,
                     stages=2, group_m=8, sched=0, raster=0)
    assert bfq.lib.bfq_gemm_workspace_bytes(1 << 21, 1 << 19, 128, ctypes.byref(t)) == size_max
    assert bfq.lib.bfq_gemm_workspace_bytes(1 << 40, 1 << 40, 128, ctypes.byref(t)) == size_max
    assert bfq.lib.bfq_gemm_workspace_bytes((1 << 21) - 1, 1 << 19, 128, ctypes.byref(t)) == \
        256 * ((1 << 21) - 1) * (1 << 19) * 4
    assert bfq.lib.bfq_moe_gemm_workspace_bytes(1 << 40, 8, 1 << 30, ctypes.byref(t)) == size_max
    assert _gemm(bfq, a_layout=7) == bfq.BFQ_ERR_ARG
    assert _gemm(bfq, w_layout=2) == bfq.BFQ_ERR_ARG
    assert _gemm(bfq, scale_fmt=2) == bfq.BFQ_ERR_ARG
    # a block-scaled-MFMA tile (sched 3) needs scales declared as powers of two
    ue = [bfq.bfq_get_tile_candidate(i, bfq.BFQ_E4M3FN, 0, bfq.BFQ_SCALE_UE8M0)
          for i in range(bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, 0, bfq.BFQ_SCALE_UE8M0))]
    t3 = next(t for t in ue if t.sched == 3 and t.variant == 0)
    assert _gemm(bfq, M=64, tile=ctypes.pointer(t3)) == bfq.BFQ_ERR_TILE
    assert "scale format" in bfq.last_error()
    assert _gemm(bfq, M=0, scale_fmt=1, tile=ctypes.pointer(t3)) >= 0
    # a tile compiled only for row-major weights is rejected for packed ones
    row_only = [bfq.bfq_get_tile_candidate(i) for i in range(bfq.bfq_num_tile_candidates())]
    packed = {tuple(bfq.bfq_get_tile_candidate(i, bfq.BFQ_E4M3FN, bfq.BFQ_W_PACKED16).as_dict().values())
              for i in range(bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, bfq.BFQ_W_PACKED16))}
    t32 = next(t for t in row_only if tuple(t.as_dict().values()) not in packed)
    assert _gemm(bfq, M=64, w_layout=1, tile=ctypes.pointer(t32)) == bfq.BFQ_ERR_TILE
    assert "weight layout" in bfq.last_error()
    bad = bfq.bfq_tile.from_dict({"variant": 0, "bm": 96, "bn": 96, "waves_m": 2, "waves_n": 2})
    assert _gemm(bfq, tile=ctypes.pointer(bad)) == bfq.BFQ_ERR_TILE
    t = bfq.bfq_get_tile_candidate(0)
    t.split_k = 4
    assert _gemm(bfq, M=64, tile=ctypes.pointer(t)) == bfq.BFQ_ERR_WORKSPACE
    t.split_k = 57      # more splits than K blocks
    assert _gemm(bfq, M=64, tile=ctypes.pointer(t)) == bfq.BFQ_ERR_TILE
    assert "split_k" in bfq.last_error()
    # M = 0 is valid and launches nothing
    assert _gemm(bfq, M=0) >= 0


def test_quant_validation_errors_without_launch(bfq):
    q = bfq.lib.bfq_quant_tokens
    args = [FAKE, 4, 7168, 128, bfq.BFQ_E4M3FN, FAKE, FAKE, 0, 56, 1e-10, 0, None]

    def call(**kw):
        a = list(args)
        names = ["x", "M", "K", "group", "qd", "q", "s", "layout", "ld", "eps", "sfmt", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return q(*a)

    assert call(x=None) == bfq.BFQ_ERR_NULL
    assert call(K=100) == bfq.BFQ_ERR_SHAPE
    assert call(group=64) == bfq.BFQ_ERR_SHAPE
    assert call(qd=bfq.BFQ_BF16) == bfq.BFQ_ERR_DTYPE
    assert call(x=FAKE + 2) == bfq.BFQ_ERR_ALIGN
    assert call(ld=55) == bfq.BFQ_ERR_SHAPE
    assert call(layout=1, ld=3) == bfq.BFQ_ERR_SHAPE
    assert call(eps=0.0) == bfq.BFQ_ERR_ARG
    assert call(eps=float("nan")) == bfq.BFQ_ERR_ARG
    assert call(sfmt=5) == bfq.BFQ_ERR_ARG
    assert call(M=0, x=None, q=None, s=None) == bfq.BFQ_OK
    w = bfq.lib.bfq_quant_weight_blocks
    assert w(FAKE, 256, 256, (ctypes.c_int32 * 2)(64, 128), bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE
    assert w(FAKE, 250, 256, BS, bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE
    assert w(None, 256, 256, BS, bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 0, None) == bfq.BFQ_ERR_NULL
    assert w(FAKE, 256, 256, BS, bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 3, None) == bfq.BFQ_ERR_ARG
    assert w(FAKE, 0, 256, BS, bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 1, None) == bfq.BFQ_OK


def test_pack_validation_errors_without_launch(bfq):
    pk = bfq.lib.bfq_pack_weights
    other = FAKE + (1 << 24)
    assert pk(None, 256, 256, bfq.BFQ_E4M3FN, other, None) == bfq.BFQ_ERR_NULL
    assert pk(FAKE, 256, 256, bfq.BFQ_E4M3FN, None, None) == bfq.BFQ_ERR_NULL
    assert pk(FAKE, 250, 256, bfq.BFQ_E4M3FN, other, None) == bfq.BFQ_ERR_SHAPE
    assert pk(FAKE, 256, 200, bfq.BFQ_E4M3FN, other, None) == bfq.BFQ_ERR_SHAPE
    assert pk(FAKE, 256, 256, bfq.BFQ_BF16, other, None) == bfq.BFQ_ERR_DTYPE
    assert pk(FAKE + 4, 256, 256, bfq.BFQ_E4M3FN, other, None) == bfq.BFQ_ERR_ALIGN
    # the buffers overlap (in place, or offset by less than N*K bytes)
    assert pk(FAKE, 256, 256, bfq.BFQ_E4M3FN, FAKE, None) == bfq.BFQ_ERR_ARG
    assert pk(FAKE, 256, 256, bfq.BFQ_E4M3FN, FAKE + 65520, None) == bfq.BFQ_ERR_ARG
    assert pk(FAKE, 0, 256, bfq.BFQ_INT8, other, None) == bfq.BFQ_OK


@pytest.mark.parametrize("sf", [0, 1])
@pytest.mark.parametrize("wl", [0, 1])
def test_candidates_enumerate(bfq, wl, sf):
    for qd in (bfq.BFQ_E4M3FN, bfq.BFQ_INT8):
        n = bfq.bfq_num_tile_candidates(qd, wl, sf)
        assert n >= 4
        seen = set()
        for i in range(n):
            t = bfq.bfq_get_tile_candidate(i, qd, wl, sf)
            assert t.split_k == 1 and t.bk == 128 and t.variant in (0, 1, 2)
            seen.add(tuple(t.as_dict().values()))
        assert len(seen) == n
        # every kernel variant is compiled for both layouts
        assert {t[0] for t in seen} == {0, 1, 2}
        # block-scaled MFMA tiles (sched 3, variants 0 and 2) exactly for fp8 with UE8M0 scales
        has3 = any(t[0] in (0, 2) and t[9] == 3 for t in seen)
        assert has3 == (qd == bfq.BFQ_E4M3FN and sf == 1)
        # UE8M0 scales can use every kernel the fp32 format can
        if sf == 1:
            fp32 = {tuple(bfq.bfq_get_tile_candidate(i, qd, wl, 0).as_dict().values())
                    for i in range(bfq.bfq_num_tile_candidates(qd, wl, 0))}
            assert fp32 <= seen
    with pytest.raises(bfq.BfqError):
        bfq.bfq_get_tile_candidate(10_000)
    assert bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, 5) == 0
    assert bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, 0, 7) == 0


def _table(entries):
    return json.dumps({"device": "gfx950", "entries": entries})


def test_table_nearest_m_and_fallback(bfq, tmp_path):
    """The config page's lookup (§4.1-§4.2): exact (N, K, dtype) key, nearest M bucket
    (M=37 -> 32, M=2050 -> 2048, ties to the smaller bucket), default + warning on a miss."""
    grid = json.load(open(os.path.join(HERE, "golden", "nearest_m.json")))
    cands = [bfq.bfq_get_tile_candidate(i).as_dict() for i in range(bfq.bfq_num_tile_candidates())]
    cfgs = {str(m): dict(cands[i % len(cands)], split_k=1 + (i % 3)) for i, m in enumerate(grid["grid"])}
    p = tmp_path / "t.json"
    p.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "block_shape": [128, 128],
                          "configs": cfgs}]))
    try:
        assert bfq.bfq_load_tile_table(str(p)) == bfq.BFQ_OK
        for m, want in grid["examples"] + grid["ties"] + grid["ends"]:
            st, t = bfq.bfq_select_tile(m, 1536, 7168)
            assert st == bfq.BFQ_OK
            exp = cfgs[str(want)]
            assert t.as_dict() == dict(exp, bk=128), (m, want)
        st, t = bfq.bfq_select_tile(64, 4096, 7168)           # no entry for this shape
        assert st == bfq.BFQ_WARN_DEFAULT_TILE
        st, t = bfq.bfq_select_tile(64, 1536, 7168, in_dtype=bfq.BFQ_INT8)   # dtype is part of the key
        assert st == bfq.BFQ_WARN_DEFAULT_TILE
        st, t = bfq.bfq_select_tile(64, 1536, 7168, w_layout=bfq.BFQ_W_PACKED16)   # so is the layout
        assert st == bfq.BFQ_WARN_DEFAULT_TILE
        st, t = bfq.bfq_select_tile(64, 1536, 7168, scale_fmt=bfq.BFQ_SCALE_UE8M0)   # and the scales
        assert st == bfq.BFQ_WARN_DEFAULT_TILE
    finally:
        bfq.bfq_load_tile_table(None)


def test_table_weight_layout_key(bfq, tmp_path):
    """An entry marked "w_layout": "packed16" serves packed weights only, and its tiles must
    name kernels compiled for that layout."""
    wl = bfq.BFQ_W_PACKED16
    cand = bfq.bfq_get_tile_candidate(0, bfq.BFQ_E4M3FN, wl).as_dict()
    p = tmp_path / "t.json"
    p.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "w_layout": "packed16",
                          "configs": {"16": dict(cand, split_k=2)}}]))
    try:
        assert bfq.bfq_load_tile_table(str(p)) == bfq.BFQ_OK
        st, t = bfq.bfq_select_tile(16, 1536, 7168, w_layout=wl)
        assert st == bfq.BFQ_OK and t.as_dict() == dict(cand, split_k=2, bk=128)
        st, t = bfq.bfq_select_tile(16, 1536, 7168)
        assert st == bfq.BFQ_WARN_DEFAULT_TILE
    finally:
        bfq.bfq_load_tile_table(None)
    bad = tmp_path / "bad.json"
    bad.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "w_layout": "tiled",
                            "configs": {"16": cand}}]))
    with pytest.raises(bfq.BfqError):
        bfq.bfq_load_tile_table(str(bad))
    bfq.bfq_load_tile_table(None)


def test_table_scale_format_key(bfq, tmp_path):
    """An entry marked "scales": "ue8m0" serves power-of-two scales only and may name
    block-scaled-MFMA tiles; the same tile in an fp32 entry is rejected."""
    sf = bfq.BFQ_SCALE_UE8M0
    ue = [bfq.bfq_get_tile_candidate(i, bfq.BFQ_E4M3FN, 0, sf).as_dict()
          for i in range(bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, 0, sf))]
    t3 = next(d for d in ue if d["sched"] == 3)
    p = tmp_path / "t.json"
    p.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "scales": "ue8m0",
                          "configs": {"4096": t3}}]))
    try:
        assert bfq.bfq_load_tile_table(str(p)) == bfq.BFQ_OK
        st, t = bfq.bfq_select_tile(4096, 1536, 7168, scale_fmt=sf)
        assert st == bfq.BFQ_OK and t.as_dict() == dict(t3, bk=128)
        st, t = bfq.bfq_select_tile(4096, 1536, 7168)
        assert st == bfq.BFQ_WARN_DEFAULT_TILE and t.sched != 3
    finally:
        bfq.bfq_load_tile_table(None)
    bad = tmp_path / "bad.json"
    bad.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "configs": {"4096": t3}}]))
    with pytest.raises(bfq.BfqError):
        bfq.bfq_load_tile_table(str(bad))
    bad.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "scales": "e5m2",
                            "configs": {"4096": t3}}]))
    with pytest.raises(bfq.BfqError):
        bfq.bfq_load_tile_table(str(bad))
    bfq.bfq_load_tile_table(None)


@pytest.mark.parametrize("text,why", [
    ("{", "truncated"),
    ('{"entries": [{"N": 1536, "K": 7168, "dtype": "fp9", "configs": {"1": {}}}]}', "dtype"),
    ('{"entries": [{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "configs": {"x": {}}}]}', "key"),
    ('{"entries": [{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "configs": {"1": '
     '{"variant": 0, "bm": 96, "bn": 96, "waves_m": 2, "waves_n": 2}}}]}', "uncompiled tile"),
    ('{"entries": [{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "block_shape": [64, 128],'
     ' "configs": {"1": {"variant": 1, "bm": 16, "bn": 128, "waves_m": 1, "waves_n": 4, '
     '"stages": 4}}}]}', "block shape"),
])
def test_bad_tables_rejected(bfq, tmp_path, text, why):
    p = tmp_path / "bad.json"
    p.write_text(text)
    with pytest.raises(bfq.BfqError) as e:
        bfq.bfq_load_tile_table(str(p))
    assert e.value.status == bfq.BFQ_ERR_TABLE, why
    with pytest.raises(bfq.BfqError):
        bfq.bfq_load_tile_table(str(tmp_path / "missing.json"))
    bfq.bfq_load_tile_table(None)


def test_default_rule(bfq, tmp_path):
    """With no tuned entry: swap-AB streaming below 32 tokens (the Hopper rule of the Helion
    page), the standard tile otherwise; split-K only while the grid is short of 256 CUs."""
    p = tmp_path / "empty.json"
    p.write_text(_table([]))
    bfq.bfq_load_tile_table(str(p))
    try:
        for M in (1, 8, 16, 31):
            st, t = bfq.bfq_select_tile(M, 24576, 7168)
            assert st == bfq.BFQ_WARN_DEFAULT_TILE and t.variant == 1
        # the default tiles exist for both weight layouts and scale formats
        for wl in (bfq.BFQ_W_ROW_MAJOR, bfq.BFQ_W_PACKED16):
            for sf in (bfq.BFQ_SCALE_FP32, bfq.BFQ_SCALE_UE8M0):
                for M in (1, 31, 64, 200, 4096):
                    st, t = bfq.bfq_select_tile(M, 24576, 7168, w_layout=wl, scale_fmt=sf)
                    assert st == bfq.BFQ_WARN_DEFAULT_TILE
                    assert _gemm(bfq, M=0, N=24576, w_layout=wl, scale_fmt=sf,
                                 tile=ctypes.pointer(t)) >= 0
        st, t = bfq.bfq_select_tile(4096, 24576, 7168, scale_fmt=bfq.BFQ_SCALE_UE8M0)
        assert t.sched == 3
        for M in (32, 64, 4096):
            st, t = bfq.bfq_select_tile(M, 24576, 7168)
            assert t.variant == 0
        st, t = bfq.bfq_select_tile(4096, 24576, 7168)
        assert t.split_k == 1 and (t.bm, t.bn) == (256, 256)
        st, t = bfq.bfq_select_tile(1, 1536, 7168)
        assert t.split_k > 1
    finally:
        bfq.bfq_load_tile_table(None)


# (M, N) pairs that reach each pick of the default rule's standard-tile list at K = 7168:
# 256x256 fills the CUs; 128x256 does (fp8) and int8 falls through to 128x128; only 128x128
# does; none does (the smallest compiled tile, plus split-K); and the swap-AB rule below 32.
DEFAULT_PICKS = [(4096, 24576), (512, 24576), (2048, 4096), (300, 4096), (200, 4096),
                 (32, 24576), (31, 1536), (1, 7168)]


@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_default_rule_names_compiled_kernels(bfq, tmp_path, qname):
    """With an empty table, every default tile names a kernel compiled for the code type,
    weight layout and scale format (fp32 / UE8M0 block scales, packed UE8M0 words, per-token x
    per-channel), so the GEMM accepts it. The int8 kernels have no 128x256 tile: at M=2048,
    N=4096 the rule passes over it to 128x128."""
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    p = tmp_path / "empty.json"
    p.write_text(_table([]))
    bfq.bfq_load_tile_table(str(p))
    try:
        for wl in (bfq.BFQ_W_ROW_MAJOR, bfq.BFQ_W_PACKED16):
            for sf, lay, ld, bs in ((0, 0, 56, BS), (1, 0, 56, BS), (1, 2, 4096, BS),
                                    (0, 0, 1, _bs(1, 7168))):
                if lay == 2 and qd == bfq.BFQ_INT8:
                    continue                # packed words are read by the e4m3fn GEMM only
                for M, N in DEFAULT_PICKS:
                    st, t = bfq.bfq_select_tile(M, N, 7168, qd, w_layout=wl, scale_fmt=sf,
                                                block_shape=tuple(bs))
                    what = (qname, wl, sf, lay, tuple(bs), M, N, t.as_dict())
                    assert st == bfq.BFQ_WARN_DEFAULT_TILE, what
                    assert _gemm(bfq, M=0, N=N, in_dtype=qd, w_layout=wl, scale_fmt=sf,
                                 a_layout=lay, a_scale_ld=ld, block_shape=bs,
                                 tile=ctypes.pointer(t)) >= 0, (what, bfq.last_error())
        st, t = bfq.bfq_select_tile(2048, 4096, 7168, qd)
        want = (128, 256) if qname == "fp8" else (128, 128)
        assert (t.variant, t.bm, t.bn) == (0, *want), t.as_dict()
    finally:
        bfq.bfq_load_tile_table(None)


def test_metric_formulas_reproduce_pages_table():
    """P10: the pages' TFLOPS and GB/s formulas (block GEMM benchmark page §4.3) recompute
    every printed row of §3.2 from its (m, n, k, us) within the rounding of the print."""
    from block_scaled_w8a8_amd import perf
    rows = [l.strip().split(",") for l in open(os.path.join(HERE, "golden", "h100_block_fp8_rows.csv"))
            if l.strip() and not l.startswith("#") and not l.startswith("impl")]
    assert len(rows) == 48
    for impl, m, n, k, us, tf, gbs in rows:
        m, n, k, t = int(m), int(n), int(k), float(us) * 1e-6
        assert perf.tflops(m, n, k, t) == pytest.approx(float(tf), rel=0.008, abs=0.06)
        assert perf.gbs_page(m, n, k, t) == pytest.approx(float(gbs), rel=0.008)
    # the averages the page prints (§3.3) are the arithmetic means of the 16 rows
    for impl, avg_tf, avg_gbs in [("deepgemm", 310.98, 1052.10), ("triton", 144.30, 715.60),
                                  ("cutlass", 286.78, 1076.67)]:
        sel = [r for r in rows if r[0] == impl]
        assert sum(float(r[5]) for r in sel) / 16 == pytest.approx(avg_tf, abs=0.01)
        assert sum(float(r[6]) for r in sel) / 16 == pytest.approx(avg_gbs, abs=0.01)


def test_batch_invariant_selection(bfq):
    """Batch-invariant mode (config page §5): tuned entries are ignored; every selected tile
    is a compiled kernel with no split-K, no in-workgroup K split, no stream-K and the fp32
    FMA scale step, and with row-major weights a standard tile."""
    assert bfq.bfq_get_batch_invariant() in (False, True)
    bfq.bfq_set_batch_invariant(True)
    try:
        assert bfq.bfq_get_batch_invariant()
        for qd in (bfq.BFQ_E4M3FN, bfq.BFQ_INT8):
            for wl in (bfq.BFQ_W_ROW_MAJOR, bfq.BFQ_W_PACKED16):
                for sf in (bfq.BFQ_SCALE_FP32, bfq.BFQ_SCALE_UE8M0):
                    for M in (1, 7, 16, 17, 33, 64, 65, 128, 129, 512, 513, 4096):
                        st, t = bfq.bfq_select_tile(M, 24576, 7168, in_dtype=qd, w_layout=wl,
                                                    scale_fmt=sf)
                        assert st == bfq.BFQ_OK
                        assert t.split_k == 1 and t.variant in (0, 1) and t.sched in (0, 1)
                        assert t.variant == 0 or (t.waves_m == 1 and wl == bfq.BFQ_W_PACKED16)
                        assert _gemm(bfq, M=0, N=24576, in_dtype=qd, w_layout=wl, scale_fmt=sf,
                                     tile=ctypes.pointer(t)) >= 0, (qd, wl, sf, M, t.as_dict())
    finally:
        bfq.bfq_set_batch_invariant(False)
    assert not bfq.bfq_get_batch_invariant()


# ------------------------------------------- per-token x per-channel format (block_shape {1, K})

def _bs(a, b):
    return (ctypes.c_int32 * 2)(a, b)


def _channel_cands(bfq, qd, wl):
    ch = bfq.channel_block_shape(7168)
    return [bfq.bfq_get_tile_candidate(i, qd, wl, 0, block_shape=ch)
            for i in range(bfq.bfq_num_tile_candidates(qd, wl, 0, block_shape=ch))]


def test_channel_gemm_validation_without_launch(bfq):
    ch = _bs(1, 7168)
    assert _gemm(bfq, M=0, block_shape=ch, a_scale_ld=1) >= 0
    assert _gemm(bfq, M=0, block_shape=ch, a_layout=1, a_scale_ld=0) >= 0
    assert _gemm(bfq, block_shape=_bs(1, 7040)) == bfq.BFQ_ERR_SHAPE       # [1, k], k != K
    assert _gemm(bfq, block_shape=_bs(2, 7168)) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, K=32896, block_shape=_bs(1, 32896), a_scale_ld=1) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, M=0, K=32768, block_shape=_bs(1, 32768), a_scale_ld=1) >= 0
    assert _gemm(bfq, M=4, block_shape=ch, a_scale_ld=0) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, M=64, block_shape=ch, a_layout=1, a_scale_ld=63) == bfq.BFQ_ERR_SHAPE
    # a block-scale tile cannot serve per-channel scales, nor the other way round
    tb = bfq.bfq_get_tile_candidate(0)
    assert _gemm(bfq, M=64, block_shape=ch, a_scale_ld=1, tile=ctypes.pointer(tb)) == bfq.BFQ_ERR_TILE
    tc = _channel_cands(bfq, bfq.BFQ_E4M3FN, 0)[0]
    assert _gemm(bfq, M=64, tile=ctypes.pointer(tc)) == bfq.BFQ_ERR_TILE
    assert _gemm(bfq, M=0, block_shape=ch, a_scale_ld=1, tile=ctypes.pointer(tc)) >= 0


def test_channel_quant_validation_without_launch(bfq):
    q = bfq.lib.bfq_quant_tokens
    # M = 0: validated, nothing launched
    assert q(FAKE, 0, 7168, 7168, bfq.BFQ_E4M3FN, FAKE, FAKE, 0, 1, 1e-10, 0, None) == bfq.BFQ_OK
    assert q(FAKE, 0, 7168, 7168, bfq.BFQ_INT8, FAKE, FAKE, 1, 0, 1e-10, 1, None) == bfq.BFQ_OK
    assert q(FAKE, 4, 7168, 7168, bfq.BFQ_E4M3FN, FAKE, FAKE, 0, 0, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE
    assert q(FAKE, 4, 7168, 3584, bfq.BFQ_E4M3FN, FAKE, FAKE, 0, 2, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE
    assert q(FAKE, 4, 32896, 32896, bfq.BFQ_E4M3FN, FAKE, FAKE, 0, 1, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE
    w = bfq.lib.bfq_quant_weight_blocks
    assert w(FAKE, 0, 7168, _bs(1, 7168), bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 0, None) == bfq.BFQ_OK
    assert w(FAKE, 256, 7168, _bs(1, 7040), bfq.BFQ_E4M3FN, FAKE, FAKE, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE
    assert w(FAKE, 256, 32896, _bs(1, 32896), bfq.BFQ_INT8, FAKE, FAKE, 1e-10, 0, None) == bfq.BFQ_ERR_SHAPE


@pytest.mark.parametrize("wl", [0, 1])
def test_channel_candidates(bfq, wl):
    """Per-channel kernels: the standard and stream-K ones use sched 4 (whole-K accumulation)
    and no block-format candidate does; the streaming kernels exist for both dtypes."""
    for qd in (bfq.BFQ_E4M3FN, bfq.BFQ_INT8):
        cands = _channel_cands(bfq, qd, wl)
        assert len(cands) >= 8
        assert {t.variant for t in cands} >= {0, 1}
        assert all(t.sched == 4 for t in cands if t.variant in (0, 2))
        for sf in (0, 1):
            block = [bfq.bfq_get_tile_candidate(i, qd, wl, sf)
                     for i in range(bfq.bfq_num_tile_candidates(qd, wl, sf))]
            assert all(t.sched != 4 for t in block)
    assert bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, 0, 0, block_shape=(64, 64)) == 0


def test_channel_default_and_invariant_tiles(bfq, tmp_path):
    """With no tuned entry the default rule and the batch-invariant mode pick compiled
    per-channel kernels for every M, both dtypes and both weight layouts."""
    p = tmp_path / "empty.json"
    p.write_text(_table([]))
    bfq.bfq_load_tile_table(str(p))
    ch = bfq.channel_block_shape(7168)
    try:
        for inv in (False, True):
            bfq.bfq_set_batch_invariant(inv)
            for qd in (bfq.BFQ_E4M3FN, bfq.BFQ_INT8):
                for wl in (0, 1):
                    for M in (1, 16, 31, 64, 200, 513, 4096):
                        st, t = bfq.bfq_select_tile(M, 24576, 7168, in_dtype=qd, w_layout=wl,
                                                    block_shape=ch)
                        assert st == (bfq.BFQ_OK if inv else bfq.BFQ_WARN_DEFAULT_TILE)
                        assert t.variant == 1 or t.sched == 4
                        if inv:   # no split-K; variant 1's waves_m is its in-workgroup K split
                            assert t.split_k == 1 and (t.variant == 0 or t.waves_m == 1)
                        assert _gemm(bfq, M=0, N=24576, in_dtype=qd, w_layout=wl,
                                     block_shape=_bs(1, 7168), a_scale_ld=1,
                                     tile=ctypes.pointer(t)) >= 0, (inv, qd, wl, M, t.as_dict())
    finally:
        bfq.bfq_set_batch_invariant(False)
        bfq.bfq_load_tile_table(None)


def test_table_channel_key(bfq, tmp_path):
    """An entry with "block_shape": [1, K] serves the per-channel format only, must name
    per-channel kernels and takes no "scales" field."""
    tc = _channel_cands(bfq, bfq.BFQ_E4M3FN, 0)[0].as_dict()
    tb = bfq.bfq_get_tile_candidate(0).as_dict()
    p = tmp_path / "t.json"
    p.write_text(_table([{"N": 1536, "K": 7168, "dtype": "fp8_w8a8", "block_shape": [1, 7168],
                          "configs": {"16": dict(tc, split_k=2)}}]))
    try:
        assert bfq.bfq_load_tile_table(str(p)) == bfq.BFQ_OK
        st, t = bfq.bfq_select_tile(16, 1536, 7168, block_shape=bfq.channel_block_shape(7168))
        assert st == bfq.BFQ_OK and t.as_dict() == dict(tc, split_k=2, bk=128)
        st, t = bfq.bfq_select_tile(16, 1536, 7168)
        assert st == bfq.BFQ_WARN_DEFAULT_TILE
    finally:
        bfq.bfq_load_tile_table(None)
    for e in ({"block_shape": [1, 7168], "configs": {"16": tb}},                     # block tile
              {"block_shape": [1, 1536], "configs": {"16": tc}},                     # [1, k != K]
              {"block_shape": [1, 7168], "scales": "ue8m0", "configs": {"16": tc}}):
        bad = tmp_path / "bad.json"
        bad.write_text(_table([dict({"N": 1536, "K": 7168, "dtype": "fp8_w8a8"}, **e)]))
        with pytest.raises(bfq.BfqError):
            bfq.bfq_load_tile_table(str(bad))
    bfq.bfq_load_tile_table(None)


# ------------------------------------------- packed UE8M0 activation-scale words (layout 2)

def test_packed_scale_validation_without_launch(bfq):
    P = bfq.BFQ_SCALES_PACKED_UE8M0
    q = bfq.lib.bfq_quant_tokens
    # M = 5 needs ld >= 8 (rows padded to a multiple of 4); UE8M0 and 1x128 groups only
    assert q(FAKE, 0, 7168, 128, bfq.BFQ_E4M3FN, FAKE, FAKE, P, 0, 1e-10, 1, None) == bfq.BFQ_OK
    assert q(FAKE, 5, 7168, 128, bfq.BFQ_E4M3FN, FAKE, FAKE, P, 7, 1e-10, 1, None) == bfq.BFQ_ERR_SHAPE
    assert q(FAKE, 5, 7168, 128, bfq.BFQ_E4M3FN, FAKE, FAKE, P, 8, 1e-10, 0, None) == bfq.BFQ_ERR_ARG
    assert q(FAKE, 5, 7168, 7168, bfq.BFQ_E4M3FN, FAKE, FAKE, P, 8, 1e-10, 1, None) == bfq.BFQ_ERR_ARG
    assert _gemm(bfq, M=0, a_layout=P, a_scale_ld=0, scale_fmt=1) >= 0
    assert _gemm(bfq, M=5, a_layout=P, a_scale_ld=4, scale_fmt=1) == bfq.BFQ_ERR_SHAPE
    assert _gemm(bfq, M=5, a_layout=P, a_scale_ld=8, scale_fmt=0) == bfq.BFQ_ERR_ARG
    assert _gemm(bfq, M=5, a_layout=P, a_scale_ld=8, scale_fmt=1,
                 in_dtype=bfq.BFQ_INT8) == bfq.BFQ_ERR_DTYPE
    assert _gemm(bfq, M=5, a_layout=P, a_scale_ld=8, scale_fmt=1,
                 block_shape=_bs(1, 7168)) == bfq.BFQ_ERR_ARG


@pytest.mark.parametrize("wl", [0, 1])
def test_packed_scales_every_ue8m0_tile_has_a_kernel(bfq, tmp_path, wl):
    """Every fp8 tile usable with UE8M0 scales, and every tile the table or the default rule
    selects for them, names a kernel that reads packed scale words."""
    P = bfq.BFQ_SCALES_PACKED_UE8M0
    sf = bfq.BFQ_SCALE_UE8M0
    tiles = [bfq.bfq_get_tile_candidate(i, bfq.BFQ_E4M3FN, wl, sf)
             for i in range(bfq.bfq_num_tile_candidates(bfq.BFQ_E4M3FN, wl, sf))]
    for M in (1, 8, 31, 64, 128, 256, 2048, 4096):
        tiles.append(bfq.bfq_select_tile(M, 24576, 7168, w_layout=wl, scale_fmt=sf)[1])
    p = tmp_path / "empty.json"
    p.write_text(_table([]))
    bfq.bfq_load_tile_table(str(p))
    try:
        for M in (1, 31, 64, 200, 4096):
            tiles.append(bfq.bfq_select_tile(M, 24576, 7168, w_layout=wl, scale_fmt=sf)[1])
    finally:
        bfq.bfq_load_tile_table(None)
    for t in tiles:
        assert _gemm(bfq, M=0, N=24576, a_layout=P, a_scale_ld=0, scale_fmt=sf, w_layout=wl,
                     tile=ctypes.pointer(t)) >= 0, t.as_dict()


# ------------------------------------------------------------------ MoE grouped GEMM

def _moe(bfq, **kw):
    a = dict(a_q=FAKE, a_scales=FAKE, a_layout=0, a_scale_ld=56, sorted_pairs=FAKE,
             expert_offsets=FAKE, topk=8, w_q=FAKE, w_scales=FAKE, w_layout=0, scale_fmt=0,
             out=FAKE, T=0, N=4096, K=7168, E=256, block_shape=BS, in_dtype=bfq.BFQ_E4M3FN,
             out_dtype=bfq.BFQ_BF16, tile=None, workspace=None, workspace_bytes=0, stream=None)
    a.update(kw)
    return bfq.lib.bfq_moe_block_gemm(*a.values())


def test_moe_validation_without_launch(bfq):
    assert _moe(bfq) >= 0                                          # T = 0: nothing launched
    assert _moe(bfq, T=4, a_q=None) == bfq.BFQ_ERR_NULL
    assert _moe(bfq, expert_offsets=None) == bfq.BFQ_ERR_NULL
    assert _moe(bfq, in_dtype=bfq.BFQ_INT8) == bfq.BFQ_ERR_DTYPE
    assert _moe(bfq, block_shape=_bs(1, 7168)) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, E=0) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, E=1024) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, topk=0) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, N=1000) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, T=300000) == bfq.BFQ_ERR_SHAPE               # T * K >= 2^31
    # K beyond 2^23: 256 weight rows x K would wrap the 32-bit weight offsets
    assert _moe(bfq, T=1, K=1 << 24, a_scale_ld=1 << 17) == bfq.BFQ_ERR_SHAPE
    assert "2^23" in bfq.last_error()
    assert _moe(bfq, T=0, K=1 << 24, a_scale_ld=1 << 17) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, a_scale_ld=10) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, T=64, a_layout=1, a_scale_ld=63) == bfq.BFQ_ERR_SHAPE
    assert _moe(bfq, a_layout=2, a_scale_ld=0) == bfq.BFQ_ERR_ARG  # packed needs UE8M0
    assert _moe(bfq, a_layout=2, a_scale_ld=0, scale_fmt=1) >= 0
    assert _moe(bfq, sorted_pairs=FAKE + 2, T=4) == bfq.BFQ_ERR_ALIGN
    dense = bfq.bfq_get_tile_candidate(0)
    dense.variant = 2                                              # no grouped stream-K
    assert _moe(bfq, T=4, tile=ctypes.pointer(dense)) == bfq.BFQ_ERR_TILE
    t = bfq.bfq_moe_get_tile_candidate(0)
    t.split_k = 2
    assert _moe(bfq, T=4, tile=ctypes.pointer(t)) == bfq.BFQ_ERR_WORKSPACE
    al = bfq.lib.bfq_moe_align
    assert al(FAKE, 4, 8, 0, FAKE, FAKE, FAKE, 1 << 20, None) == bfq.BFQ_ERR_SHAPE
    assert al(FAKE, 4, 8, 256, None, FAKE, FAKE, 1 << 20, None) == bfq.BFQ_ERR_NULL
    assert al(FAKE, 4, 8, 256, FAKE, FAKE, None, 0, None) == bfq.BFQ_ERR_WORKSPACE
    assert bfq.lib.bfq_moe_align_workspace_bytes(4096, 8, 256) == 257 * 32 * 4


@pytest.mark.parametrize("wl", [0, 1])
def test_moe_candidates_default_and_invariant_tiles(bfq, tmp_path, wl):
    """Grouped kernels exist for both layouts; the default rule and the batch-invariant mode
    name compiled grouped kernels for every token count, fp32 / UE8M0 / packed scales."""
    for sf in (0, 1):
        n = bfq.bfq_moe_num_tile_candidates(wl, sf)
        cands = [bfq.bfq_moe_get_tile_candidate(i, wl, sf) for i in range(n)]
        assert n >= 10 and {t.variant for t in cands} == {0, 1}
        assert len({tuple(t.as_dict().values()) for t in cands}) == n
    p = tmp_path / "empty.json"
    p.write_text(_table([]))
    bfq.bfq_load_tile_table(str(p))
    try:
        for inv in (False, True):
            bfq.bfq_set_batch_invariant(inv)
            for sf, lay, ld in ((0, 0, 56), (1, 0, 56), (1, 2, 0)):
                for T in (1, 4, 32, 128, 512, 2048, 4096, 16384):
                    st, t = bfq.bfq_moe_select_tile(T, 8, 256, 4096, 7168, w_layout=wl, scale_fmt=sf)
                    assert st == (bfq.BFQ_OK if inv else bfq.BFQ_WARN_DEFAULT_TILE)
                    assert t.split_k == 1 and t.variant in (0, 1)
                    assert _moe(bfq, w_layout=wl, scale_fmt=sf, a_layout=lay, a_scale_ld=ld,
                                tile=ctypes.pointer(t)) >= 0, (inv, sf, lay, T, t.as_dict())
    finally:
        bfq.bfq_set_batch_invariant(False)
        bfq.bfq_load_tile_table(None)


def test_table_moe_key(bfq, tmp_path):
    """An entry with "E" serves grouped selection for that expert count only (buckets are
    token counts); its tiles must name grouped kernels."""
    tm = bfq.bfq_moe_get_tile_candidate(3).as_dict()
    p = tmp_path / "t.json"
    p.write_text(_table([{"N": 4096, "K": 7168, "dtype": "fp8_w8a8", "E": 256,
                          "configs": {"64": tm, "1024": dict(tm, split_k=2)}}]))
    try:
        assert bfq.bfq_load_tile_table(str(p)) == bfq.BFQ_OK
        st, t = bfq.bfq_moe_select_tile(70, 8, 256, 4096, 7168)
        assert st == bfq.BFQ_OK and t.as_dict() == dict(tm, bk=128)
        st, t = bfq.bfq_moe_select_tile(900, 8, 256, 4096, 7168)
        assert st == bfq.BFQ_OK and t.split_k == 2
        assert bfq.bfq_moe_select_tile(70, 8, 128, 4096, 7168)[0] == bfq.BFQ_WARN_DEFAULT_TILE
        assert bfq.bfq_select_tile(70, 4096, 7168)[0] == bfq.BFQ_WARN_DEFAULT_TILE   # dense
    finally:
        bfq.bfq_load_tile_table(None)
    bad = tmp_path / "bad.json"
    stream_k = next(bfq.bfq_get_tile_candidate(i).as_dict() for i in range(bfq.bfq_num_tile_candidates())
                    if bfq.bfq_get_tile_candidate(i).variant == 2)
    bad.write_text(_table([{"N": 4096, "K": 7168, "dtype": "fp8_w8a8", "E": 256,
                            "configs": {"64": stream_k}}]))
    with pytest.raises(bfq.BfqError):
        bfq.bfq_load_tile_table(str(bad))
    bfq.bfq_load_tile_table(None)


def test_probe_validation_without_launch(bfq):
    f = bfq.lib.bfq_probe_mfma_peak
    assert f(4, 10, None, None) == bfq.BFQ_ERR_NULL
    assert f(0, 10, FAKE, None) == bfq.BFQ_ERR_SHAPE
    assert f(4, 0, FAKE, None) == bfq.BFQ_ERR_SHAPE
    assert f(4, 10, FAKE + 2, None) == bfq.BFQ_ERR_ALIGN
    # 8 waves x 8 chains x iters x (2 * 16 * 16 * 128) flops per workgroup
    assert bfq.lib.bfq_probe_mfma_flops(3, 5) == 3 * 8 * 8 * 5 * 65536


def test_noalloc_validation_without_launch(bfq):
    """The allocation-free GEMM validates like bfq_block_gemm and rejects, before any launch,
    explicit tiles whose workspace exceeds its static buffer (stream-K slots, large split-K)."""
    f = bfq.lib.bfq_block_gemm_noalloc
    base = [FAKE, FAKE, 0, 56, FAKE, FAKE, 0, 0, FAKE, 0, 24576, 7168, BS, bfq.BFQ_E4M3FN,
            bfq.BFQ_BF16, None, None]

    def call(**kw):
        a = list(base)
        names = ["a_q", "a_scales", "a_layout", "ld", "w_q", "w_scales", "w_layout", "sfmt",
                 "out", "M", "N", "K", "bs", "qd", "od", "tile", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert bfq.bfq_noalloc_scratch_bytes() == 32 << 20
    assert call() >= 0                                   # M = 0: nothing launched
    assert call(w_q=None) == bfq.BFQ_ERR_NULL
    assert call(K=7000) == bfq.BFQ_ERR_SHAPE
    assert call(w_q=FAKE + 8) == bfq.BFQ_ERR_ALIGN
    cands = [bfq.bfq_get_tile_candidate(i) for i in range(bfq.bfq_num_tile_candidates())]
    sk = next(t for t in cands if t.variant == 2)
    assert call(M=1024, tile=ctypes.pointer(sk)) == bfq.BFQ_ERR_WORKSPACE
    assert "allocation-free" in bfq.last_error()
    t = bfq.bfq_get_tile_candidate(0)
    t.split_k = 4                                        # 4 * 1024 * 24576 * 4 bytes
    assert call(M=1024, tile=ctypes.pointer(t)) == bfq.BFQ_ERR_WORKSPACE
