"""Pins of the CPU oracle against things other than itself (CPU only, "not gpu").

Each test names what fixes the expected value: the e4m3fn format definition, a library
codec (torch.float8_e4m3fn, numpy int64/fp64 matmul), brute force, closed forms, exact
special cases, or figures printed on the pages.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _f(v):
    return float(v) if not isinstance(v, str) else float(v)


# ------------------------------------------------------------------------ codec

def test_decode_all_codes_format_definition(orc):
    """P1: decode follows the format (subnormals m*2^-9, normals (8+m)*2^(E-10)), is
    strictly increasing over 0x00..0x7E and mirrors in sign; 0x7F/0xFF are NaN."""
    vals = [orc.e4m3_decode(c) for c in range(256)]
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert vals[0x7E] == 448.0 and vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9
    assert vals[0x07] == 7 * 2.0 ** -9 and vals[0x38] == 1.0 and vals[0x00] == 0.0
    pos = vals[:0x7F]
    assert all(b > a for a, b in zip(pos, pos[1:]))
    for c in range(0x7F):
        assert vals[c | 0x80] == -vals[c]
    assert np.signbit(vals[0x80])


def test_decode_matches_torch_float8(orc):
    """P1: decode equals the library codec torch.float8_e4m3fn on all 256 codes."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.e4m3_decode(c) for c in range(256)])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(ref[~both_nan], got[~both_nan])


def test_roundtrip_all_codes(orc):
    """P1: every non-NaN code decodes and re-encodes to itself (including -0 = 0x80)."""
    for c in range(256):
        v = orc.e4m3_decode(c)
        if np.isnan(v):
            assert orc.e4m3_encode(np.float32("nan")) == 0x7F
            continue
        assert orc.e4m3_encode(np.float32(v)) == c, hex(c)


def test_worked_encodings(orc):
    """P3: worked encodings derived from the format definition (tests/golden)."""
    g = json.load(open(os.path.join(GOLDEN, "e4m3_worked.json")))
    for case in g["cases"]:
        assert orc.e4m3_encode(np.float32(_f(case["x"]))) == int(case["code"], 16), case
    for case in g["int8_cases"]:
        assert orc.int8_encode(np.float32(_f(case["x"]))) == case["code"], case


def test_encode_matches_torch_in_range(orc):
    """P2 (library): within |x| <= 464 the saturating reading and torch's non-saturating
    float8_e4m3fn cast agree; compare on every bf16 pattern in range and on fp32 values
    that sit on, just above and just below each rounding midpoint."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 464)]
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    v = v[np.isfinite(v)]
    v = np.unique(v)
    mids = ((v[1:].astype(np.float64) + v[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf))])
    near = near[np.abs(near) <= 464]
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(200000) * 50).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 464]
    allx = np.concatenate([x, near, -near, rnd])
    ref = torch.from_numpy(allx).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_encode_array(allx)
    assert np.array_equal(got, ref)


def test_encode_exhaustive_bruteforce(orc, tmp_path):
    """P2 (brute force): all 2^32 fp32 patterns against a nearest-value search written
    from the format definition (tests/native/e4m3_exhaustive.c)."""
    exe = tmp_path / "e4m3_exhaustive"
    src = os.path.join(HERE, "native", "e4m3_exhaustive.c")
    libdir = os.path.dirname(orc.LIB_PATH)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-std=c11", "-o", str(exe), src, "-L" + libdir,
                    "-loracle", "-Wl,-rpath," + libdir, "-lm"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stderr


def test_int8_encode_library(orc):
    """int8 codes equal numpy's round-half-even (np.rint) clamped to [-127, 127]."""
    rng = np.random.default_rng(1)
    y = np.concatenate([(rng.standard_normal(100000) * 80).astype(np.float32),
                        np.arange(-300, 300, 0.5, dtype=np.float32)])
    ref = np.clip(np.rint(y.astype(np.float64)), -127, 127).astype(np.int8)
    assert np.array_equal(orc.int8_encode_array(y), ref)


def test_bf16_rne_library(orc):
    """bf16 rounding equals torch's float32 -> bfloat16 cast (round to nearest even)."""
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 1e3,
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.f32_to_bf16_bits_array(x), ref)


# ------------------------------------------------------------------ quantizers

def _dequant_fp8(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def test_group_quant_invariants(orc):
    """P4: per group, scale = amax/448 (amax from numpy), the largest |code| is 0x7E
    (decodes to 448), and every code is the e4m3 value nearest to x/scale (brute force
    over all 254 finite codes)."""
    x = synth.activations(6, 1536, seed=3)
    bits = synth.bf16_bits(x)
    q, s = orc.quant_groups(bits)
    xf = x.float().numpy().reshape(6, 12, 128)
    amax = np.abs(xf).max(axis=2)
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    mags = (q.reshape(6, 12, 128) & 0x7F).max(axis=2)
    assert (mags == 0x7E).all()
    codes = np.arange(256, dtype=np.uint8)
    vals = _dequant_fp8(codes)
    finite = np.isfinite(vals)
    y = (xf / s[:, :, None]).astype(np.float32).astype(np.float64).ravel()
    deq = _dequant_fp8(q).ravel()
    # nearest: no finite code is strictly closer to y than the chosen one
    dist = np.abs(vals[finite][None, :] - y[:, None]).min(axis=1)
    assert np.array_equal(np.abs(deq - y), dist)


def test_group_quant_dequant_error_bound(orc):
    """P4: |dec(q)*s - x| <= half a code step: 2^-4 |x| for normal codes, 2^-10 s below."""
    x = synth.activations(16, 7168, seed=4)
    q, s = orc.quant_groups(synth.bf16_bits(x))
    xf = x.double().numpy()
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(_dequant_fp8(q) * srep - xf)
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * srep) * (1 + 1e-6)
    assert (err <= bound).all()


def test_group_quant_special_groups(orc):
    """All-zero group -> codes 0 and scale eps/448; -0 keeps its sign; a NaN group gets a
    NaN scale and NaN codes; an Inf group gets an Inf scale, signed-zero codes and NaN
    codes for the infinities; int8: max |q| = 127 and scale = amax/127."""
    x = np.zeros((4, 256), dtype=np.float32)
    x[0, 5] = -0.0
    x[1, :128] = np.linspace(-3, 3, 128)
    x[1, 200] = np.nan
    x[2, 3] = np.inf
    x[2, 4] = -2.0
    x[2, 130] = -np.inf
    x[3, :] = np.linspace(-1, 5, 256)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bits = bits.copy()
    bits[0, 5] = 0x8000
    q, s = orc.quant_groups(bits)
    eps = np.float32(1e-10)
    assert s[0, 0] == np.float32(eps / np.float32(448)) and s[0, 1] == s[0, 0]
    assert q[0, 5] == 0x80 and (np.delete(q[0], 5) == 0).all()
    assert np.isnan(s[1, 1]) and (q[1, 128:] == 0x7F).all() and not np.isnan(s[1, 0])
    assert np.isinf(s[2, 0]) and np.isinf(s[2, 1])
    assert q[2, 3] == 0x7F and q[2, 4] == 0x80 and q[2, 130] == 0x7F and q[2, 0] == 0x00
    qi, si = orc.quant_groups(bits, qtype=orc.INT8)
    assert np.abs(qi[3]).max() == 127 and si[3, 1] == np.float32(np.float32(5.0) / np.float32(127))
    assert (qi[1, 128:] == 0).all() and np.isnan(si[1, 1])


def test_block_quant_invariants(orc):
    """P4 for weight blocks: scale = block amax / 448, one 0x7E-magnitude code per block
    at least, and codes nearest to w/scale (checked by the dequant error bound)."""
    w = synth.weights(256, 384, seed=5).numpy()
    q, s = orc.quant_blocks(w)
    blocks = w.reshape(2, 128, 3, 128).transpose(0, 2, 1, 3)
    amax = np.abs(blocks).max(axis=(2, 3))
    assert np.array_equal(s, (amax / np.float32(448)).astype(np.float32))
    qb = q.reshape(2, 128, 3, 128).transpose(0, 2, 1, 3)
    assert ((qb & 0x7F).max(axis=(2, 3)) == 0x7E).all()
    srep = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)
    err = np.abs(_dequant_fp8(q) * srep - w)
    assert (err <= np.maximum(2.0 ** -4 * np.abs(w), 2.0 ** -10 * srep) * (1 + 1e-6)).all()
    qi, si = orc.quant_blocks(w, qtype=orc.INT8)
    assert np.abs(qi).max() == 127


# ------------------------------------------------------------------------ GEMM

def _quantized_case(M, N, K, seed, qtype):
    import oracle as orc
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), qtype=qtype)
    qw, sw = orc.quant_blocks(w, qtype=qtype)
    return qa, sa, qw, sw


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 384), (8, 128, 384), (8, 256, 128)])
def test_gemm_vs_fp64_dequant_matmul(orc, M, N, K):
    """P5: against an fp64 dequantize-then-matmul written with library routines (torch's
    e4m3fn decode, numpy fp64 matmul): |C32 - D| <= 1e-5 * rms(D)."""
    qa, sa, qw, sw = _quantized_case(M, N, K, 7, orc.FP8)
    c32, c16 = orc.block_gemm(qa, sa, qw, sw)
    a = _dequant_fp8(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    b = _dequant_fp8(qw) * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    d = a @ b.T
    rms = np.sqrt((d * d).mean())
    assert np.abs(c32 - d).max() <= 1e-5 * rms
    # the oracle's own brute force agrees with the library one
    assert np.abs(orc.dequant_gemm_f64(qa, sa, qw, sw) - d).max() <= 1e-12 * rms


def test_gemm_exact_integer_case(orc):
    """P6: codes restricted to e4m3 integers |v| <= 8 and every scale 2^-4: every partial
    sum is an integer multiple of 2^-8 below 2^24 ulps, so any correct evaluation equals
    the integer matmul (numpy int64) times 2^-8 exactly, and bf16 out = torch's RNE cast."""
    rng = np.random.default_rng(11)
    ints = np.arange(-8, 9)
    enc = {int(v): torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
           for v in ints}
    M, N, K = 5, 256, 512
    ia = rng.integers(-8, 9, size=(M, K))
    iw = rng.integers(-8, 9, size=(N, K))
    qa = np.vectorize(enc.get)(ia).astype(np.uint8)
    qw = np.vectorize(enc.get)(iw).astype(np.uint8)
    sa = np.full((M, K // 128), 2.0 ** -4, dtype=np.float32)
    sw = np.full((N // 128, K // 128), 2.0 ** -4, dtype=np.float32)
    c32, c16 = orc.block_gemm(qa, sa, qw, sw)
    exact = (ia.astype(np.int64) @ iw.T.astype(np.int64)).astype(np.float64) * 2.0 ** -8
    assert np.array_equal(c32.astype(np.float64), exact)
    ref16 = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(c16, ref16.numpy().view(np.uint16))


def test_gemm_one_hot_rows(orc):
    """P6: a token row that is the code 1.0 at column k (scale 1) reproduces the weight
    column k dequantized: C[m, n] = fp32(dec(qw[n, k]) * sw[n/128, k/128])."""
    _, _, qw, sw = _quantized_case(1, 256, 384, 13, orc.FP8)
    M, K = 4, 384
    ks = [0, 127, 200, 383]
    qa = np.zeros((M, K), dtype=np.uint8)
    for m, k in enumerate(ks):
        qa[m, k] = 0x38
    sa = np.ones((M, K // 128), dtype=np.float32)
    c32, _ = orc.block_gemm(qa, sa, qw, sw)
    for m, k in enumerate(ks):
        ref = (_dequant_fp8(qw[:, k]).astype(np.float32) * np.repeat(sw[:, k // 128], 128))
        assert np.array_equal(c32[m], ref.astype(np.float32))


def test_int8_partials_vs_numpy(orc):
    """P7: int8 per-block int32 partials equal numpy int64 matmuls of the code blocks."""
    qa, sa, qw, sw = _quantized_case(7, 256, 512, 17, orc.INT8)
    part = orc.block_partials_i32(qa, qw)
    for kb in range(4):
        ref = qa[:, kb * 128:(kb + 1) * 128].astype(np.int64) @ \
            qw[:, kb * 128:(kb + 1) * 128].astype(np.int64).T
        assert np.array_equal(part[kb].astype(np.int64), ref)
    # and the int8 GEMM is the exact partials rescaled: compare with fp64 dequant matmul
    c32, _ = orc.block_gemm(qa, sa, qw, sw, qtype=orc.INT8)
    d = orc.dequant_gemm_f64(qa, sa, qw, sw, qtype=orc.INT8)
    a = qa.astype(np.float64) * np.repeat(sa.astype(np.float64), 128, axis=1)
    b = qw.astype(np.float64) * np.repeat(np.repeat(sw.astype(np.float64), 128, 0), 128, 1)
    assert np.abs(d - a @ b.T).max() <= 1e-12 * np.abs(d).max()
    assert np.abs(c32 - d).max() <= 1e-5 * np.sqrt((d * d).mean())


def test_gemm_sampled_matches_full(orc):
    qa, sa, qw, sw = _quantized_case(9, 384, 256, 19, orc.FP8)
    c32, _ = orc.block_gemm(qa, sa, qw, sw)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, 9, 100)
    ns = rng.integers(0, 384, 100)
    assert np.array_equal(orc.block_gemm_sampled(qa, sa, qw, sw, ms, ns), c32[ms, ns])


def test_calc_diff_closed_forms():
    """calc_diff (block GEMM benchmark page §4.4): 0 for equal tensors, 2 for x vs -x,
    1 - 2*2/(1+4) = 0.2 for x vs 2x."""
    from oracle.metrics import calc_diff
    x = np.random.default_rng(3).standard_normal(1000)
    assert calc_diff(x, x) == pytest.approx(0.0, abs=1e-15)
    assert calc_diff(x, -x) == pytest.approx(2.0)
    assert calc_diff(x, 2 * x) == pytest.approx(0.2)


def test_calc_diff_matches_pages_accuracy(orc):
    """P8: on the pages' setup (randn bf16 A (64, 7168) and B (4096, 7168), seed 42, B per
    128x128 block and A per 1x128 group quantized to e4m3fn, C_ref = bf16 A @ B^T) the
    pages print an average calc_diff of 0.000684 for all three kernels (block GEMM benchmark
    page §3.3). The oracle's bf16 output must land at that level: [6.0e-4, 7.7e-4]."""
    from oracle.metrics import bf16_bits_to_f32, calc_diff
    g = torch.Generator().manual_seed(42)
    m, n, k = 64, 4096, 7168
    A = torch.randn((m, k), generator=g).to(torch.bfloat16)
    B = torch.randn((n, k), generator=g).to(torch.bfloat16)
    c_ref = (A @ B.t()).float().numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(A))
    qw, sw = orc.quant_blocks(B.float().numpy())
    _, c16 = orc.block_gemm(qa, sa, qw, sw)
    d = calc_diff(bf16_bits_to_f32(c16), c_ref)
    assert 6.0e-4 <= d <= 7.7e-4, d


# ------------------------------------------------------------------ selection

def test_nearest_m_rule_pages_examples():
    """P9: the config page's examples (M=37 -> 32, M=2050 -> 2048) and tie/end cases."""
    from oracle.select import nearest_bucket
    g = json.load(open(os.path.join(GOLDEN, "nearest_m.json")))
    for m, want in g["examples"] + g["ties"] + g["ends"]:
        assert nearest_bucket(m, g["grid"]) == want, (m, want)


# ------------------------------------------------------------------ packed weight layout

def test_pack16_is_the_stated_byte_map(orc):
    """The packed 16-row fragment layout, read back byte by byte with a plain loop that
    decodes each destination offset (fragment, half, lane, byte) into a source row and
    column, agrees with the vectorized oracle on a shape with several fragments per row
    group and several row groups."""
    N, K = 48, 384
    rng = np.random.default_rng(7)
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    p = orc.pack16(w).ravel()
    KB = K // 128
    for d in range(N * K):
        frag, within = divmod(d, 2048)
        f, kb = divmod(frag, KB)
        h, rest = divmod(within, 1024)
        lane, b = divmod(rest, 16)
        assert p[d] == w[16 * f + lane % 16, 128 * kb + 64 * h + 16 * (lane // 16) + b], d


def test_pack16_permutation_and_fragment_contents(orc):
    """pack16 applied to an array of source positions is a permutation of them; every 2 KB
    fragment holds exactly one 16-row x 128-column block; and each lane's two 16-byte slots
    (one per half) come from a single row — the row the lane feeds to a 16-row MFMA."""
    N, K = 64, 512
    KB = K // 128
    pos = np.arange(N * K, dtype=np.int64).reshape(N, K)
    p = orc.pack16(pos).ravel()
    assert np.array_equal(np.sort(p), np.arange(N * K))
    rows, cols = p // K, p % K
    for frag in range(N * K // 2048):
        f, kb = divmod(frag, KB)
        sl = slice(frag * 2048, (frag + 1) * 2048)
        assert set(rows[sl]) == set(range(16 * f, 16 * f + 16))
        assert set(cols[sl]) == set(range(128 * kb, 128 * kb + 128))
        for lane in range(64):
            a = frag * 2048 + 16 * lane
            lane_rows = np.concatenate([rows[a:a + 16], rows[a + 1024:a + 1040]])
            assert np.all(lane_rows == 16 * f + lane % 16)


# ------------------------------------------------------------------ UE8M0 scales

def _group_with_amax(amax, k=1536):
    """One token row whose first 128-group has absolute maximum `amax` (exact in bf16)."""
    row = np.zeros((1, k), dtype=np.float32)
    row[0, :128] = np.linspace(-amax, amax / 2, 128, dtype=np.float32)
    row[0, 7] = -amax
    t = torch.from_numpy(row).to(torch.bfloat16)
    assert float(t.float().abs()[0, :128].max()) == amax
    return synth.bf16_bits(t)


def test_ue8m0_worked_scales(orc):
    """Worked UE8M0 scales (tests/golden/ue8m0_worked.json): the block GEMM benchmark page
    §4.1 rounds amax / fp8_max up to a power of two when use_ue8m0 is set."""
    g = json.load(open(os.path.join(GOLDEN, "ue8m0_worked.json")))
    for c in g["cases"]:
        qt = orc.FP8 if c["qmax"] == 448 else orc.INT8
        _, s = orc.quant_groups(_group_with_amax(c["amax"]), qtype=qt, scale_fmt=orc.SCALE_UE8M0)
        assert float(s[0, 0]) == c["scale"], c
        # the fp32 format of the same group is the plain quotient
        _, s32 = orc.quant_groups(_group_with_amax(c["amax"]), qtype=qt)
        t = np.float32(max(c["amax"], 1e-10)) / np.float32(c["qmax"])
        assert s32[0, 0] == t, c


@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_ue8m0_group_and_block_invariants(orc, qname):
    """UE8M0 scales on outlier-laden activations and on weights: every scale is a power of
    two s with s/2 < t <= s for t = amax/Qmax (numpy fp32 quotient); every code is the
    nearest code to x/s (fp8: brute force over the 254 finite codes; int8: numpy rint +
    clip); amax/s lies in (Qmax/2, Qmax], so the largest |code| of a group decodes into
    [Qmax/2, Qmax] (rounding can land on Qmax/2 itself, e.g. 225 -> 224)."""
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    qmax = np.float32(448 if qname == "fp8" else 127)
    x = synth.activations(6, 1536, seed=8)
    q, s = orc.quant_groups(synth.bf16_bits(x), qtype=qt, scale_fmt=orc.SCALE_UE8M0)
    xf = x.float().numpy().reshape(6, 12, 128)
    t = (np.abs(xf).max(axis=2) / qmax).astype(np.float32)
    mant, _ = np.frexp(s)
    assert (mant == 0.5).all()
    assert ((s / 2 < t) & (t <= s)).all()
    y = (xf / s[:, :, None]).astype(np.float32)
    if qname == "fp8":
        vals = _dequant_fp8(np.arange(256, dtype=np.uint8))
        fin = vals[np.isfinite(vals)]
        deq = _dequant_fp8(q).reshape(6, 12, 128)
        dist = np.abs(fin[None, :] - y.astype(np.float64).ravel()[:, None]).min(axis=1)
        assert np.array_equal(np.abs(deq.ravel() - y.astype(np.float64).ravel()), dist)
        top = np.abs(deq).max(axis=2)
    else:
        want = np.clip(np.rint(y), -127, 127).astype(np.int8)
        assert np.array_equal(q.reshape(6, 12, 128), want)
        top = np.abs(q.reshape(6, 12, 128).astype(np.float64)).max(axis=2)
    assert ((top >= qmax / 2) & (top <= qmax)).all()
    w = synth.weights(256, 384, seed=9).numpy()
    qw, sw = orc.quant_blocks(w, qtype=qt, scale_fmt=orc.SCALE_UE8M0)
    tw = (np.abs(w.reshape(2, 128, 3, 128)).max(axis=(1, 3)) / qmax).astype(np.float32)
    assert (np.frexp(sw)[0] == 0.5).all() and ((sw / 2 < tw) & (tw <= sw)).all()


def test_ue8m0_calc_diff_matches_pages_accuracy(orc):
    """The pages' accuracy setup as printed (block GEMM benchmark page §4.1): B quantized per
    128x128 block with use_ue8m0=True, A per 1x128 group with plain fp32 scales, randn bf16
    operands seed 42, m=64, n=4096, k=7168; the page prints an average calc_diff of
    0.000684 (§3.3). The oracle lands in [6.0e-4, 7.7e-4]; with UE8M0 scales on both sides
    too (the fully power-of-two format) it stays in that band."""
    from oracle.metrics import bf16_bits_to_f32, calc_diff
    g = torch.Generator().manual_seed(42)
    m, n, k = 64, 4096, 7168
    A = torch.randn((m, k), generator=g).to(torch.bfloat16)
    B = torch.randn((n, k), generator=g).to(torch.bfloat16)
    c_ref = (A @ B.t()).float().numpy()
    qw, sw = orc.quant_blocks(B.float().numpy(), scale_fmt=orc.SCALE_UE8M0)
    for a_fmt in (orc.SCALE_FP32, orc.SCALE_UE8M0):
        qa, sa = orc.quant_groups(synth.bf16_bits(A), scale_fmt=a_fmt)
        _, c16 = orc.block_gemm(qa, sa, qw, sw)
        d = calc_diff(bf16_bits_to_f32(c16), c_ref)
        assert 6.0e-4 <= d <= 7.7e-4, (a_fmt, d)


# ------------------------------------------- per-token x per-channel formats
# Helion linear-backend page, scope section: FP8_Dynamic and W8A8_INT8 scale activations per
# token and weights per output channel. The oracle reaches them through group = K (tokens)
# and block = (1, K) (channels) of the same quantizers, and through channel_gemm.

@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_token_quant_invariants(orc, qname):
    """Per token: scale = row amax / Qmax (amax from numpy), the largest |code| of each row
    is the top code (0x7E / 127), codes within half a step of x / scale, and an all-zero row
    gets codes 0 and scale eps / Qmax."""
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    Q = np.float32(448 if qname == "fp8" else 127)
    M, K = 6, 1536
    x = synth.activations(M, K, seed=21)
    bits = synth.bf16_bits(x).copy()
    bits[5] = 0
    q, s = orc.quant_groups(bits, group=K, qtype=qt)
    assert s.shape == (M, 1)
    xf = x.float().numpy()
    xf[5] = 0
    amax = np.abs(xf).max(axis=1)
    assert np.array_equal(s[:5, 0], (amax[:5] / Q).astype(np.float32))
    assert s[5, 0] == np.float32(np.float32(1e-10) / Q) and (q[5] == 0).all()
    if qt == orc.FP8:
        assert ((q[:5] & 0x7F).max(axis=1) == 0x7E).all()
        deq = _dequant_fp8(q)
        bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * s.astype(np.float64))
    else:
        assert (np.abs(q[:5].astype(np.int32)).max(axis=1) == 127).all()
        deq = q.astype(np.float64)
        bound = 0.5 * s.astype(np.float64) * np.ones_like(xf, dtype=np.float64)
    err = np.abs(deq * s.astype(np.float64) - xf)
    assert (err <= bound * (1 + 1e-6)).all()


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_token_scale_is_max_of_group_scales(orc, fmt):
    """max(amax, eps) / Qmax and the rounding up to a power of two are monotonic, so a token's
    scale is the largest of its 1x128 group scales, and every group whose scale equals it
    gets the same codes in both granularities."""
    sf = orc.SCALE_FP32 if fmt == "fp32" else orc.SCALE_UE8M0
    M, K = 8, 7168
    bits = synth.bf16_bits(synth.activations(M, K, seed=22))
    qg, sg = orc.quant_groups(bits, qtype=orc.FP8, scale_fmt=sf)
    qt, st = orc.quant_groups(bits, group=K, qtype=orc.FP8, scale_fmt=sf)
    assert np.array_equal(st[:, 0], sg.max(axis=1))
    hits = 0
    for m in range(M):
        for g in np.nonzero(sg[m] == st[m, 0])[0]:
            assert np.array_equal(qt[m, g * 128:(g + 1) * 128], qg[m, g * 128:(g + 1) * 128])
            hits += 1
    assert hits >= M


def test_token_quant_worked_values(orc):
    """Worked from the definition: a row whose largest magnitude is 896 has scale 2 (fp8),
    so 1.0 encodes as 0.5 (0x30) and 896 as 448 (0x7E); int8 with amax 254 has scale 2,
    3.0 -> 1.5 -> 2 (ties to even) and 5.0 -> 2.5 -> 2."""
    x = np.ones((2, 256), dtype=np.float32)
    x[0, 17] = -896.0
    x[1, :] = 0.0
    x[1, 3], x[1, 4], x[1, 200] = 3.0, 5.0, 254.0
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = orc.quant_groups(bits.copy(), group=256, qtype=orc.FP8)
    assert s[0, 0] == 2.0 and q[0, 17] == 0xFE and q[0, 0] == 0x30
    qi, si = orc.quant_groups(bits.copy(), group=256, qtype=orc.INT8)
    assert si[1, 0] == 2.0 and qi[1, 3] == 2 and qi[1, 4] == 2 and qi[1, 200] == 127


def test_channel_quant_invariants(orc):
    """Per output channel (block 1 x K): scale = row amax / 448, top code in every row, codes
    within half a step; int8 max |q| = 127 per row."""
    N, K = 256, 1536
    w = synth.weights(N, K, seed=23).numpy()
    q, s = orc.quant_blocks(w, block=(1, K))
    assert s.shape == (N, 1)
    assert np.array_equal(s[:, 0], (np.abs(w).max(axis=1) / np.float32(448)).astype(np.float32))
    assert ((q & 0x7F).max(axis=1) == 0x7E).all()
    err = np.abs(_dequant_fp8(q) * s.astype(np.float64) - w)
    assert (err <= np.maximum(2.0 ** -4 * np.abs(w), 2.0 ** -10 * s.astype(np.float64)) * (1 + 1e-6)).all()
    qi, si = orc.quant_blocks(w, block=(1, K), qtype=orc.INT8)
    assert (np.abs(qi.astype(np.int32)).max(axis=1) == 127).all()


def _channel_case(M, N, K, seed, qtype):
    import oracle as orc
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), group=K, qtype=qtype)
    qw, sw = orc.quant_blocks(w, block=(1, K), qtype=qtype)
    return qa, sa[:, 0].copy(), qw, sw[:, 0].copy()


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 384), (8, 128, 1536)])
def test_channel_gemm_vs_fp64_dequant_matmul(orc, M, N, K):
    """Against an fp64 dequantize-then-matmul from library routines (torch's e4m3fn decode,
    numpy fp64 matmul): |C32 - D| <= 1e-5 * rms(D)."""
    qa, sa, qw, sw = _channel_case(M, N, K, 24, orc.FP8)
    c32, c16 = orc.channel_gemm(qa, sa, qw, sw)
    d = (_dequant_fp8(qa) * sa.astype(np.float64)[:, None]) @ \
        (_dequant_fp8(qw) * sw.astype(np.float64)[:, None]).T
    assert np.abs(c32 - d).max() <= 1e-5 * np.sqrt((d * d).mean())
    ref16 = torch.from_numpy(c32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(c16, ref16)


def test_channel_gemm_exact_integer_case(orc):
    """Codes restricted to e4m3 integers |v| <= 8, token scales 2^-(m mod 3) and channel
    scales 2^-(n mod 4): every step is exact in fp32, so the result is the numpy int64 matmul
    times the two powers of two exactly. Scales that differ per row and per column catch a
    transposed or mis-indexed scale."""
    rng = np.random.default_rng(25)
    enc = {int(v): torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
           for v in range(-8, 9)}
    M, N, K = 6, 256, 1024
    ia = rng.integers(-8, 9, size=(M, K))
    iw = rng.integers(-8, 9, size=(N, K))
    qa = np.vectorize(enc.get)(ia).astype(np.uint8)
    qw = np.vectorize(enc.get)(iw).astype(np.uint8)
    ea = -(np.arange(M) % 3)
    ew = -(np.arange(N) % 4)
    sa = (2.0 ** ea).astype(np.float32)
    sw = (2.0 ** ew).astype(np.float32)
    c32, _ = orc.channel_gemm(qa, sa, qw, sw)
    exact = (ia.astype(np.int64) @ iw.T.astype(np.int64)).astype(np.float64)
    exact *= (2.0 ** ea)[:, None] * (2.0 ** ew)[None, :]
    assert np.array_equal(c32.astype(np.float64), exact)


def test_channel_gemm_int8_is_rounded_exact_dot(orc):
    """int8: the dot product over the whole K is the numpy int64 matmul, rounded once to
    fp32 and scaled token-then-channel; sums beyond 2^24 exercise that single rounding."""
    qa, sa, qw, sw = _channel_case(4, 128, 7168, 26, orc.INT8)
    rng = np.random.default_rng(26)
    qa[2:] = rng.integers(60, 128, size=(2, 7168)).astype(np.int8)   # same-sign rows:
    qw[64:] = rng.integers(60, 128, size=(64, 7168)).astype(np.int8)  # sums near 6e7
    c32, _ = orc.channel_gemm(qa, sa, qw, sw, qtype=orc.INT8)
    p = qa.astype(np.int64) @ qw.astype(np.int64).T
    assert np.abs(p).max() > 2 ** 24 and (p.astype(np.float32).astype(np.int64) != p).any()
    ref = (p.astype(np.float32) * sa[:, None]).astype(np.float32) * sw[None, :]
    assert np.array_equal(c32, ref.astype(np.float32))


def test_channel_gemm_agrees_with_block_gemm(orc):
    """With every group of a token sharing its scale and every 128 channels sharing one
    scale, the block-scaled GEMM computes the same quantity by another summation order."""
    qa, sa, qw, sw = _channel_case(5, 256, 768, 27, orc.FP8)
    sw = np.repeat(sw.reshape(2, 128)[:, :1], 128, axis=1).reshape(-1).copy()
    c_ch, _ = orc.channel_gemm(qa, sa, qw, sw)
    sa_b = np.repeat(sa[:, None], 768 // 128, axis=1)
    sw_b = np.repeat(sw.reshape(2, 128)[:, :1], 768 // 128, axis=1)
    c_bl, _ = orc.block_gemm(qa, sa_b, qw, sw_b)
    rms = np.sqrt((c_bl.astype(np.float64) ** 2).mean())
    assert np.abs(c_ch.astype(np.float64) - c_bl).max() <= 1e-5 * rms


def test_channel_gemm_sampled_matches_full(orc):
    qa, sa, qw, sw = _channel_case(9, 384, 256, 28, orc.INT8)
    c32, _ = orc.channel_gemm(qa, sa, qw, sw, qtype=orc.INT8)
    rng = np.random.default_rng(1)
    ms = rng.integers(0, 9, 100)
    ns = rng.integers(0, 384, 100)
    assert np.array_equal(orc.channel_gemm_sampled(qa, sa, qw, sw, ms, ns, qtype=orc.INT8), c32[ms, ns])


# --------------------------------------------------------- packed UE8M0 scale words
# Per-token-group kernel page (output_s_packed): four UE8M0 bytes per 32-bit word, words
# token-major, token count padded to a multiple of 4.

def test_pack_scales_worked_values(orc):
    """From the E8M0 definition (value 2^(code - 127)): 1 -> 127, 2 -> 128, 0.5 -> 126,
    2^-42 -> 85, 2^10 -> 137, NaN -> 255; byte j of a word holds group 4w + j."""
    s = np.array([[1.0, 2.0, 0.5, 2.0 ** -42, 2.0 ** 10, np.nan]], dtype=np.float32)
    words = orc.pack_scales_ue8m0(s)
    assert words.shape == (2, 4)
    assert words[0, 0] == 127 | (128 << 8) | (126 << 16) | (85 << 24)
    assert words[1, 0] == 137 | (255 << 8)          # groups 6, 7 past G: zero bytes
    assert (words[:, 1:] == 0).all()                # rows 1..3 pad to a multiple of 4


def test_pack_scales_round_trip_and_padding(orc):
    """On quantizer output: decoding every byte with numpy ldexp gives back the scales; bytes
    past the last group and rows past M are zero; a wider ld only adds untouched columns."""
    M, K = 13, 7 * 128
    _, s = orc.quant_groups(synth.bf16_bits(synth.activations(M, K, seed=31)),
                            scale_fmt=orc.SCALE_UE8M0)
    G = s.shape[1]
    words = orc.pack_scales_ue8m0(s)
    assert words.shape == (2, 16)
    codes = np.stack([(words >> (8 * j)) & 0xFF for j in range(4)], axis=1)  # [w, j, m]
    codes = codes.transpose(2, 0, 1).reshape(16, 8)[:, :G]                    # [m, g]
    assert np.array_equal(np.ldexp(1.0, codes[:M].astype(np.int64) - 127), s.astype(np.float64))
    assert (codes[M:] == 0).all() and ((words[1] >> 24) == 0).all()
    wide = orc.pack_scales_ue8m0(s, ld=21)
    assert np.array_equal(wide[:, :16], words) and (wide[:, 16:] == 0).all()


# ------------------------------------------------------------ MoE grouped GEMM
# Config page §5: the MoE kernels' tables add an expert count E. Pairs q = t*topk + j are
# grouped by expert; each pair's output row is its token's block GEMM with its expert.

def test_moe_align_is_a_stable_sort_by_expert(orc):
    """Against numpy: a stable argsort of the flat expert ids and a bincount prefix."""
    for T, E, topk, seed in [(1, 8, 2, 0), (37, 16, 4, 1), (300, 256, 8, 2), (5, 3, 1, 3)]:
        ids = synth.routing(T, E, topk, seed=seed).numpy()
        off, srt = orc.moe_align(ids, E)
        flat = ids.reshape(-1)
        assert np.array_equal(srt, np.argsort(flat, kind="stable").astype(np.int32))
        cnt = np.bincount(flat, minlength=E)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32))
        # each token's experts are distinct
        assert all(len(set(r)) == topk for r in ids.tolist())
    off, srt = orc.moe_align(np.zeros((0, 4), np.int32), 6)
    assert (off == 0).all() and srt.size == 0


def _moe_case(orc, T, E, topk, N, K, seed, qtype=0):
    x = synth.activations(T, K, seed=seed)
    ids = synth.routing(T, E, topk, seed=seed).numpy()
    w = synth.expert_weights(E, N, K, seed=seed).numpy()
    qa, sa = orc.quant_groups(synth.bf16_bits(x), qtype=qtype)
    qs = [orc.quant_blocks(w[e], qtype=qtype) for e in range(E)]
    return qa, sa, ids, np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])


def test_moe_gemm_vs_fp64_per_pair(orc):
    """Every pair row against an fp64 dequantize-then-matmul of its token with its expert
    (torch's e4m3fn decode, numpy fp64): within 1e-5 rms."""
    qa, sa, ids, qw, sw = _moe_case(orc, 9, 6, 3, 256, 384, 41)
    c = orc.moe_gemm(qa, sa, ids, qw, sw)
    a = _dequant_fp8(qa) * np.repeat(sa.astype(np.float64), 128, axis=1)
    for q in range(9 * 3):
        t, e = q // 3, ids[q // 3, q % 3]
        b = _dequant_fp8(qw[e]) * np.repeat(np.repeat(sw[e].astype(np.float64), 128, 0), 128, 1)
        d = a[t] @ b.T
        assert np.abs(c[q] - d).max() <= 1e-5 * np.sqrt((d * d).mean()), q


def test_moe_gemm_exact_integer_case(orc):
    """Integer codes |v| <= 8 and power-of-two scales that differ per expert: bit-exact with
    numpy int64 matmuls of each token with its expert, times the scales."""
    rng = np.random.default_rng(42)
    T, E, topk, N, K = 7, 5, 2, 128, 256
    enc = {int(v): torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
           for v in range(-8, 9)}
    ia = rng.integers(-8, 9, size=(T, K))
    iw = rng.integers(-8, 9, size=(E, N, K))
    qa = np.vectorize(enc.get)(ia).astype(np.uint8)
    qw = np.vectorize(enc.get)(iw).astype(np.uint8)
    sa = np.full((T, K // 128), 2.0 ** -3, dtype=np.float32)
    sw = np.stack([np.full((N // 128, K // 128), 2.0 ** -(e + 1), dtype=np.float32) for e in range(E)])
    ids = synth.routing(T, E, topk, seed=42).numpy()
    c = orc.moe_gemm(qa, sa, ids, qw, sw)
    for q in range(T * topk):
        t, e = q // topk, ids[q // topk, q % topk]
        exact = (iw[e].astype(np.int64) @ ia[t].astype(np.int64)).astype(np.float64)
        assert np.array_equal(c[q].astype(np.float64), exact * 2.0 ** -3 * 2.0 ** -(e + 1)), q


def test_moe_gemm_single_expert_is_the_block_gemm(orc):
    """E = 1, topk = 1: the grouped GEMM is the plain block GEMM, bit for bit; sampled
    outputs equal the full ones."""
    qa, sa, ids, qw, sw = _moe_case(orc, 11, 1, 1, 256, 512, 43)
    c = orc.moe_gemm(qa, sa, ids, qw, sw)
    c_dense, _ = orc.block_gemm(qa, sa, qw[0], sw[0])
    assert np.array_equal(c, c_dense)
    qa, sa, ids, qw, sw = _moe_case(orc, 9, 4, 2, 128, 256, 44, qtype=orc.INT8)
    c = orc.moe_gemm(qa, sa, ids, qw, sw, qtype=orc.INT8)
    rng = np.random.default_rng(2)
    qs, ns = rng.integers(0, 18, 60), rng.integers(0, 128, 60)
    assert np.array_equal(orc.moe_gemm_sampled(qa, sa, ids, qw, sw, qs, ns, qtype=orc.INT8),
                          c[qs, ns])
