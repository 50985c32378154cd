"""GPU parity of the quantizers (through the C-ABI) against the CPU oracle: codes and fp32
scales must be bit-exact, with plain fp32 scales and with UE8M0 (power-of-two) scales."""
import numpy as np
import pytest
import torch

from block_scaled_w8a8_amd import synth

pytestmark = pytest.mark.gpu


def _codes_np(t):
    return t.cpu().numpy()


def _gpu_quant_tokens(bfq, x_cpu, qdtype, layout, ld_pad=0, sfmt=0):
    dev = torch.device("cuda:0")
    x = x_cpu.to(dev)
    M, K = x.shape
    if qdtype == bfq.BFQ_E4M3FN:
        q = torch.full((M, K), 0xAA, dtype=torch.uint8, device=dev)   # prefill: unwritten shows
    else:
        q = torch.full((M, K), 77, dtype=torch.int8, device=dev)
    G = K // 128
    if layout == bfq.BFQ_SCALES_ROW_MAJOR:
        s = torch.full((M, G + ld_pad), float("nan"), dtype=torch.float32, device=dev)
    else:
        s = torch.full((G, M + ld_pad), float("nan"), dtype=torch.float32, device=dev)
    bfq.bfq_quant_tokens(x, q, s, layout=layout, scale_ld=s.stride(0), scale_fmt=sfmt)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    s = s[:, :G] if layout == bfq.BFQ_SCALES_ROW_MAJOR else s[:, :M].T.copy()
    return q.cpu().numpy(), s


SHAPES = [(8, 1536), (1, 7168), (24, 1536), (37, 7168), (128, 7168), (64, 18432), (1024, 7168),
          (4096, 7168), (4096, 18432), (3, 128), (5, 640)]


@pytest.mark.parametrize("sfmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_tokens_bit_exact(bfq, orc, M, K, qname, sfmt):
    print(f"quant_tokens M={M} K={K} {qname} {sfmt}", flush=True)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    ot = orc.FP8 if qname == "fp8" else orc.INT8
    sf = 1 if sfmt == "ue8m0" else 0
    x = synth.activations(M, K, seed=M + K)
    qg, sg = _gpu_quant_tokens(bfq, x, qd, bfq.BFQ_SCALES_ROW_MAJOR, sfmt=sf)
    qo, so = orc.quant_groups(synth.bf16_bits(x), qtype=ot, scale_fmt=sf)
    assert np.array_equal(qg.view(np.uint8), qo.view(np.uint8))
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("layout", ["row", "col"])
def test_quant_tokens_layouts_and_ld(bfq, orc, layout):
    M, K = 33, 1536
    lay = bfq.BFQ_SCALES_ROW_MAJOR if layout == "row" else bfq.BFQ_SCALES_COL_MAJOR
    x = synth.activations(M, K, seed=9)
    qg, sg = _gpu_quant_tokens(bfq, x, bfq.BFQ_E4M3FN, lay, ld_pad=5)
    qo, so = orc.quant_groups(synth.bf16_bits(x))
    assert np.array_equal(qg, qo)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))


def _special_input():
    """Rows of bf16 bit patterns covering zero/-0, NaN, +-Inf, subnormal bf16, huge and
    tiny magnitudes, and groups below eps."""
    rng = np.random.default_rng(5)
    M, K = 12, 512
    b = (rng.standard_normal((M, K)).astype(np.float32))
    bits = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    bits[0, :] = 0
    bits[0, 7] = 0x8000                 # -0
    bits[1, 130] = 0x7FC0               # NaN in group 1
    bits[2, 3] = 0x7F80                 # +Inf
    bits[2, 260] = 0xFF80               # -Inf in group 2
    bits[3, :] = rng.integers(0, 0x80, K) | (rng.integers(0, 2, K) << 15)   # bf16 subnormals
    bits[4, :128] = 0x7F7F              # max finite bf16
    bits[4, 1] = 0x0001                 # tiny next to huge
    bits[5, :] = 0x2E00                 # ~2.9e-11: below eps
    bits[6, :] = rng.integers(0, 0x7F80, K) | (rng.integers(0, 2, K) << 15)  # any finite
    bits[7, :] = 0x3F80                 # all 1.0
    bits[8, 0] = 0xFFC1                 # negative NaN with payload
    return bits


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_tokens_special_values(bfq, orc, qname, sfmt):
    bits = _special_input()
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    ot = orc.FP8 if qname == "fp8" else orc.INT8
    qg, sg = _gpu_quant_tokens(bfq, x, qd, bfq.BFQ_SCALES_ROW_MAJOR, sfmt=sfmt)
    qo, so = orc.quant_groups(bits, qtype=ot, scale_fmt=sfmt)
    assert np.array_equal(qg.view(np.uint8), qo.view(np.uint8))
    nan_g, nan_o = np.isnan(sg), np.isnan(so)
    assert np.array_equal(nan_g, nan_o)
    assert np.array_equal(sg[~nan_g].view(np.uint32), so[~nan_o].view(np.uint32))


@pytest.mark.parametrize("sfmt", [0, 1])
@pytest.mark.parametrize("N,K", [(1536, 1536), (7168, 1536), (1536, 7168), (4096, 7168),
                                 (24576, 7168), (256, 384)])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_weight_blocks_bit_exact(bfq, orc, N, K, qname, sfmt):
    if N * K > 50_000_000 and qname == "int8":
        pytest.skip("the large shape is covered by the fp8 case")
    print(f"quant_weight_blocks N={N} K={K} {qname} sfmt={sfmt}", flush=True)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    ot = orc.FP8 if qname == "fp8" else orc.INT8
    w = synth.weights(N, K, seed=N ^ K)
    wg = w.to("cuda:0")
    # sentinel-filled, so an element the kernel fails to write cannot pass on stale memory
    q = torch.full((N, K), 0x55, dtype=torch.uint8 if qname == "fp8" else torch.int8, device="cuda:0")
    s = torch.full((N // 128, K // 128), float("nan"), dtype=torch.float32, device="cuda:0")
    bfq.bfq_quant_weight_blocks(wg, q, s, scale_fmt=sfmt)
    torch.cuda.synchronize()
    qo, so = orc.quant_blocks(w.numpy(), qtype=ot, scale_fmt=sfmt)
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("sfmt", [0, 1])
def test_weight_blocks_special_values(bfq, orc, sfmt):
    w = synth.weights(256, 256, seed=1).numpy().copy()
    w[0:128, 0:128] = 0.0
    w[5, 130] = np.nan
    w[200, 7] = np.inf
    w[201, 8] = -np.inf
    w[130:256, 130:256] *= 1e-30
    wg = torch.from_numpy(w).to("cuda:0")
    q = torch.full((256, 256), 0x55, dtype=torch.uint8, device="cuda:0")
    s = torch.full((2, 2), float("nan"), dtype=torch.float32, device="cuda:0")
    bfq.bfq_quant_weight_blocks(wg, q, s, scale_fmt=sfmt)
    torch.cuda.synchronize()
    qo, so = orc.quant_blocks(w, scale_fmt=sfmt)
    assert np.array_equal(q.cpu().numpy(), qo)
    sg = s.cpu().numpy()
    assert np.array_equal(np.isnan(sg), np.isnan(so))
    assert np.array_equal(sg[~np.isnan(sg)].view(np.uint32), so[~np.isnan(so)].view(np.uint32))


def _encode_class_inputs():
    """Every fp32 value whose top 16 bits take all 2^16 patterns and whose low 16 bits are
    one of {0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF}: the e4m3 rounding decision depends on
    the sign, exponent, the mantissa bits down to the round bit (all within the top 16)
    and on whether any lower bit is set (sticky), and these low patterns give both sticky
    values next to every round-bit state. Restricted to finite |x| < 464."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).ravel()
    x = u.view(np.float32)
    return x[np.isfinite(x) & (np.abs(x) < 464)].copy()


def test_device_fp8_encoder_all_rounding_classes(bfq, orc):
    x = _encode_class_inputs()
    xg = torch.from_numpy(x).to("cuda:0")
    out = torch.full((x.size,), 0x55, dtype=torch.uint8, device="cuda:0")
    bfq.bfq_debug_encode(xg, out, bfq.BFQ_E4M3FN)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = orc.e4m3_encode_array(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:8]]


@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_device_encoder_every_fp32_pattern(bfq, orc, qname):
    """The device encoder on every fp32 bit pattern of its stated domain (e4m3fn: finite with
    |x| < 464, subnormals and both zeros included; int8: every finite value), swept over all
    2^32 patterns in 16 chunks of 2^28, against the oracle's encoder (itself pinned on all
    2^32 patterns to a brute-force search from the format definition): every code equal."""
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    enc = orc.e4m3_encode_array if qname == "fp8" else orc.int8_encode_array
    limit = 0x43E80000 if qname == "fp8" else 0x7F800000    # |x| below 464 / below +Inf
    CH = 1 << 28
    out = torch.empty(CH, dtype=torch.uint8 if qname == "fp8" else torch.int8, device="cuda:0")
    covered = 0
    for hi in range(16):
        start = hi * CH
        print(f"{qname} encoder patterns {start:#010x}..{start + CH - 1:#010x}", flush=True)
        bits = torch.arange(start, start + CH, dtype=torch.int64, device="cuda:0")
        bits = torch.where(bits >= (1 << 31), bits - (1 << 32), bits).to(torch.int32)
        out.fill_(0x55)
        bfq.bfq_debug_encode(bits.view(torch.float32), out, qd)
        torch.cuda.synchronize()
        del bits
        got = out.cpu().numpy()
        u = np.arange(start, start + CH, dtype=np.uint64).astype(np.uint32)
        keep = (u & np.uint32(0x7FFFFFFF)) < np.uint32(limit)
        covered += int(keep.sum())
        ref = enc(u.view(np.float32))
        bad = np.nonzero(keep & (got != ref))[0]
        assert bad.size == 0, [(hex(start + int(i)), int(got[i]), int(ref[i])) for i in bad[:8]]
    expect = 2 * limit
    assert covered == expect, (covered, expect)


def test_device_int8_encoder(bfq, orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([np.arange(-300, 300, 0.25, dtype=np.float32),
                        (rng.standard_normal(1 << 20) * 100).astype(np.float32)])
    xg = torch.from_numpy(x).to("cuda:0")
    out = torch.full((x.size,), 0x55, dtype=torch.int8, device="cuda:0")
    bfq.bfq_debug_encode(xg, out, bfq.BFQ_INT8)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), orc.int8_encode_array(x))


def test_quant_tokens_m0_is_noop(bfq):
    x = torch.empty((0, 1536), dtype=torch.bfloat16, device="cuda:0")
    q = torch.empty((0, 1536), dtype=torch.uint8, device="cuda:0")
    s = torch.empty((0, 12), dtype=torch.float32, device="cuda:0")
    assert bfq.bfq_quant_tokens(x, q, s, scale_ld=12) == bfq.BFQ_OK


# ------------------------------------------------------ packed UE8M0 scale words

@pytest.mark.parametrize("M,K", [(1, 7168), (5, 640), (37, 1536), (128, 7168), (4096, 7168),
                                 (3, 128), (64, 18432)])
@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_tokens_packed_words_bit_exact(bfq, orc, M, K, qname):
    """BFQ_SCALES_PACKED_UE8M0: the words equal the oracle's packing of its UE8M0 scales
    (groups past the last one and rows up to a multiple of 4 zero), the codes equal the
    unpacked quantizer's, and nothing is written past the padded rows."""
    print(f"quant packed M={M} K={K} {qname}", flush=True)
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    qt = orc.FP8 if qname == "fp8" else orc.INT8
    x = synth.activations(M, K, seed=M * 3 + K)
    G, Mp = K // 128, (M + 3) // 4 * 4
    ld = Mp + 3
    dev = torch.device("cuda:0")
    q = torch.full((M, K), 0x55, dtype=torch.uint8 if qname == "fp8" else torch.int8, device=dev)
    words = torch.full(((G + 3) // 4, ld), -1431655766, dtype=torch.int32, device=dev)  # 0xAAAAAAAA
    bfq.bfq_quant_tokens(x.to(dev), q, words, layout=bfq.BFQ_SCALES_PACKED_UE8M0, scale_ld=ld,
                         scale_fmt=bfq.BFQ_SCALE_UE8M0)
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(synth.bf16_bits(x), qtype=qt, scale_fmt=orc.SCALE_UE8M0)
    want = orc.pack_scales_ue8m0(so)
    got = words.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:, :Mp], want)
    assert (got[:, Mp:] == 0xAAAAAAAA).all()
    assert np.array_equal(q.cpu().numpy().view(np.uint8), qo.view(np.uint8))


def test_quant_tokens_packed_special_values(bfq, orc):
    """NaN and Inf groups get code 255 (E8M0 has no infinity); zero and sub-eps groups the
    code of eps / 448 rounded up to a power of two."""
    bits = _special_input()
    M, K = bits.shape
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    q, words = bfq.quant_tokens(x.to("cuda:0"), layout=bfq.BFQ_SCALES_PACKED_UE8M0,
                                scale_fmt=bfq.BFQ_SCALE_UE8M0)
    torch.cuda.synchronize()
    qo, so = orc.quant_groups(bits, scale_fmt=orc.SCALE_UE8M0)
    assert np.array_equal(words.cpu().numpy().view(np.uint32), orc.pack_scales_ue8m0(so))
    assert np.array_equal(q.cpu().numpy(), qo)


def _reciprocal_straddles(orc, qmax, encode, want=24, trials=20000, seed=5):
    """(amax, x) bf16 pairs for which the code of x * fl(1/s) differs from the code of the IEEE
    quotient x / s (s = fl(amax / qmax)): the products land on the other side of a rounding
    midpoint. Found by search over every positive bf16 x <= amax, all in numpy float32."""
    rng = np.random.default_rng(seed)
    allx = ((np.arange(1, 0x7F80, dtype=np.uint32)) << 16).view(np.float32)
    hits = []
    for _ in range(trials):
        amax = np.float32(np.ldexp(rng.uniform(1.0, 2.0), int(rng.integers(-30, 30))))
        amax = (np.array([amax]).view(np.uint32) & 0xFFFF0000).view(np.float32)[0]   # a bf16
        s = np.float32(amax) / np.float32(qmax)
        xs = allx[allx <= amax]
        q = xs / s
        p = xs * (np.float32(1.0) / s)
        bad = np.nonzero(encode(q) != encode(p))[0]
        hits += [(amax, xs[i]) for i in bad[:2]]
        if len(hits) >= want:
            break
    return hits


@pytest.mark.parametrize("qname", ["fp8", "int8"])
def test_quant_tokens_quotients_near_rounding_midpoints(bfq, orc, qname):
    """Groups built so that a reciprocal-multiply would round some elements to the wrong
    code (the values straddle a rounding midpoint between x * (1/s) and x / s): the device
    codes still equal the oracle's IEEE-quotient codes bit for bit."""
    qd = bfq.BFQ_E4M3FN if qname == "fp8" else bfq.BFQ_INT8
    ot = orc.FP8 if qname == "fp8" else orc.INT8
    qmax = 448.0 if qname == "fp8" else 127.0
    enc = orc.e4m3_encode_array if qname == "fp8" else orc.int8_encode_array
    hits = _reciprocal_straddles(orc, qmax, enc)
    assert len(hits) >= 8, len(hits)
    rng = np.random.default_rng(9)
    G = 4
    rows = (len(hits) + G - 1) // G
    x = np.zeros((rows, G * 128), dtype=np.float32)
    for i, (amax, v) in enumerate(hits):
        grp = x[i // G, (i % G) * 128:(i % G + 1) * 128]
        grp[:] = rng.uniform(-1.0, 1.0, 128).astype(np.float32) * amax * 0.9
        grp[0] = amax
        sign = -1.0 if i % 2 else 1.0
        grp[1 + (i % 127)] = sign * v
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert float(xt.float().abs().max()) > 0
    qg, sg = _gpu_quant_tokens(bfq, xt, qd, bfq.BFQ_SCALES_COL_MAJOR)
    qo, so = orc.quant_groups(synth.bf16_bits(xt), qtype=ot)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg.view(np.uint8), qo.view(np.uint8))
