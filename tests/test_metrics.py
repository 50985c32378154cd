"""Pins of the parity checker (oracle/metrics.py) -- the functions that decide pass/fail for
every GEMM parity test. Each case is built so that a plausible lenient mistake in the checker
fails it: 'or' for 'and' between the two bounds, a missing absolute value, the element bound
taken from the output instead of the reference, a missing relative-Frobenius test, an
inverted or missing rounding-midpoint (straddle) test, and a step count that admits two bf16
steps. The bar itself (relative Frobenius <= 1e-3, max |diff| <= 2^-7 * rms(ref) + 1e-3) is
the tolerance stated for the GEMM outputs; calc_diff is the accuracy measure of the block GEMM
benchmark page (§4.4)."""
import numpy as np
import pytest
import torch

from oracle import metrics


def _bf16(x):
    """bf16 bits of fp32 values, round to nearest even (torch's conversion)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ elementary helpers

def test_rms_and_bound_closed_forms():
    assert metrics.rms([3.0, 4.0]) == pytest.approx(np.sqrt(12.5), rel=1e-15)
    assert metrics.rms(np.full(10, -2.0)) == 2.0
    assert metrics.rms(np.zeros(0)) == 0.0
    ref = np.array([3.0, -4.0])
    assert metrics.max_diff_bound(ref) == pytest.approx(np.sqrt(12.5) / 128 + 1e-3, rel=1e-15)
    assert metrics.max_diff_bound(np.zeros(5)) == 1e-3


def test_rel_frobenius_closed_forms():
    ref = np.array([3.0, 4.0])
    assert metrics.rel_frobenius(ref, ref) == 0.0
    assert metrics.rel_frobenius(ref * 1.5, ref) == pytest.approx(0.5, rel=1e-14)
    # ||(0, 1)|| / ||(3, 4)|| = 1/5, whichever way the difference points
    assert metrics.rel_frobenius([3.0, 5.0], ref) == pytest.approx(0.2, rel=1e-14)
    assert metrics.rel_frobenius([3.0, 3.0], ref) == pytest.approx(0.2, rel=1e-14)
    # the norm is the reference's, not the output's: (6, 8) vs (3, 4) is 1, not 0.5
    assert metrics.rel_frobenius([6.0, 8.0], ref) == pytest.approx(1.0, rel=1e-14)
    # a zero reference falls back to the output's norm
    assert metrics.rel_frobenius([3.0, 4.0], [0.0, 0.0]) == 5.0


def test_max_abs_diff_takes_the_absolute_value():
    ref = np.zeros(4)
    assert metrics.max_abs_diff([0.0, -3.0, 1.0, 0.0], ref) == 3.0
    assert metrics.max_abs_diff(np.zeros(0), np.zeros(0)) == 0.0


def test_calc_diff_closed_forms():
    x = np.array([1.0, -2.0, 3.0])
    assert metrics.calc_diff(x, x) == pytest.approx(0.0, abs=1e-15)
    assert metrics.calc_diff(x, -x) == pytest.approx(2.0, rel=1e-15)
    assert metrics.calc_diff(x, np.zeros(3)) == pytest.approx(1.0, rel=1e-15)
    # 1 - 2*<x,y> / (|x|^2 + |y|^2) with x = (1, 0), y = (1, 1): 1 - 2/3
    assert metrics.calc_diff([1.0, 0.0], [1.0, 1.0]) == pytest.approx(1.0 / 3.0, rel=1e-14)


# ------------------------------------------------------------------ fp32 report

N = 100_000
REF = np.ones(N)                       # rms 1, element bound 1/128 + 1e-3
BOUND = 1.0 / 128 + 1e-3


def test_fp32_report_exact_match_passes():
    r = metrics.gemm_fp32_report(REF.copy(), REF)
    assert r["ok"] and r["rel_frobenius"] == 0.0 and r["max_abs_diff"] == 0.0
    assert r["max_diff_bound"] == pytest.approx(BOUND, rel=1e-15)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_fp32_report_one_element_past_the_bound_fails(sign):
    """One element just past 2^-7*rms+1e-3 (either sign) fails although the relative
    Frobenius error stays ~3e-5: the two bounds are both required."""
    out = REF.copy()
    out[5] += sign * BOUND * (1 + 1e-6)
    r = metrics.gemm_fp32_report(out, REF)
    assert r["rel_frobenius"] < 1e-4 and not r["ok"], r
    out[5] = REF[5] + sign * BOUND * (1 - 1e-6)
    assert metrics.gemm_fp32_report(out, REF)["ok"]


def test_fp32_report_relative_frobenius_just_past_1e3_fails():
    """A uniform relative error of 1.01e-3 keeps every element far inside the element bound
    (1.01e-3 < 8.8e-3) and must still fail; 0.99e-3 passes."""
    r = metrics.gemm_fp32_report(REF * (1 + 1.01e-3), REF)
    assert r["max_abs_diff"] < BOUND and not r["ok"], r
    assert metrics.gemm_fp32_report(REF * (1 + 0.99e-3), REF)["ok"]


def test_fp32_report_bound_comes_from_the_reference():
    """The output's rms exceeds the reference's by 5e-4 relative; one element lies between
    the bound computed from the reference (fails) and one computed from the output (would
    pass)."""
    out = REF * (1 + 5e-4)
    d = 0.008814                          # 0.0088125 (ref bound) < d < 0.0088164 (out bound)
    out[0] = 1.0 + d
    assert metrics.max_diff_bound(REF) < d < metrics.max_diff_bound(out)
    r = metrics.gemm_fp32_report(out, REF)
    assert r["rel_frobenius"] < 1e-3 and not r["ok"], r


# ------------------------------------------------------------------ bf16 straddle report

def _straddle_case(ref32_0, gpu32_0, out16_0=None, n=100_000, bg=2.0):
    """n elements of bg (2.0) plus one large element at index 0 whose bf16 step (0.5 at 100)
    exceeds the element bound (rms ~2.0 -> bound ~0.017) while one such step keeps the
    relative Frobenius error at ~8e-4."""
    ref32 = np.full(n, bg, dtype=np.float32)
    gpu32 = ref32.copy()
    ref32[0], gpu32[0] = ref32_0, gpu32_0
    r16 = _bf16(ref32)
    o16 = _bf16(gpu32)
    if out16_0 is not None:
        o16[0] = _bf16([out16_0])[0]
    return o16, r16, gpu32, ref32


def test_straddle_exact_match_passes():
    o16, r16, g32, r32 = _straddle_case(100.24, 100.24)
    r = metrics.bf16_straddle_report(o16, r16, g32, r32)
    assert r["ok"] and r["beyond_bound"] == 0, r


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_straddle_one_step_explained_by_the_midpoint_passes(sign):
    """Oracle fp32 100.24 rounds to 100.0, GPU fp32 100.26 to 100.5: one bf16 step, beyond
    the element bound, and the midpoint 100.25 lies between the two fp32 values."""
    o16, r16, g32, r32 = _straddle_case(sign * 100.24, sign * 100.26)
    assert abs(int(o16[0]) - int(r16[0])) == 1
    r = metrics.bf16_straddle_report(o16, r16, g32, r32)
    assert r["ok"] and r["beyond_bound"] == 1 and r["unexplained"] == 0, r


def test_straddle_one_step_without_a_straddle_fails():
    """The GPU's bf16 is one step up (100.5) while both fp32 values (100.1, 100.2) lie below
    the midpoint 100.25: a rounding the fp32 values do not explain."""
    o16, r16, g32, r32 = _straddle_case(100.1, 100.2, out16_0=100.5)
    r = metrics.bf16_straddle_report(o16, r16, g32, r32)
    assert r["beyond_bound"] == 1 and r["unexplained"] == 1 and not r["ok"], r


def test_straddle_two_steps_fails():
    """Two bf16 steps (oracle 100.2 -> 100.0, GPU 100.8 -> 101.0) fail although the midpoint
    of the two bf16 values (100.5) lies between the fp32 values and the relative Frobenius
    error (a background of 4.0 keeps it at ~8e-4) passes: only the step count rejects it."""
    o16, r16, g32, r32 = _straddle_case(100.2, 100.8, bg=4.0)
    assert abs(int(o16[0]) - int(r16[0])) == 2
    r = metrics.bf16_straddle_report(o16, r16, g32, r32)
    assert r["rel_frobenius"] < 1e-3 and not r["ok"] and r["unexplained"] == 1, r


def test_straddle_relative_frobenius_is_required():
    """Every element one bf16 step off (7.8e-3 at 1.0, inside the element bound 8.8e-3, so no
    element is 'beyond'): the relative Frobenius error 7.8e-3 alone must fail it."""
    ref32 = np.ones(1000, dtype=np.float32)
    gpu32 = np.full(1000, 1.0 + 2.0 ** -7, dtype=np.float32)
    r = metrics.bf16_straddle_report(_bf16(gpu32), _bf16(ref32), gpu32, ref32)
    assert r["beyond_bound"] == 0 and not r["ok"], r
