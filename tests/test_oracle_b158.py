"""Pins for the oracle's b1.58 path (CPU only): absmean ternarisation, the int8
activation quantiser, exact accumulation and the rescaling epilogue."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rne(fr: Fraction) -> int:
    n = fr.numerator // fr.denominator
    rem = fr - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2):
        n += 1
    return n


# ----------------------------------------------------------------------------- exact sum / fp32 rounding
def test_exact_abs_sum_against_fraction_and_fsum():
    rg = synth.rng(1, 1)
    W = (rg.standard_normal(3000) * np.exp2(rg.integers(-140, 60, 3000))).astype(np.float32)
    W[:5] = [1e-45, -1e-45, 3e-39, 0.0, -0.0]           # subnormals and zeros
    brute = sum((Fraction(float(v)) for v in np.abs(W.astype(np.float64))), Fraction(0))
    assert oracle.exact_abs_sum(W) == brute
    fs = math.fsum(float(abs(v)) for v in W)
    assert abs(float(brute) - fs) <= math.ulp(fs)


def test_f32_nearest_matches_single_rounding():
    rg = synth.rng(1, 2)
    vals = rg.standard_normal(2000) * np.exp2(rg.integers(-160, 120, 2000))
    for v in vals:
        assert oracle.f32_nearest(Fraction(float(v))) == np.float32(v)
    # exact ties between neighbouring fp32 values round to the even one
    for a in [1.0, 3.0, 1.5e-40, 7.25]:
        lo = np.float32(a)
        hi = np.nextafter(lo, np.float32(np.inf))
        mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
        even = lo if (lo.view(np.uint32) & 1) == 0 else hi
        assert oracle.f32_nearest(mid) == even
    assert np.isinf(oracle.f32_nearest(Fraction(2) ** 128))
    assert oracle.f32_nearest(Fraction(1, 2 ** 151)) == 0.0     # below half the smallest subnormal


# ----------------------------------------------------------------------------- absmean ternarisation
def test_absmean_zero_fraction_closed_form():
    """W ~ N(0, s^2): code 0 iff |W| <= mean|W|/2 = s*sqrt(2/pi)/2, which has
    probability erf(1/(2 sqrt(pi))) ~ 0.3101; +-1 split the rest evenly."""
    W = synth.normal_fp32((512, 512), 0, 1, 0, 0, std=0.02)
    codes, beta = oracle.ternarize_absmean(W)
    n = codes.size
    p0 = math.erf(0.5 / math.sqrt(math.pi))
    sd = math.sqrt(p0 * (1 - p0) / n)
    assert abs(np.count_nonzero(codes == 0) / n - p0) < 5 * sd
    assert abs(np.count_nonzero(codes == 1) / n - (1 - p0) / 2) < 5 * sd
    assert abs(float(beta) - 0.02 * math.sqrt(2 / math.pi)) < 3e-4


def test_absmean_threshold_and_signs():
    W = synth.normal_fp32((256, 192), 0, 1, 0, 1, std=0.02)
    codes, beta = oracle.ternarize_absmean(W)
    assert set(np.unique(codes)) <= {-1, 0, 1}
    exact_mean = oracle.exact_abs_sum(W) / W.size
    assert abs(Fraction(float(beta)) - exact_mean) <= Fraction(float(np.spacing(beta))) / 2
    ratio = np.abs(W.astype(np.float64)) / float(beta)
    clearly_zero = ratio < 0.5 - 1e-6
    clearly_one = ratio > 0.5 + 1e-6
    assert np.all(codes[clearly_zero] == 0)
    assert np.all(codes[clearly_one] == np.sign(W[clearly_one]))


def test_absmean_degenerate():
    codes, beta = oracle.ternarize_absmean(np.zeros((64, 64), np.float32))
    assert beta == 0 and not codes.any()
    W = np.ones((64, 64), np.float32)
    W[3, 3] = np.nan
    codes, beta = oracle.ternarize_absmean(W)
    assert np.isnan(beta) and not codes.any()
    # constant magnitude: beta equals it and every code is the sign
    W = np.where(synth.rng(0, 3).random((64, 64)) < 0.5, -0.75, 0.75).astype(np.float32)
    codes, beta = oracle.ternarize_absmean(W)
    assert beta == np.float32(0.75) and np.array_equal(codes, np.sign(W).astype(np.int8))


def test_absmean_tie_rounds_to_even():
    W = np.tile(np.array([2.0, -2.0, 1.0, 1.0], np.float32), (64, 16))   # mean |W| = 1.5
    codes, beta = oracle.ternarize_absmean(W)
    assert beta == np.float32(1.5) and list(codes[0, :4]) == [1, -1, 1, 1]
    W = np.tile(np.array([1.0, 3.0, 0.5, 1.5], np.float32), (64, 16))    # 3/1.5 = 2 clips to 1
    codes, beta = oracle.ternarize_absmean(W)
    assert beta == np.float32(1.5) and list(codes[0, :4]) == [1, 1, 0, 1]
    W = np.tile(np.array([0.5, 1.5, 1.0, 1.0], np.float32), (64, 16))    # mean 1: 0.5 is a tie -> 0
    codes, beta = oracle.ternarize_absmean(W)
    assert beta == 1.0 and list(codes[0, :4]) == [0, 1, 1, 1]


# ----------------------------------------------------------------------------- int8 activations
def test_quant_worked_ties():
    """gamma = 127 makes 127 x / gamma == x exactly, so the codes are x rounded
    half to even and clipped to [-127, 127]."""
    x = np.array([[127, 0.5, 1.5, 2.5, -2.5, 3.5, -127, -0.5]], dtype=np.float16)
    q, gamma, rowsum = oracle.quant_act_int8(x)
    assert gamma[0] == 127
    assert list(q[0]) == [127, 0, 2, 2, -2, 4, -127, 0]
    assert rowsum[0] == sum([127, 0, 2, 2, -2, 4, -127, 0])


def test_quant_matches_exact_rational_rounding():
    """q = rne(correctly rounded fp32 of 127 x / gamma), checked with exact rationals."""
    rg = synth.rng(2, 1)
    all16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = all16[np.isfinite(all16)]
    for gamma in [np.float16(65504), np.float16(1.0), np.float16(3.140625), np.float16(6.1035e-05),
                  np.float16(127), np.float16(0.0999)]:
        cand = finite[np.abs(finite.astype(np.float32)) <= np.float32(gamma)]
        xs = rg.choice(cand, size=min(1500, cand.size), replace=False)
        x = np.stack([xs, np.full_like(xs, gamma)], axis=1)            # rows [x, gamma]
        q, g, _ = oracle.quant_act_int8(x)
        assert np.all(g == np.float32(gamma))
        for xv, qv in zip(xs, q[:, 0]):
            r = Fraction(127) * Fraction(float(xv)) / Fraction(float(gamma))
            assert qv == max(-127, min(127, _rne(Fraction(float(oracle.f32_nearest(r))))))


def test_quant_properties():
    x = synth.normal_fp16((16, 512), 0, 2, 0)
    q, gamma, rowsum = oracle.quant_act_int8(x)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    assert np.all(gamma == np.abs(x.astype(np.float32)).max(axis=1))
    arg = np.abs(x.astype(np.float32)).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(16), arg]) == 127)
    qn, gn, _ = oracle.quant_act_int8(-x)
    assert np.array_equal(qn, -q) and np.array_equal(gn, gamma)
    r = x.astype(np.float64) * 127 / gamma.astype(np.float64)[:, None]
    assert np.all(np.abs(r - q) <= 0.5 + 1e-6)
    assert np.array_equal(rowsum, q.astype(np.int64).sum(axis=1))


def test_quant_degenerate_rows():
    x = np.zeros((3, 64), dtype=np.float16)
    x[1, 5] = np.float16(np.inf)
    x[2, :] = 1
    x[2, 7] = np.float16(np.nan)
    q, gamma, rowsum = oracle.quant_act_int8(x)
    assert gamma[0] == 0 and np.isnan(gamma[1]) and np.isnan(gamma[2])
    assert not q.any() and not rowsum.any()


# ----------------------------------------------------------------------------- accumulation and output
def test_acc_brute_force_tiny():
    rg = synth.rng(3, 1)
    q = rg.integers(-127, 128, size=(3, 64)).astype(np.int8)
    w = rg.integers(-1, 2, size=(5, 64)).astype(np.int8)
    acc = oracle.acc_exact(q, w)
    for m in range(3):
        for n in range(5):
            assert acc[m, n] == sum(int(q[m, k]) * int(w[n, k]) for k in range(64))


def test_acc_identities():
    rg = synth.rng(3, 2)
    K = 28672
    q = np.full((2, K), 127, dtype=np.int8)
    q[1] = -127
    w = np.ones((3, K), dtype=np.int8)
    w[2] = -1
    acc = oracle.acc_exact(q, w)                         # extremes: +-127*K fits int32
    assert acc[0, 0] == 127 * K and acc[1, 2] == 127 * K and acc[1, 0] == -127 * K
    q = rg.integers(-127, 128, size=(4, 640)).astype(np.int8)
    w = synth.ternary_codes(7, 96, 640)
    assert np.array_equal(oracle.acc_exact(q, np.ones((1, 640), np.int8))[:, 0], q.astype(np.int64).sum(1))
    onehot = np.zeros((1, 640), np.int8)
    onehot[0, 321] = 127
    assert np.array_equal(oracle.acc_exact(onehot, w)[0], 127 * w[:, 321].astype(np.int64))
    assert np.array_equal(oracle.acc_exact(q, w), (q.astype(np.int64) @ w.astype(np.int64).T))


def test_bitlinear_reproduces_float_product_when_exactly_representable():
    """With W = c * (+-1) the absmean codes are the signs and beta = c; with integer x
    whose row max is 127 the codes are x itself. The layer must then equal the
    plain float product x W^T exactly: this pins both scalings together."""
    rg = synth.rng(4, 1)
    x = rg.integers(-127, 128, size=(8, 512)).astype(np.float16)
    x[:, 3] = 127
    W = (np.where(rg.random((64, 512)) < 0.5, -1.0, 1.0) * 0.03125).astype(np.float32)
    codes, beta = oracle.ternarize_absmean(W)
    y, acc, q, gamma = oracle.bitlinear_forward(x, codes, beta)
    assert np.array_equal(q, x.astype(np.int8)) and beta == np.float32(0.03125)
    assert np.array_equal(y, x.astype(np.float64) @ W.astype(np.float64).T)


def test_bitlinear_config1_dequantised_product():
    x = synth.normal_fp16((8, 512), 0, 1, 0, 10)
    W = synth.normal_fp32((512, 512), 0, 1, 0, 11, std=0.02)
    codes, beta = oracle.ternarize_absmean(W)
    y, acc, q, gamma = oracle.bitlinear_forward(x, codes, beta)
    xd = q.astype(np.float64) * (gamma.astype(np.float64)[:, None] / 127)
    wd = codes.astype(np.float64) * float(beta)
    np.testing.assert_allclose(y, xd @ wd.T, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    # and the quantised layer tracks the float layer it stands in for
    yf = x.astype(np.float64) @ W.astype(np.float64).T
    corr = np.corrcoef(y.ravel(), yf.ravel())[0, 1]
    assert corr > 0.85


def test_ternary_bits_golden():
    g = json.load(open(os.path.join(GOLDEN, "b158_bits.json")))
    assert round(math.log2(g["levels"]), g["printed_decimals"]) == g["bits_printed"]
