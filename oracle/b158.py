"""BitNet b1.58 linear layer: absmean ternary weights, per-token absmax int8 activations.

ORACLE — test infrastructure only (see the package docstring).

Source [b158], "BitNet b1.58 介绍": every weight is one of -1, 0, +1; activations
are scaled per token into [-Q_b, Q_b] with no zero point; BitLinear stands in for
nn.Linear with no bias. "实验及结果" (energy paragraph, Fig. 3): the matrix
product then needs only int8 additions. The page prints neither quantiser
formula; the readings used here are:

* weights: beta = mean |W| over the whole tensor (one scale per tensor), codes
  = clip(round(W / beta), -1, 1). beta is the fp32 value nearest the exact mean;
  the division and the rounding are done in fp32 (round half to even), the
  precision the kernel decides the code in.
* activations: Q_b = 127; gamma_m = max_k |x_mk|; q = clip(rne(fl32(fl32(127 x) / gamma)), -127, 127).
  127 x is exact in fp32 for fp16 x, so there is a single rounding (the division).
* output: y_mn = acc_mn * (gamma_m / Q_b) * beta_n, the inverse of both scalings.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

QB = 127  # [b158] activation range [-Q_b, Q_b]; Q_b = 127 for 8-bit activations


# ------------------------------------------------------------------------------------------
# exact mean of |W| and its nearest fp32 value
# ------------------------------------------------------------------------------------------
def exact_abs_sum(W: np.ndarray) -> Fraction:
    """Exact sum of |W| for a finite fp32 array, as a Fraction.

    Each fp32 magnitude is m * 2^(e-150) with an integer significand m < 2^24
    (subnormals: e = 1 and no hidden bit). Summing the integers m per exponent is
    exact in int64 for fewer than 2^39 elements; the per-exponent totals are then
    combined exactly with Python integers. Parity: pinned against a Fraction sum
    of every element and against math.fsum."""
    a = np.abs(np.asarray(W, dtype=np.float32)).ravel()
    assert np.isfinite(a).all()
    bits = a.view(np.uint32)
    e = (bits >> np.uint32(23)).astype(np.int64)
    m = (bits & np.uint32(0x7FFFFF)).astype(np.int64)
    m = np.where(e > 0, m | 0x800000, m)
    e = np.where(e > 0, e, 1)
    total = 0                                   # in units of 2^-149
    for ev in np.unique(e):
        total += int(m[e == ev].sum()) << (int(ev) - 1)
    return Fraction(total, 1 << 149)


def f32_nearest(v: Fraction) -> np.float32:
    """The fp32 value nearest to the rational v (ties to even); overflow gives inf.

    Written from IEEE 754 binary32: 24-bit significands, minimum normal exponent
    -126, subnormal spacing 2^-149. Parity: pinned against NumPy's fp64->fp32
    conversion (a single correct rounding) on exact fp64 inputs and ties."""
    v = Fraction(v)
    if v == 0:
        return np.float32(0.0)
    sign = -1 if v < 0 else 1
    v = abs(v)
    e = v.numerator.bit_length() - v.denominator.bit_length()   # 2^e <= v < 2^(e+2)
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    q = max(e, -126) - 23                      # spacing of fp32 values around v is 2^q
    scaled = v / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * Fraction(2) ** q
    if value >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(value))     # exact: value is an fp32 number


def absmean_beta(W: np.ndarray) -> np.float32:
    """beta = the fp32 value nearest mean |W|; NaN if W holds a non-finite value."""
    W = np.asarray(W, dtype=np.float32)
    if W.size == 0 or not np.isfinite(W).all():
        return np.float32(np.nan)
    return f32_nearest(exact_abs_sum(W) / W.size)


def ternarize_absmean(W: np.ndarray):
    """Float W [N, K] -> (int8 codes in {-1,0,1} [N, K], fp32 beta).

    beta == 0 or non-finite gives all-zero codes (the division would be undefined).
    Parity: pinned by the closed-form zero fraction of a Gaussian, the threshold
    characterisation |W/beta| <= 1/2 <=> code 0, and sign agreement."""
    W = np.asarray(W, dtype=np.float32)
    beta = absmean_beta(W)
    if not np.isfinite(beta) or beta == 0:
        return np.zeros(W.shape, dtype=np.int8), beta
    r = W / beta                                  # fp32 IEEE division
    return np.clip(np.rint(r), -1, 1).astype(np.int8), beta


# ------------------------------------------------------------------------------------------
# per-token absmax int8 activations
# ------------------------------------------------------------------------------------------
def quant_act_int8(x16: np.ndarray):
    """fp16 x [M, K] -> (int8 q [M, K], fp32 gamma [M], int32 rowsum [M]).

    Rows holding a non-finite value get gamma = NaN and q = 0 (their outputs are
    then NaN); all-zero rows get gamma = 0 and q = 0. Parity: pinned by a worked
    tie example, the correctly rounded fp32 quotient (checked against exact
    rationals), |q| <= 127, odd symmetry and the absmax element mapping to +-127."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)   # exact widening
    M, K = x.shape
    q = np.zeros((M, K), dtype=np.int8)
    gamma = np.zeros(M, dtype=np.float32)
    for m in range(M):
        row = x[m]
        if not np.isfinite(row).all():
            gamma[m] = np.nan
            continue
        g = np.max(np.abs(row)) if K else np.float32(0)
        gamma[m] = g
        if g == 0:
            continue
        v = row * np.float32(QB)                  # exact
        r = v / g                                 # one IEEE fp32 rounding
        q[m] = np.clip(np.rint(r), -QB, QB).astype(np.int8)
    rowsum = q.astype(np.int64).sum(axis=1).astype(np.int32)
    return q, gamma, rowsum


# ------------------------------------------------------------------------------------------
# integer accumulation and the rescaling epilogue
# ------------------------------------------------------------------------------------------
def acc_exact(q: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k codes[n, k] * q[m, k], exact, returned as int32 [M, N].

    Uses an fp64 matrix product: every partial sum is an integer of magnitude at
    most 127*K < 2^53, so no rounding can occur. Parity: pinned against a
    brute-force triple loop and int64 products on small shapes."""
    q = np.asarray(q, dtype=np.int8)
    codes = np.asarray(codes, dtype=np.int8)
    K = q.shape[1]
    assert codes.shape[1] == K and QB * K < 2 ** 31
    a = q.astype(np.float64) @ codes.astype(np.float64).T
    out = a.astype(np.int64)
    assert np.all(out == a)
    return out.astype(np.int32)


def bitlinear_output(acc: np.ndarray, gamma: np.ndarray, beta) -> np.ndarray:
    """y[m, n] = acc[m, n] * (gamma_m / Q_b) * beta_n in fp64 (beta scalar or [N])."""
    beta = np.broadcast_to(np.asarray(beta, dtype=np.float64), (acc.shape[1],))
    return acc.astype(np.float64) * (gamma.astype(np.float64)[:, None] / QB) * beta[None, :]


def bitlinear_forward(x16: np.ndarray, codes: np.ndarray, beta):
    """The whole b1.58 linear: quantise x, accumulate, rescale. Returns (y fp64, acc, q, gamma)."""
    q, gamma, _ = quant_act_int8(x16)
    acc = acc_exact(q, codes)
    return bitlinear_output(acc, gamma, beta), acc, q, gamma
