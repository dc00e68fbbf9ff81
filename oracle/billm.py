"""Residual binarisation as an inference format (BiLLM's salient-weight scheme).

ORACLE — test infrastructure only (see the package docstring).

Source [billm], "方法细节", step 2 (binary residual approximation): binarise W
once (alpha_o * B_o), binarise the residual again (alpha_r * B_r) and use the
sum; the page states the residual scheme's error never exceeds direct
binarisation's. "存储位开销分析" gives the bit cost of a salient fraction r:
N_param = 2r + 1*(1 - r) bits per weight (two sign planes on salient weights,
one elsewhere) and N_storing = 1 + 1/b_size for the group flags.

Readings (the page prints no formula for alpha or the precision):
* groups are (output row, block of 128 consecutive inputs); the format applies the
  residual to every weight (the salient-column search needs calibration data);
* B = sign(.) with sign(0) = +1 (bit set iff the value is negative);
* alpha is the mean magnitude over the group (the least-squares scale of a sign
  approximation): the fp32 value nearest the exact mean, i.e. an exact sum and one
  rounding (ties to even), the same rule as the absmean weight scale. No summation
  order is part of the definition. A group holding NaN gets alpha = NaN; one holding
  inf (and no NaN) alpha = inf, as any IEEE sum of the magnitudes would;
* R = fl32(W - alpha_o * B_o) (alpha_o * B_o = +-alpha_o is exact; one rounding);
* activations stay fp16, unquantised (BiLLM quantises weights only).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128


def exact_group_abs_sums(a: np.ndarray) -> list:
    """Exact sums of |a| over the last axis of a finite fp32 array, one Python int per
    group, in units of 2^-149.

    Each magnitude is m * 2^(e-150) with an integer significand m < 2^24 (subnormals:
    e = 1 and no hidden bit), i.e. m << (e-1) units. That integer is split into 32-bit
    limbs at fixed bit positions; per group and limb the pieces (each < 2^32) are summed
    in int64, exactly, and the limbs are joined as a Python int. Parity: pinned against
    ``exact_abs_sum`` (a per-exponent Fraction sum) row by row."""
    a = np.abs(np.asarray(a, dtype=np.float32))
    G = a.reshape(-1, a.shape[-1])
    assert np.isfinite(G).all()
    bits = G.view(np.uint32).astype(np.int64)
    e = bits >> 23
    m = np.where(e > 0, (bits & 0x7FFFFF) | 0x800000, bits & 0x7FFFFF)
    p = np.maximum(e, 1) - 1                    # weight of m's lowest bit, in units
    limb = p >> 5
    v = m << (p & 31)                           # < 2^55: limb `limb` and limb + 1
    lo, hi = v & 0xFFFFFFFF, v >> 32
    totals = [0] * G.shape[0]
    for j in np.union1d(np.unique(limb), np.unique(limb) + 1):
        part = np.where(limb == j, lo, 0).sum(axis=1) + np.where(limb + 1 == j, hi, 0).sum(axis=1)
        for g in np.nonzero(part)[0]:
            totals[g] += int(part[g]) << (32 * int(j))
    return totals


def f32_nearest_dyadic(S: int, k: int) -> np.float32:
    """The fp32 value nearest to S * 2^-k for an integer S >= 0 (ties to even).

    Written from IEEE 754 binary32: a 24-bit significand, so the spacing near a value
    whose leading bit is 2^(P-k) is 2^(P-k-23), never finer than the subnormal spacing
    2^-149. Parity: pinned against ``f32_nearest`` (Fraction arithmetic) on random,
    subnormal, tie and carry cases."""
    if S == 0:
        return np.float32(0.0)
    P = S.bit_length() - 1
    shift = max(P - 23, k - 149)                # drop `shift` low bits of S
    if shift <= 0:
        mant, shift = S, 0
    else:
        mant = S >> shift
        rem = S - (mant << shift)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (mant & 1)):
            mant += 1
    value = math.ldexp(mant, shift - k)         # exact in fp64 (mant <= 2^24)
    return np.float32(value) if value < 2.0 ** 128 else np.float32(np.inf)


def group_abs_mean_f32(a: np.ndarray) -> np.ndarray:
    """fp32 [..., 128] -> fp32 [...]: the fp32 value nearest the exact mean of |a| over
    the last axis (one rounding, ties to even); NaN in a group gives NaN, inf (without
    NaN) gives inf."""
    a = np.asarray(a, dtype=np.float32)
    assert a.shape[-1] == BLOCK
    flat = np.abs(a.reshape(-1, BLOCK))
    out = np.empty(flat.shape[0], dtype=np.float32)
    has_nan = np.isnan(flat).any(axis=1)
    has_inf = np.isinf(flat).any(axis=1) & ~has_nan
    fin = ~(has_nan | has_inf)
    out[has_nan], out[has_inf] = np.nan, np.inf
    idx = np.nonzero(fin)[0]
    sums = exact_group_abs_sums(flat[idx]) if idx.size else []
    for i, S in zip(idx, sums):
        out[i] = f32_nearest_dyadic(S, 149 + 7)   # mean = S * 2^-149 / 2^7
    return out.reshape(a.shape[:-1])


def _sign(a):
    return np.where(a < 0, np.float32(-1), np.float32(1))


def residual_binarize(W: np.ndarray):
    """W fp32 [N, K] -> (B_o int8 [N, K], alpha_o fp32 [N, K/128], B_r, alpha_r).

    Parity: the group means are pinned against exact rational means (Fraction sums and
    correctly rounded division), constructed ties and constant-magnitude groups; the
    format by exact recovery of constant-magnitude groups (alpha_r = 0) and the
    never-worse-than-direct property."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % BLOCK == 0
    Wb = W.reshape(N, K // BLOCK, BLOCK)
    Bo = _sign(Wb)
    ao = group_abs_mean_f32(Wb)
    with np.errstate(invalid="ignore"):
        R = Wb - ao[:, :, None] * Bo                  # fp32, one rounding per element
    Br = _sign(R)
    ar = group_abs_mean_f32(R)
    return (Bo.reshape(N, K).astype(np.int8), ao, Br.reshape(N, K).astype(np.int8), ar)


def residual_forward(x: np.ndarray, Bo, ao, Br, ar) -> np.ndarray:
    """y = x @ (alpha_o ⊙ B_o + alpha_r ⊙ B_r)^T in fp64 (x fp16 or float).

    Parity: pinned against an explicitly formed dequantised matrix."""
    Wd = (np.repeat(np.asarray(ao, np.float64), BLOCK, axis=1) * Bo +
          np.repeat(np.asarray(ar, np.float64), BLOCK, axis=1) * Br)
    return np.asarray(x, dtype=np.float64) @ Wd.T


def residual_error_scale(x: np.ndarray, ao, ar) -> np.ndarray:
    """Per-element error scale sum_b (|alpha_o| + |alpha_r|)[n, b] * sum_{k in b} |x_mk|.

    It bounds |y| itself (each |x_k| is multiplied by |alpha_o| + |alpha_r| at most), so a
    bound of 1e-3 times it holds for any fp32 summation order at these K. Parity: pinned by
    closed forms (constant scales: 2 * sum |x|; one nonzero group) in the CPU tests."""
    xa = np.abs(np.asarray(x, dtype=np.float64))
    M, K = xa.shape
    xb = xa.reshape(M, K // BLOCK, BLOCK).sum(axis=2)              # [M, KB]
    return xb @ (np.abs(np.asarray(ao, np.float64)) + np.abs(np.asarray(ar, np.float64))).T


def billm_storage_bits_per_param(r_salient: float, block: int):
    """(N_param, N_storing) from the page's bit-cost formulas."""
    return 2 * r_salient + 1 * (1 - r_salient), 1 + 1 / block
