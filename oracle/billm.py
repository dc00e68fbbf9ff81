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
* alpha is the mean magnitude over the group, the least-squares scale of a sign
  approximation, computed in fp32 as a balanced pairwise sum over the group's inputs in
  order (pairs (0,1), (2,3), ..., then pairs of pairs) times 1/128. B_r depends on alpha_o
  through R = W - alpha_o * B_o, so both sides compute alpha in this same fp32 order;
* R = fl32(W - alpha_o * B_o) (alpha_o * B_o = +-alpha_o is exact; one rounding);
* activations stay fp16, unquantised (BiLLM quantises weights only).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def pairwise_sum_f32(a: np.ndarray) -> np.ndarray:
    """Balanced pairwise fp32 sum over the last axis (length a power of two), in order."""
    a = np.asarray(a, dtype=np.float32)
    while a.shape[-1] > 1:
        a = a[..., 0::2] + a[..., 1::2]
    return a[..., 0]


def _sign(a):
    return np.where(a < 0, np.float32(-1), np.float32(1))


def residual_binarize(W: np.ndarray):
    """W fp32 [N, K] -> (B_o int8 [N, K], alpha_o fp32 [N, K/128], B_r, alpha_r).

    Parity: pinned by the exact-rational bound of the pairwise sums, exact recovery of
    constant-magnitude groups and the never-worse-than-direct property."""
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % BLOCK == 0
    Wb = W.reshape(N, K // BLOCK, BLOCK)
    Bo = _sign(Wb)
    ao = pairwise_sum_f32(np.abs(Wb)) * np.float32(1.0 / BLOCK)
    R = Wb - ao[:, :, None] * Bo                      # fp32, one rounding per element
    Br = _sign(R)
    ar = pairwise_sum_f32(np.abs(R)) * np.float32(1.0 / BLOCK)
    return (Bo.reshape(N, K).astype(np.int8), ao, Br.reshape(N, K).astype(np.int8), ar)


def residual_forward(x: np.ndarray, Bo, ao, Br, ar) -> np.ndarray:
    """y = x @ (alpha_o ⊙ B_o + alpha_r ⊙ B_r)^T in fp64 (x fp16 or float)."""
    Wd = (np.repeat(np.asarray(ao, np.float64), BLOCK, axis=1) * Bo +
          np.repeat(np.asarray(ar, np.float64), BLOCK, axis=1) * Br)
    return np.asarray(x, dtype=np.float64) @ Wd.T


def residual_error_scale(x: np.ndarray, ao, ar) -> np.ndarray:
    """Per-element error scale sum_b (|alpha_o| + |alpha_r|)[n, b] * sum_{k in b} |x_mk|."""
    xa = np.abs(np.asarray(x, dtype=np.float64))
    M, K = xa.shape
    xb = xa.reshape(M, K // BLOCK, BLOCK).sum(axis=2)              # [M, KB]
    return xb @ (np.abs(np.asarray(ao, np.float64)) + np.abs(np.asarray(ar, np.float64))).T


def billm_storage_bits_per_param(r_salient: float, block: int):
    """(N_param, N_storing) from the page's bit-cost formulas."""
    return 2 * r_salient + 1 * (1 - r_salient), 1 + 1 / block
