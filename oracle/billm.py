"""Residual binarisation as an inference format (BiLLM's salient-weight scheme).

ORACLE — test infrastructure only (see the package docstring).

Source [billm], "方法细节", step 2 (binary residual approximation): binarise W
once (alpha_o * B_o), binarise the residual again (alpha_r * B_r) and use the
sum; the page states the residual scheme's error never exceeds direct
binarisation's. "存储位开销分析" gives the bit cost of a salient fraction r:
N_param = 2r + 1*(1 - r) bits per weight (two sign planes on salient weights,
one elsewhere) and N_storing = 1 + 1/b_size for the group flags.
Readings: B = sign(.) with sign(0) = +1; alpha is the mean magnitude over each
(output row, block of `block` inputs) group, the least-squares scale for a sign
approximation; the Hessian-based column search, breakpoint split and error
compensation need calibration data and are not part of this format.
"""
from __future__ import annotations

import numpy as np


def _sign(a):
    return np.where(a < 0, -1.0, 1.0)


def residual_binarize(W: np.ndarray, block: int = 128):
    """W [N, K] -> (B_o, alpha_o [N, K/block], B_r, alpha_r) in fp64."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    assert K % block == 0
    Wb = W.reshape(N, K // block, block)
    Bo = _sign(Wb)
    ao = np.abs(Wb).mean(axis=2)
    R = Wb - ao[:, :, None] * Bo
    Br = _sign(R)
    ar = np.abs(R).mean(axis=2)
    return Bo.reshape(N, K), ao, Br.reshape(N, K), ar


def residual_forward(x: np.ndarray, Bo, ao, Br, ar, block: int = 128) -> np.ndarray:
    """y = x @ (alpha_o ⊙ B_o + alpha_r ⊙ B_r)^T in fp64."""
    W = np.repeat(ao, block, axis=1) * Bo + np.repeat(ar, block, axis=1) * Br
    return np.asarray(x, dtype=np.float64) @ W.T


def billm_storage_bits_per_param(r_salient: float, block: int):
    """(N_param, N_storing) from the page's bit-cost formulas."""
    return 2 * r_salient + 1 * (1 - r_salient), 1 + 1 / block
