"""OneBit linear layer: +-1 weights with two FP16 value vectors.

ORACLE — test infrastructure only (see the package docstring).

Source [onebit], "OneBit 框架 / 1. 新的1bit结构" and Fig. 3: the weight matrix is
all +-1 and only the value vectors g and h stay FP16; the layer computes
y = ((x ⊙ g) · sign(W)^T) ⊙ h. The 4096 x 4096 storage count in the same section
is a 4096x4096 one-bit matrix plus two 4096-long 16-bit vectors.
Readings: g has one entry per input (length K) and h one per output (length N),
the only dimensionally consistent reading; activations stay fp16 (the pages list
activation quantisation as future work, "讨论与分析").
"""
from __future__ import annotations

import numpy as np


def onebit_forward(x16: np.ndarray, g16: np.ndarray, S: np.ndarray, h16: np.ndarray) -> np.ndarray:
    """y[m, n] = h_n * sum_k S[n, k] * (x[m, k] * g_k), in fp64.

    x*g is exact in fp64 (an 11-bit by 11-bit product). Parity: pinned by the
    explicit-matrix identity x @ (diag(g) S^T diag(h)), the S = 1, g = h = 1 row-sum
    case against math.fsum and a brute-force loop on tiny shapes."""
    t = np.asarray(x16, dtype=np.float16).astype(np.float64) * np.asarray(g16, dtype=np.float16).astype(np.float64)[None, :]
    y = t @ np.asarray(S, dtype=np.float64).T
    return y * np.asarray(h16, dtype=np.float16).astype(np.float64)[None, :]


def onebit_error_scale(x16: np.ndarray, g16: np.ndarray, h16: np.ndarray) -> np.ndarray:
    """Per-element error scale |h_n| * sum_k |x_mk g_k| [M, N].

    Reading: fp32 summation of K signed terms can cancel to a result near 0, where
    a plain relative error is ill-posed; the error of any summation order is
    bounded by a multiple of this scale, so the tolerance is stated against it."""
    t = np.abs(np.asarray(x16, dtype=np.float16).astype(np.float64) * np.asarray(g16, dtype=np.float16).astype(np.float64)[None, :])
    return t.sum(axis=1)[:, None] * np.abs(np.asarray(h16, dtype=np.float16).astype(np.float64))[None, :]


def onebit_storage_bits(N: int, K: int) -> int:
    """Bits stored by one OneBit layer: N*K sign bits plus two FP16 vectors (K and N long)."""
    return N * K + 16 * (N + K)


def onebit_param_count(N: int, K: int) -> int:
    """Parameters of one OneBit layer: N*K signs plus N + K values."""
    return N * K + N + K


def svid_rank1(W: np.ndarray):
    """SVID initialisation: W ~ sign(W) ⊙ (h g^T) with h g^T a rank-1 fit of |W|.

    Source [onebit], "2. 基于 SVID 初始化量化模型": sign and magnitude are split
    and the magnitude gets a rank-1 approximation (SVD or NMF); reordering the
    products then matches the 1-bit layer, so the rank-1 factors become the value
    vectors. Readings: the SVD's leading singular value is split evenly,
    h = sqrt(s1) |u1| (one per output row) and g = sqrt(s1) |v1| (one per input);
    both are rounded to fp16. The leading singular vectors of a nonnegative
    matrix can be chosen nonnegative, so the rank-1 SVD and rank-1 NMF coincide.
    Returns (S int8 +-1 [N, K], g fp16 [K], h fp16 [N], g64, h64 in fp64).
    Parity: pinned by exact recovery when |W| is itself rank one."""
    W = np.asarray(W, dtype=np.float64)
    S = np.where(W < 0, -1, 1).astype(np.int8)
    U, s, Vt = np.linalg.svd(np.abs(W), full_matrices=False)
    h64 = np.sqrt(s[0]) * np.abs(U[:, 0])
    g64 = np.sqrt(s[0]) * np.abs(Vt[0, :])
    return S, g64.astype(np.float16), h64.astype(np.float16), g64, h64
