"""Pins for the oracle's OneBit path, the residual-binarisation format and the
synthetic-input generators (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_onebit_storage_count_golden():
    """The page's count for a 4096x4096 layer: sign bits plus two FP16 vectors."""
    g = json.load(open(os.path.join(GOLDEN, "onebit_storage_4096.json")))
    N, K = g["N"], g["K"]
    bits = 8 * oracle.sign_packed_bytes(N, K) + 16 * (N + K)
    assert bits == g["total_bits"] == oracle.onebit_storage_bits(N, K)
    assert oracle.onebit_param_count(N, K) == g["total_params"]
    assert round(bits / g["total_params"], g["printed_digits"]) == g["bits_per_param_printed"]


@pytest.mark.slow
def test_onebit_storage_count_from_packer():
    g = json.load(open(os.path.join(GOLDEN, "onebit_storage_4096.json")))
    W = synth.normal_fp32((g["N"], g["K"]), 0, 2, 0, 0)
    packed = oracle.pack_sign(W)
    assert 8 * packed.size + 16 * (g["N"] + g["K"]) == g["total_bits"]


def _inputs(M, N, K, seed=0):
    x = synth.normal_fp16((M, K), seed, 2, 1)
    g = synth.uniform_fp16((K,), 0.5, 1.5, seed, 2, 2)
    h = synth.uniform_fp16((N,), 0.5, 1.5, seed, 2, 3)
    W = synth.normal_fp32((N, K), seed, 2, 4)
    return x, g, h, W


def test_onebit_explicit_matrix_identity():
    """y = ((x*g) S^T) * h equals x @ (diag(g) S^T diag(h)) formed as an explicit
    fp64 matrix (the operation reordering that lets SVID feed the layer)."""
    M, N, K = 5, 192, 256
    x, g, h, W = _inputs(M, N, K)
    S = np.where(W < 0, -1, 1).astype(np.int8)
    y = oracle.onebit_forward(x, g, S, h)
    D = np.diag(g.astype(np.float64)) @ S.astype(np.float64).T @ np.diag(h.astype(np.float64))
    ref = x.astype(np.float64) @ D
    scale = oracle.onebit_error_scale(x, g, h)
    assert np.all(np.abs(y - ref) <= 1e-12 * scale)


def test_onebit_row_sums_and_brute_force():
    M, N, K = 3, 64, 128
    x, g, h, W = _inputs(M, N, K, seed=1)
    ones = np.ones((N, K), np.int8)
    y = oracle.onebit_forward(x, np.ones(K, np.float16), ones, np.ones(N, np.float16))
    for m in range(M):
        assert np.all(y[m] == math.fsum(float(v) for v in x[m]))
    S = np.where(W < 0, -1, 1).astype(np.int8)
    y = oracle.onebit_forward(x, g, S, h)
    for m in range(M):
        for n in range(0, N, 7):
            terms = [int(S[n, k]) * float(x[m, k]) * float(g[k]) for k in range(K)]
            ref = math.fsum(terms) * float(h[n])
            assert abs(y[m, n] - ref) <= 1e-13 * math.fsum(abs(t) for t in terms) * float(h[n])


def test_onebit_g_is_per_input_h_is_per_output():
    """Non-square shape: scaling g[k0] only changes the k0 term; scaling h[n0] only row n0."""
    M, N, K = 2, 64, 256
    x, g, h, W = _inputs(M, N, K, seed=2)
    S = np.where(W < 0, -1, 1).astype(np.int8)
    y = oracle.onebit_forward(x, g, S, h)
    h2 = h.copy()
    h2[9] = np.float16(2) * h2[9]
    y2 = oracle.onebit_forward(x, g, S, h2)
    assert np.array_equal(np.delete(y2, 9, axis=1), np.delete(y, 9, axis=1))
    assert np.allclose(y2[:, 9], 2 * y[:, 9], rtol=1e-15)


def test_sign_flip_is_a_bit_assignment():
    """(-1)*t equals t with its IEEE sign bit flipped, for fp32 t (the multiply-free step)."""
    t = synth.normal_fp32(4096, 0, 2, 9) * np.float32(1e3)
    t[:4] = [0.0, -0.0, np.float32(1e-45), np.inf]
    flipped = (t.view(np.uint32) ^ np.uint32(0x80000000)).view(np.float32)
    assert np.array_equal((np.float32(-1) * t).view(np.uint32), flipped.view(np.uint32))


def test_svid_exact_for_rank_one_magnitude():
    rg = synth.rng(5, 1)
    a = rg.uniform(0.5, 2.0, 128)
    b = rg.uniform(0.5, 2.0, 256)
    S0 = np.where(rg.random((128, 256)) < 0.5, -1, 1)
    W = S0 * np.outer(a, b)
    S, g16, h16, g, h = oracle.svid_rank1(W)
    assert np.array_equal(S, S0)
    assert np.allclose(np.outer(h, g), np.outer(a, b), rtol=1e-12, atol=0)
    x = synth.normal_fp16((4, 256), 5, 2)
    y = oracle.onebit_forward(x, g16, S, h16)
    Wd = S * np.outer(h16.astype(np.float64), g16.astype(np.float64))
    assert np.allclose(y, x.astype(np.float64) @ Wd.T, rtol=0, atol=1e-10)


def test_svid_beats_sign_only():
    W = synth.normal_fp32((128, 256), 5, 3)
    S, g16, h16, g, h = oracle.svid_rank1(W)
    err_svid = np.linalg.norm(W - S * np.outer(h, g))
    err_sign = min(np.linalg.norm(W - c * S) for c in [np.abs(W).mean()])
    assert err_svid <= err_sign * (1 + 1e-12)


# ----------------------------------------------------------------------------- residual binarisation
def test_billm_storage_golden():
    g = json.load(open(os.path.join(GOLDEN, "billm_storage.json")))
    n_param, n_store = oracle.billm_storage_bits_per_param(g["r_salient"], g["block"])
    assert round(n_param, g["printed_decimals"]) == g["n_param_printed"]
    assert round(n_store, g["printed_decimals"]) == g["n_storing_printed"]


def test_pairwise_sum_within_its_error_bound():
    """The fp32 pairwise tree is within log2(n) * 2^-24 * sum|a| of the exact sum, and
    equals it when every partial sum is exact (small integers)."""
    from fractions import Fraction
    rg = synth.rng(6, 3)
    a = (rg.standard_normal((40, 128)) * np.exp2(rg.integers(-20, 20, (40, 128)))).astype(np.float32)
    got = oracle.pairwise_sum_f32(a)
    for row, s in zip(a, got):
        exact = sum((Fraction(float(v)) for v in row), Fraction(0))
        bound = 7 * 2.0 ** -24 * float(sum(abs(float(v)) for v in row))
        assert abs(float(Fraction(float(s)) - exact)) <= bound
    ints = rg.integers(-1000, 1000, (5, 128)).astype(np.float32)
    assert np.array_equal(oracle.pairwise_sum_f32(ints), ints.astype(np.int64).sum(1).astype(np.float32))


def test_residual_never_worse_than_direct():
    W = synth.normal_fp32((64, 512), 6, 1)
    Bo, ao, Br, ar = oracle.residual_binarize(W)
    direct = np.repeat(ao.astype(np.float64), 128, axis=1) * Bo
    both = direct + np.repeat(ar.astype(np.float64), 128, axis=1) * Br
    for n in range(64):
        for blk in range(4):
            sl = slice(128 * blk, 128 * blk + 128)
            e_both = np.sum((W[n, sl] - both[n, sl]) ** 2)
            e_dir = np.sum((W[n, sl] - direct[n, sl]) ** 2)
            assert e_both <= e_dir * (1 + 1e-6)
    Wc = np.where(synth.rng(6, 2).random((64, 256)) < 0.5, -0.375, 0.375).astype(np.float32)
    Bo, ao, Br, ar = oracle.residual_binarize(Wc)
    assert np.all(ao == np.float32(0.375)) and np.all(ar == 0)
    assert np.array_equal(Bo, np.sign(Wc).astype(np.int8))


def test_residual_forward_matches_explicit_matrix():
    W = synth.normal_fp32((64, 256), 6, 4)
    x = synth.normal_fp16((3, 256), 6, 5)
    Bo, ao, Br, ar = oracle.residual_binarize(W)
    y = oracle.residual_forward(x, Bo, ao, Br, ar)
    Wd = np.zeros((64, 256))
    for n in range(64):
        for k in range(256):
            Wd[n, k] = float(ao[n, k // 128]) * Bo[n, k] + float(ar[n, k // 128]) * Br[n, k]
    assert np.allclose(y, x.astype(np.float64) @ Wd.T, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- synthetic inputs
def test_splitmix64_published_vectors():
    """SplitMix64 seeded with 0: the first three outputs of the reference generator."""
    out = synth.splitmix64(0, np.arange(1, 4, dtype=np.uint64))
    assert [int(v) for v in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_ternary_codes_distribution_and_rows():
    key = synth.matrix_key(0, 3, 0, 0)
    c = synth.ternary_codes(key, 256, 1024)
    for v in (-1, 0, 1):
        assert abs(np.count_nonzero(c == v) / c.size - 1 / 3) < 0.005
    assert np.array_equal(synth.ternary_codes(key, 256, 1024, rows=[7, 200]), c[[7, 200]])
