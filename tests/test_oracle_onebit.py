"""Pins for the oracle's OneBit path, the residual-binarisation format and the
synthetic-input generators (CPU only)."""
import json
import math
import os

from fractions import Fraction

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


def _fraction_mean_f32(row):
    """Independent route to the group mean: a Fraction sum of every element, one division,
    then the general rational-to-fp32 rounding."""
    total = sum((Fraction(float(abs(v))) for v in row), Fraction(0))
    return oracle.f32_nearest(total / len(row))


def test_group_sums_match_per_exponent_sums():
    """The limb sums equal the per-exponent exact sum (and a Fraction sum) on groups that
    span the whole fp32 range: subnormals, the largest finite value, zeros of both signs."""
    rg = synth.rng(6, 3)
    a = (rg.standard_normal((24, 128)) * np.exp2(rg.integers(-149, 127, (24, 128)))).astype(np.float32)
    a[0] = np.float32(3.4028235e38)                        # 128 x FLT_MAX: the largest sum
    a[1, :64] = np.float32(1e-45)                          # smallest subnormal
    a[2, ::2] = -0.0
    sums = oracle.exact_group_abs_sums(a)
    for row, S in zip(a, sums):
        assert Fraction(S, 1 << 149) == oracle.exact_abs_sum(row)
        assert Fraction(S, 1 << 149) == sum((Fraction(float(abs(v))) for v in row), Fraction(0))


def test_f32_nearest_dyadic_matches_rational_rounding():
    rg = synth.rng(6, 4)
    cases = [(int(s), int(k)) for s, k in zip(rg.integers(1, 1 << 62, 300), rg.integers(0, 300, 300))]
    cases += [((1 << 24) + 1, 1), ((1 << 24) + 3, 1), ((1 << 25) - 1, 2),   # ties; carry to 2^24
              (1, 149), (1, 150), (3, 150), (1, 151), ((1 << 23) - 1, 149),  # subnormal grid
              ((1 << 24) - 1, 150), ((1 << 24) - 1, 149 + 7), (0xFFFFFF << 104, 0),  # FLT_MAX
              (0xFFFFFF8 << 100, 0)]                                         # rounds to inf
    for S, k in cases:
        got = oracle.f32_nearest_dyadic(S, k)
        want = oracle.f32_nearest(Fraction(S, 1 << k))
        assert got.view(np.uint32) == want.view(np.uint32), (S, k)


def test_group_mean_is_exact_rational_mean():
    """alpha = the fp32 value nearest the exact group mean. The constructed groups separate
    it from any fp32 summation order: tiny terms that an fp32 running sum (sequential or
    pairwise) absorbs, and exact ties broken to even."""
    rg = synth.rng(6, 5)
    groups = [(rg.standard_normal(128) * np.exp2(rg.integers(-140, 100, 128))).astype(np.float32)
              for _ in range(20)]
    g = np.full(128, np.float32(2.0 ** -25)); g[0] = 1.0
    groups.append(g)                       # mean 2^-7 + 127 * 2^-32: not 2^-7 (sequential fp32)
    t = np.ones(128, np.float32); t[5] = np.float32(1 + 2.0 ** -17)
    groups.append(t)                       # mean 1 + 2^-24, a tie: even -> 1.0
    t3 = np.ones(128, np.float32); t3[9] = np.float32(1 + 3 * 2.0 ** -17)
    groups.append(t3)                      # mean 1 + 3 * 2^-24, a tie: even -> 1 + 2^-22
    sub = np.zeros(128, np.float32); sub[3] = np.float32(2.0 ** -149 * 192)
    groups.append(sub)                     # mean 1.5 * 2^-149, a subnormal tie -> 2 * 2^-149
    a = np.stack(groups)
    got = oracle.group_abs_mean_f32(a)
    for row, v in zip(a, got):
        assert v.view(np.uint32) == _fraction_mean_f32(row).view(np.uint32)
    assert got[-4] == np.float32(2.0 ** -7 + 128 * 2.0 ** -32) != np.float32(2.0 ** -7)
    assert got[-3] == np.float32(1.0)
    assert got[-2] == np.float32(1 + 2.0 ** -22)
    assert got[-1] == np.float32(2 * 2.0 ** -149)
    seq = np.float32(0)
    for v in g:
        seq = np.float32(seq + v)
    assert seq / np.float32(128) == np.float32(2.0 ** -7) != got[-4]   # an fp32 sum misses it
    c = np.float32(0.1)
    assert oracle.group_abs_mean_f32(np.where(rg.random(128) < 0.5, -c, c).astype(np.float32)) == c
    bad = np.ones((3, 128), np.float32)
    bad[0, 7], bad[1, 7], bad[2, [7, 8]] = np.nan, np.inf, [np.inf, np.nan]
    m = oracle.group_abs_mean_f32(bad)
    assert np.isnan(m[0]) and m[1] == np.inf and np.isnan(m[2])


def test_onebit_error_scale_closed_forms():
    """|h_n| * sum_k |x_k g_k|: with x = +-1 alternating, g = 2 and h = -0.5 every element's
    scale is K although the signed sum (and y for S = 1) is 0; a dropped |.| on the sum or
    on h would give 0 or -K. The scale bounds |y| for any S."""
    K, N = 256, 64
    x = np.where(np.arange(K) % 2 == 0, 1.0, -1.0).astype(np.float16)[None, :]
    g = np.full(K, 2.0, np.float16)
    h = np.full(N, -0.5, np.float16)
    sc = oracle.onebit_error_scale(x, g, h)
    assert sc.shape == (1, N) and np.all(sc == K)
    assert np.all(oracle.onebit_forward(x, g, np.ones((N, K), np.int8), h) == 0)
    xs = synth.normal_fp16((3, K), 6, 7)
    gs = synth.uniform_fp16((K,), 0.5, 1.5, 6, 8)
    hs = -synth.uniform_fp16((N,), 0.5, 1.5, 6, 9)
    S = np.where(synth.rng(6, 10).random((N, K)) < 0.5, -1, 1).astype(np.int8)
    sc = oracle.onebit_error_scale(xs, gs, hs)
    want = np.abs(xs.astype(np.float64) * gs.astype(np.float64)).sum(1)[:, None] * np.abs(hs.astype(np.float64))[None, :]
    assert np.allclose(sc, want, rtol=1e-15, atol=0)
    assert np.all(np.abs(oracle.onebit_forward(xs, gs, S, hs)) <= sc * (1 + 1e-12))
    assert np.all(np.abs(oracle.onebit_forward(xs, gs, np.ones((N, K), np.int8), -hs)) <= sc * (1 + 1e-12))


def test_residual_error_scale_closed_forms():
    """sum_b (|alpha_o| + |alpha_r|)[n, b] * sum_{k in b} |x_mk|: constant scales 1 give
    2 * sum |x| (a signed sum would cancel for alternating x); one nonzero group gives
    |alpha| times that group's sum |x|; negative scales count by magnitude."""
    K, N = 512, 64
    x = np.where(np.arange(K) % 2 == 0, 1.5, -1.5).astype(np.float16)[None, :]
    ones = np.ones((N, K // 128), np.float32)
    assert np.all(oracle.residual_error_scale(x, ones, ones) == 2 * 1.5 * K)
    ao = np.zeros((N, K // 128), np.float32)
    ar = np.zeros_like(ao)
    ao[3, 2], ar[5, 1] = -0.25, 4.0
    xs = synth.normal_fp16((2, K), 6, 11)
    sc = oracle.residual_error_scale(xs, ao, ar)
    gsum = np.abs(xs.astype(np.float64)).reshape(2, K // 128, 128).sum(2)
    assert np.allclose(sc[:, 3], 0.25 * gsum[:, 2], rtol=1e-15, atol=0)
    assert np.allclose(sc[:, 5], 4.0 * gsum[:, 1], rtol=1e-15, atol=0)
    assert np.all(np.delete(sc, [3, 5], axis=1) == 0)
    Bo = np.where(synth.rng(6, 12).random((N, K)) < 0.5, -1, 1).astype(np.int8)
    Br = np.where(synth.rng(6, 13).random((N, K)) < 0.5, -1, 1).astype(np.int8)
    a1 = synth.uniform_fp16((N, K // 128), 0.5, 1.5, 6, 14).astype(np.float32)
    a2 = synth.uniform_fp16((N, K // 128), 0.0, 0.5, 6, 15).astype(np.float32)
    assert np.all(np.abs(oracle.residual_forward(xs, Bo, a1, Br, a2)) <=
                  oracle.residual_error_scale(xs, a1, a2) * (1 + 1e-12))


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
