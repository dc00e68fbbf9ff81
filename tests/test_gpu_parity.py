"""GPU parity: every libbitlinear entry point against the CPU oracle on the same seeded
inputs. Integer results (packed bytes, codes, beta bits, int8 activations, bit planes,
int32 accumulators, residual-binarisation signs and scales) must match exactly; fp32
outputs within 1e-3 of the fp64 oracle (relative per element for b1.58; against
|h| * sum|x g| for OneBit; against sum_b (|alpha_o| + |alpha_r|) sum_{k in b} |x| for the
residual format)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import synth.gpu as sgpu
import ternary_weight_linear_amd as tw
from tests.gpu_util import (DEV, assert_rel, assert_scaled, dev, finite_fp16, gamma_ladder,
                            host, say)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- packing
@pytest.mark.parametrize("N,K", [(64, 64), (192, 320), (512, 512), (1024, 3200)])
def test_pack_unpack_ternary(N, K):
    say("pack_ternary", N, K)
    codes = synth.ternary_codes(synth.matrix_key(0, 90, N, K), N, K)
    codes[0, :5] = [1, -1, 0, 1, -1]
    ref = oracle.pack_ternary(codes)
    g = tw.bl_pack_ternary(dev(codes))
    assert np.array_equal(host(g), ref)
    back = tw.bl_unpack_ternary(g, N, K)
    assert np.array_equal(host(back), codes)


def test_pack_ternary_invalid_codes():
    say("pack_ternary invalid")
    codes = np.zeros((64, 128), np.int8)
    codes[3, 7] = 5
    codes[9, 100] = -2
    codes[10, 0] = 1
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    g = tw.bl_pack_ternary(dev(codes), n_invalid=cnt)
    ref, bad = oracle.pack_ternary(codes, count_invalid=True)
    assert np.array_equal(host(g), ref) and int(host(cnt)[0]) == bad == 2
    gb = g.clone()
    gb[0] |= 1
    gb[8] |= 1                                           # (P, N) = (1, 1) at (0, 0)
    cnt.zero_()
    back = tw.bl_unpack_ternary(gb, 64, 128, n_invalid=cnt)
    ref_codes, ref_bad = oracle.unpack_ternary(host(gb), 64, 128, count_invalid=True)
    assert np.array_equal(host(back), ref_codes) and int(host(cnt)[0]) == ref_bad == 1


@pytest.mark.parametrize("N,K", [(64, 128), (192, 256), (512, 512), (4096, 4096)])
def test_pack_unpack_sign(N, K):
    say("pack_sign", N, K)
    W = synth.normal_fp32((N, K), 0, 91, N, K)
    W[0, :4] = [0.0, -0.0, np.nan, -np.inf]
    ref = oracle.pack_sign(W)
    g = tw.bl_pack_sign(dev(W))
    assert np.array_equal(host(g), ref)
    assert np.array_equal(host(tw.bl_unpack_sign(g, N, K)), oracle.unpack_sign(ref, N, K))
    if (N, K) == (4096, 4096):
        # the storage count of the OneBit page, from the bytes the GPU packer produced
        assert 8 * g.numel() + 16 * (N + K) == 16908288


# ----------------------------------------------------------------------------- absmean
def _ternarize_case(W):
    packed, beta, codes = tw.bl_ternarize_absmean(dev(W), want_codes=True)
    rc, rb = oracle.ternarize_absmean(W)
    gb = host(beta)
    if np.isnan(rb):
        assert np.isnan(gb[0])
    else:
        assert gb.view(np.uint32)[0] == np.float32(rb).view(np.uint32)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(packed), oracle.pack_ternary(rc))


@pytest.mark.parametrize("N,K,std", [(512, 512, 0.02), (192, 320, 1.0), (3200, 3200, 0.02)])
def test_ternarize_absmean(N, K, std):
    say("ternarize_absmean", N, K, std)
    W = synth.normal_fp32((N, K), 0, 1, N, K, std=std)
    _ternarize_case(W)


def test_ternarize_absmean_edge_cases():
    say("ternarize_absmean edge")
    _ternarize_case(np.zeros((64, 64), np.float32))
    W = synth.normal_fp32((64, 128), 0, 92, 1)
    W[5, 5] = np.nan
    _ternarize_case(W)
    W = np.tile(np.array([0.5, 1.5, 1.0, 1.0], np.float32), (64, 16))      # exact tie at 0.5
    _ternarize_case(W)
    rg = synth.rng(0, 93)
    W = (rg.standard_normal((128, 192)) * np.exp2(rg.integers(-149, 30, (128, 192)))).astype(np.float32)
    _ternarize_case(W)                                                       # wide exponents, subnormals


# ----------------------------------------------------------------------------- quantiser
def _quant_case(x):
    """Both kernels: with bit planes (LDS row, lane order of the planes) and without (the
    row kept in registers); q, gamma and row sums identical to the oracle either way."""
    M, K = x.shape
    rq, rg, rr = oracle.quant_act_int8(x)
    for want_planes in (True, False):
        q, gamma, rowsum, planes = tw.bl_quant_act_int8(dev(x), want_planes=want_planes)
        gg = host(gamma)
        assert np.array_equal(np.isnan(gg), np.isnan(rg))
        assert np.array_equal(gg[~np.isnan(rg)].view(np.uint32), rg[~np.isnan(rg)].view(np.uint32))
        assert np.array_equal(host(q), rq)
        assert np.array_equal(host(rowsum), rr)
        if want_planes:
            assert np.array_equal(host(planes).view(np.uint32).reshape(M, K // 64, 16),
                                  oracle.act_planes(rq))


# Rows of up to 64 take 1024-thread workgroups with 1, 2 or 4 loads per thread (K up to 8192,
# 16384, 32768), more rows 256-thread workgroups with 2, 4, 8 or 16 (K up to 4096, 8192, 16384,
# 32768): each build at its largest K and just past it, and the 3B-shaped prefill inputs.
@pytest.mark.parametrize("M,K", [(1, 64), (8, 512), (3, 640), (1, 8192), (4, 28672), (512, 3200),
                                 (65, 8192), (70, 28672), (64, 8256), (2, 16384), (3, 16448),
                                 (66, 4096), (66, 4160), (100, 16384), (512, 8640)])
def test_quant_act(M, K):
    say("quant_act", M, K)
    x = synth.normal_fp16((M, K), 0, 2, M, K)
    if M == 512:
        x, _ = synth.with_outlier_channels(x, 0.01, 20.0, 0, 3, K)
    _quant_case(x)


def test_quant_act_degenerate_rows():
    say("quant_act degenerate")
    x = synth.normal_fp16((5, 128), 0, 94, 0)
    x[1] = 0
    x[2, 17] = np.float16(np.inf)
    x[3, 100] = np.float16(np.nan)
    x[4, :] = np.float16(-65504)
    _quant_case(x)


def ladder_rows(K):
    """Rows [x_0 .. x_{K-2}, gamma]: for every gamma of the ladder, every finite fp16 x with
    |x| <= gamma, K - 1 per row (the last row of a gamma zero-padded), so that each row's
    maximum is its gamma. Returns fp16 [R, K]."""
    finite = finite_fp16()
    rows = []
    for gamma in gamma_ladder():
        xs = finite[np.abs(finite.astype(np.float32)) <= np.float32(gamma)]
        for i in range(0, xs.size, K - 1):
            r = np.zeros(K, np.float16)
            r[:min(K - 1, xs.size - i)] = xs[i:i + K - 1]
            r[K - 1] = gamma
            rows.append(r)
    return np.stack(rows)


def test_quant_act_exhaustive_fp16():
    """Every finite fp16 x against every gamma of the ladder (84 values: subnormal gammas,
    powers of two and their one-ulp neighbours, spread mantissas), both kernels."""
    x = ladder_rows(64)
    say("quant exhaustive", x.shape)
    _quant_case(x)


# ----------------------------------------------------------------------------- products
def _weights(N, K, seed=0):
    codes = synth.ternary_codes(synth.matrix_key(seed, 95, N, K), N, K)
    return codes, tw.bl_pack_ternary(dev(codes))


def _acts(M, K, seed=0):
    x = synth.normal_fp16((M, K), seed, 96, M, K)
    return x, tw.bl_quant_act_int8(dev(x))


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (1, 192, 320), (2, 512, 512), (3, 128, 1024),
                                   (4, 320, 192), (1, 4096, 4096), (1, 1024, 8192),
                                   (2, 4096, 11008)])
def test_gemv_acc_and_output(M, N, K):
    say("gemv", M, N, K)
    codes, packed = _weights(N, K)
    x, (q, gamma, rowsum, planes) = _acts(M, K)
    rq, rg, _ = oracle.quant_act_int8(x)
    ref_acc = oracle.acc_exact(rq, codes)
    acc = tw.bl_bitlinear_acc_i32(packed, N, K, planes=planes, path=tw.BL_PATH_GEMV)
    assert np.array_equal(host(acc), ref_acc)
    beta = np.float32(synth.BETA_DIRECT)
    y = tw.bl_bitlinear_gemv(planes, gamma, packed, dev(np.array([beta])), N, K)
    assert_rel(host(y), oracle.bitlinear_output(ref_acc, rg, beta))
    # per-output-row beta (stacked matrices) and a second run: identical bits
    betas = synth.uniform_fp16((N,), 0.01, 0.02, 0, 97, N).astype(np.float32)
    y2 = tw.bl_bitlinear_gemv(planes, gamma, packed, dev(betas), N, K)
    assert_rel(host(y2), oracle.bitlinear_output(ref_acc, rg, betas))
    y3 = tw.bl_bitlinear_gemv(planes, gamma, packed, dev(betas), N, K)
    assert np.array_equal(host(y2).view(np.uint32), host(y3).view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (5, 192, 320), (8, 512, 512), (16, 640, 1024),
                                   (33, 384, 448), (64, 1024, 8192), (100, 256, 640),
                                   (512, 3200, 3200), (512, 8640, 3200)])
def test_gemm_acc_and_output(M, N, K):
    say("gemm", M, N, K)
    codes, packed = _weights(N, K, seed=1)
    x, (q, gamma, rowsum, planes) = _acts(M, K, seed=1)
    rq, rg, _ = oracle.quant_act_int8(x)
    ref_acc = oracle.acc_exact(rq, codes)
    acc = tw.bl_bitlinear_acc_i32(packed, N, K, q=q, path=tw.BL_PATH_GEMM)
    assert np.array_equal(host(acc), ref_acc)
    beta = np.float32(synth.BETA_DIRECT)
    y = tw.bl_bitlinear_gemm(q, gamma, packed, dev(np.array([beta])), N)
    assert_rel(host(y), oracle.bitlinear_output(ref_acc, rg, beta))
    y2 = tw.bl_bitlinear_gemm(q, gamma, packed, dev(np.array([beta])), N)
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


def test_gemv_row_equals_gemm_row():
    say("gemv vs gemm rows")
    N, K = 768, 2048
    codes, packed = _weights(N, K, seed=2)
    x, (q, gamma, rowsum, planes) = _acts(4, K, seed=2)
    a1 = host(tw.bl_bitlinear_acc_i32(packed, N, K, planes=planes, path=tw.BL_PATH_GEMV))
    a2 = host(tw.bl_bitlinear_acc_i32(packed, N, K, q=q, path=tw.BL_PATH_GEMM))
    assert np.array_equal(a1, a2)


@pytest.mark.parametrize("M,N,K,path", [(1, 512, 512, 0), (2, 192, 320, 1), (8, 512, 512, 0),
                                        (3, 256, 256, 2), (512, 3200, 3200, 0), (3, 256, 640, 1),
                                        (4, 320, 1024, 1), (1, 10240, 8192, 1), (1, 8192, 28672, 0)])
def test_forward_fp16_in(M, N, K, path):
    say("forward", M, N, K, path)
    x = synth.normal_fp16((M, K), 3, 98, M, K)
    W = synth.normal_fp32((N, K), 3, 99, N, K, std=0.02)
    packed, beta, _ = tw.bl_ternarize_absmean(dev(W))
    y = tw.bl_bitlinear_forward(dev(x), packed, beta, N, path=path)
    codes, rbeta = oracle.ternarize_absmean(W)
    yref, _, _, _ = oracle.bitlinear_forward(x, codes, rbeta)
    assert_rel(host(y), yref)


def test_forward_fused_gemv_exact_integers():
    """Integer-valued x with row max 127 makes q == x; with beta = 1 the fused
    quantise+GEMV output is acc * 127/127 and must equal the exact accumulators.
    A row holding NaN must come out NaN."""
    say("fused gemv integers")
    N, K = 384, 1024
    codes, packed = _weights(N, K, seed=4)
    rg = synth.rng(4, 5)
    x = rg.integers(-127, 128, size=(3, K)).astype(np.float16)
    x[:, 0] = 127
    x[2, 5] = np.float16(np.nan)
    one = dev(np.array([1.0], np.float32))
    y = host(tw.bl_bitlinear_forward(dev(x), packed, one, N, path=tw.BL_PATH_GEMV))
    acc = oracle.acc_exact(x[:2].astype(np.int8), codes)
    assert np.array_equal(y[:2], acc.astype(np.float32))
    assert np.all(np.isnan(y[2]))


# The 7B-shaped decode linears (stacked q|k|v 12288 x 4096, stacked gate|up 22016 x 4096,
# down 4096 x 11008) and row lengths that select each of the fused kernel's row-load
# variants: 2 / 4 / 8 / 16 loads per thread (K <= 4096 / 8192 / 16384 / 28672 at M = 1,
# the longest row the entry point takes) and, at M = 2, the loop past 16384.
@pytest.mark.parametrize("M,N,K", [(1, 12288, 4096), (2, 12288, 4096), (1, 22016, 4096),
                                   (2, 22016, 4096), (1, 4096, 11008), (2, 4096, 11008),
                                   (1, 128, 16384), (2, 192, 16384), (2, 64, 16448),
                                   (1, 256, 16448), (1, 256, 28672), (2, 128, 28672)])
def test_forward_fused_gemv_shapes(M, N, K):
    """Fused quantise + add-only GEMV (the decode path of bl_bitlinear_forward): fp32 output
    against the oracle on every element, and the int32 accumulators of the add-only kernel
    bit-exact; the fused output is bitwise the unfused GEMV's (same integers, same
    epilogue)."""
    say("fused gemv shape", M, N, K)
    codes, packed = _weights(N, K, seed=6)
    x = synth.normal_fp16((M, K), 6, 100, M, K)
    beta = np.float32(synth.BETA_DIRECT)
    db = dev(np.array([beta]))
    y = tw.bl_bitlinear_forward(dev(x), packed, db, N, path=tw.BL_PATH_GEMV)
    rq, rg, _ = oracle.quant_act_int8(x)
    ref_acc = oracle.acc_exact(rq, codes)
    assert_rel(host(y), oracle.bitlinear_output(ref_acc, rg, beta))
    q, gamma, _, planes = tw.bl_quant_act_int8(dev(x))
    acc = tw.bl_bitlinear_acc_i32(packed, N, K, planes=planes, path=tw.BL_PATH_GEMV)
    assert np.array_equal(host(acc), ref_acc)
    y2 = tw.bl_bitlinear_gemv(planes, gamma, packed, db, N, K)
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


@pytest.mark.parametrize("K", [1024, 11008, 28672])
def test_forward_fused_gemv_exact_integers_long_rows(K):
    """As test_forward_fused_gemv_exact_integers, for the 8- and 16-load row variants."""
    say("fused gemv integers", K)
    N = 384
    codes, packed = _weights(N, K, seed=7)
    x = synth.rng(7, 6, K).integers(-127, 128, size=(2, K)).astype(np.float16)
    x[:, 0] = 127
    one = dev(np.array([1.0], np.float32))
    for m in (1, 2):
        y = host(tw.bl_bitlinear_forward(dev(x[:m]), packed, one, N, path=tw.BL_PATH_GEMV))
        assert np.array_equal(y, oracle.acc_exact(x[:m].astype(np.int8), codes).astype(np.float32))


def _fused_q(x, packed_eye, K):
    """Run the fused quantise + GEMV over an identity weight matrix with beta = 1, where
    y = q * fp32(gamma / 127) exactly up to one rounding, and recover q (exact: |q| <= 127)."""
    one = dev(np.array([1.0], np.float32))
    y = host(tw.bl_bitlinear_forward(dev(x), packed_eye, one, K, path=tw.BL_PATH_GEMV))
    _, rg, _ = oracle.quant_act_int8(x)
    scale = (rg / np.float32(127)).astype(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return y, np.rint(y.astype(np.float64) / scale[:, None])


@pytest.mark.parametrize("M,K", [(1, 8192), (2, 8192), (3, 2048), (4, 2048), (1, 11008),
                                 (2, 16384), (1, 28672), (2, 28672)])
def test_forward_fused_quantiser_exhaustive(M, K):
    """The fused kernel quantises x itself; every finite fp16 x against every gamma of the
    ladder (rows [x..., gamma]) must give the oracle's q to the bit, including quotients
    that are exact half-integers (ties to even) and ones within an ulp of them. K picks the
    kernel's row-load variant (2, 4, 8, 16 loads per thread, or the loop)."""
    eye = dev(np.eye(K, dtype=np.int8))
    packed = tw.bl_pack_ternary(eye)
    del eye
    rows = ladder_rows(K)
    say("fused quant exhaustive", M, K, rows.shape)
    for r0 in range(0, rows.shape[0], M):
        x = np.zeros((M, K), np.float16)
        chunk = rows[r0:r0 + M]
        x[:chunk.shape[0]] = chunk
        x[chunk.shape[0]:, K - 1] = 1.0
        rq, _, _ = oracle.quant_act_int8(x)
        _, q = _fused_q(x, packed, K)
        assert np.array_equal(q, rq.astype(np.float64)), (r0, x[:, K - 1])
    # degenerate rows: all zero, one NaN, one inf, all -65504
    x = synth.normal_fp16((M, K), 0, 94, 1)
    x[0] = 0
    if M > 1:
        x[1, 17] = np.float16(np.inf if M > 2 else np.nan)
    y, q = _fused_q(x, packed, K)
    rq, rg, _ = oracle.quant_act_int8(x)
    assert np.array_equal(y[0], np.zeros(K, np.float32))
    for m in range(1, M):
        if np.isnan(rg[m]):
            assert np.all(np.isnan(y[m]))
        else:
            assert np.array_equal(q[m], rq[m].astype(np.float64))


def test_config1_tiny_end_to_end():
    """x fp16 [8, 512] ~ N(0,1), W fp32 [512, 512] ~ N(0, 0.02^2), seed 0, both paths."""
    say("config1 tiny")
    x = synth.normal_fp16((8, 512), 0, 1, 0, 10)
    W = synth.normal_fp32((512, 512), 0, 1, 0, 11, std=0.02)
    codes, rbeta = oracle.ternarize_absmean(W)
    yref, acc_ref, rq, _ = oracle.bitlinear_forward(x, codes, rbeta)
    packed, beta, gcodes = tw.bl_ternarize_absmean(dev(W), want_codes=True)
    assert np.array_equal(host(gcodes), codes)
    q, gamma, _, planes = tw.bl_quant_act_int8(dev(x))
    assert np.array_equal(host(tw.bl_bitlinear_acc_i32(packed, 512, 512, q=q, path=2)), acc_ref)
    for path in (1, 2):
        xs = dev(x[:4]) if path == 1 else dev(x)
        yy = tw.bl_bitlinear_forward(xs, packed, beta, 512, path=path)
        assert_rel(host(yy), yref[:4] if path == 1 else yref)


# ----------------------------------------------------------------------------- OneBit
def _onebit_inputs(M, N, K, seed=0):
    x = synth.normal_fp16((M, K), seed, 2, 1, M, K)
    g = synth.uniform_fp16((K,), 0.5, 1.5, seed, 2, 2, K)
    h = synth.uniform_fp16((N,), 0.5, 1.5, seed, 2, 3, N)
    W = synth.normal_fp32((N, K), seed, 2, 4, N, K)
    return x, g, h, W


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (1, 192, 256), (2, 512, 512), (8, 512, 512),
                                   (5, 320, 384), (1, 4096, 4096), (16, 4096, 4096), (3, 448, 1024),
                                   (4, 256, 640), (33, 192, 512), (17, 1024, 8192),
                                   (1, 512, 8192), (1, 16384, 256), (2, 16384, 384),
                                   (4, 16384, 5120), (1, 2048, 12288), (8, 1024, 8192),
                                   (12, 16384, 256), (1, 16384, 4224), (3, 16384, 6144)])
def test_onebit(M, N, K):
    """Covers the three workgroup mappings: at M <= 4 one 16-column fragment per workgroup
    (few bands; (1, 512, 8192) also splits K) or one band per workgroup with x and g staged
    in LDS (N = 16384: 256 bands; (4, 16384, 5120) splits K because its range would not fit
    LDS; K = 4224 and 6144 take the build for 33..64 tiles per range), and the band kernel
    above M = 4."""
    say("onebit", M, N, K)
    x, g, h, W = _onebit_inputs(M, N, K)
    S = np.where(W < 0, -1, 1).astype(np.int8)
    sp = tw.bl_pack_sign(dev(W))
    y = tw.bl_onebit_linear(dev(x), dev(g), sp, dev(h))
    yref = oracle.onebit_forward(x, g, S, h)
    assert_scaled(host(y), yref, oracle.onebit_error_scale(x, g, h))
    # plain elementwise relative error, reported beside the componentwise bound (it is
    # ill-posed where the sum cancels to ~0, so it is not asserted)
    rel = np.abs(host(y).astype(np.float64) - yref) / np.maximum(np.abs(yref), 1e-300)
    say("onebit plain relative error", M, N, K, "max", float(rel.max()),
        "elements above 1e-3:", int((rel > 1e-3).sum()), "of", rel.size)
    y2 = tw.bl_onebit_linear(dev(x), dev(g), sp, dev(h))
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


# ----------------------------------------------------------------------------- SVID
def _fp16_ulp(a16):
    a = np.abs(a16.astype(np.float32))
    return np.spacing(a.astype(np.float16)).astype(np.float32)


@pytest.mark.parametrize("N,K,std,kind", [(512, 512, 0.02, "gauss"), (192, 640, 1.0, "gauss"),
                                          (4096, 4096, 1.0, "gauss"), (256, 384, 1.0, "rank1")])
def test_svid_rank1(N, K, std, kind):
    """Power-iteration SVID against the oracle's SVD: signs bit-exact, g and h within one
    fp16 ulp of the oracle's fp16 values, h g^T within 1e-3 of the fp64 rank-1 fit."""
    say("svid", N, K, kind)
    if kind == "rank1":
        rg = synth.rng(8, 1)
        W = (np.where(rg.random((N, K)) < 0.5, -1.0, 1.0) *
             np.outer(rg.uniform(0.5, 2.0, N), rg.uniform(0.5, 2.0, K))).astype(np.float32)
    else:
        W = synth.normal_fp32((N, K), 0, 8, N, K, std=std)
    sp, g, h, sigma = tw.bl_svid_rank1(dev(W), iters=20)
    S, g16, h16, g64, h64 = oracle.svid_rank1(W.astype(np.float64))
    assert np.array_equal(host(sp), oracle.pack_sign(W))
    gg, hh = host(g), host(h)
    assert np.all(np.abs(gg.astype(np.float32) - g16.astype(np.float32)) <= _fp16_ulp(g16))
    assert np.all(np.abs(hh.astype(np.float32) - h16.astype(np.float32)) <= _fp16_ulp(h16))
    ref = np.outer(h64, g64)
    fit = np.outer(hh.astype(np.float64), gg.astype(np.float64))
    assert np.linalg.norm(fit - ref) <= 1e-3 * np.linalg.norm(ref)
    s1 = np.linalg.svd(np.abs(W.astype(np.float64)), compute_uv=False)[0]
    assert abs(float(host(sigma)[0]) - s1) <= 1e-5 * s1


def test_svid_then_onebit_layer():
    """For a weight whose magnitudes vary by row and column (the structure SVID captures), a
    layer initialised by SVID on the GPU tracks the float layer better than a
    per-tensor-scaled sign matrix."""
    say("svid + onebit")
    N, K, M = 512, 1024, 4
    rg = synth.rng(8, 2)
    W = (synth.normal_fp32((N, K), 0, 8, 99, std=0.02) *
         np.outer(rg.uniform(0.2, 3.0, N), rg.uniform(0.2, 3.0, K))).astype(np.float32)
    x = synth.normal_fp16((M, K), 0, 8, 98)
    sp, g, h, _ = tw.bl_svid_rank1(dev(W))
    y = host(tw.bl_onebit_linear(dev(x), g, sp, h))
    yf = x.astype(np.float64) @ W.astype(np.float64).T
    S = np.where(W < 0, -1.0, 1.0)
    ys = x.astype(np.float64) @ (np.abs(W).mean() * S).T
    assert np.linalg.norm(y - yf) < np.linalg.norm(ys - yf)


# ----------------------------------------------------------------------------- residual binarisation
def _residual_weight(N, K, seed=0):
    """Gaussian weight with the special groups the format has: an all-zero group, signed
    zeros, a constant-magnitude group (residual exactly zero), subnormal magnitudes and a
    group holding inf."""
    W = synth.normal_fp32((N, K), seed, 12, N, K, std=0.02)
    W[0, :128] = 0.0
    W[1, :128] = np.where(synth.rng(seed, 12, 1).random(128) < 0.5, -0.375, 0.375)
    W[2, :6] = [0.0, -0.0, -0.0, 0.0, -0.0, -0.0]
    W[3, :128] = synth.normal_fp32(128, seed, 12, 2) * np.float32(1e-39)
    W[4, :128] = np.float32(2.0 ** -25)       # exact mean 2^-7 + 127 * 2^-32: an fp32 running
    W[4, 0] = 1.0                             # sum (any order) absorbs the small terms
    W[5, :128] = 1.0                          # mean 1 + 2^-24: a tie, to even (1.0)
    W[5, 77] = np.float32(1 + 2.0 ** -17)
    W[6, :128] = 0.0                          # mean 1.5 * 2^-149: a subnormal tie
    W[6, 100] = np.float32(2.0 ** -149 * 192)
    W[7, :128] = np.float32(3.4028235e38)     # 128 x FLT_MAX: the largest exact sum
    W[7, 1::2] *= -1
    if N > 64:
        W[64, :128] = 1.0
        W[64, 5] = np.inf
    return W


def _bits_equal(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    fin = np.isfinite(b)
    return (np.array_equal(a[fin].view(np.uint32), b[fin].view(np.uint32)) and
            np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~fin & ~np.isnan(b)],
                                                                        b[~fin & ~np.isnan(b)]))


@pytest.mark.parametrize("N,K", [(64, 128), (192, 384), (512, 1024), (4096, 4096)])
def test_residual_binarize(N, K):
    """Sign planes bit-exact; both scales bit-exact (each the fp32 value nearest the exact
    group mean, so no summation order is shared with the oracle)."""
    say("residual_binarize", N, K)
    W = _residual_weight(N, K)
    po, ao, pr, ar = tw.bl_residual_binarize(dev(W))
    Bo, ao_ref, Br, ar_ref = oracle.residual_binarize(W)
    assert np.array_equal(host(po), oracle.pack_sign(Bo.astype(np.float32)))
    assert np.array_equal(host(pr), oracle.pack_sign(Br.astype(np.float32)))
    assert _bits_equal(host(ao), ao_ref)
    assert _bits_equal(host(ar), ar_ref)
    assert ao_ref[0, 0] == 0 and ar_ref[1, 0] == 0 and 0 < ao_ref[3, 0] < np.float32(1e-38)
    assert ao_ref[4, 0] == np.float32(2.0 ** -7 + 128 * 2.0 ** -32) and ao_ref[5, 0] == 1.0
    assert ao_ref[6, 0] == np.float32(2 * 2.0 ** -149) and ao_ref[7, 0] == np.float32(3.4028235e38)


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (1, 4096, 4096), (2, 320, 384), (3, 192, 1280),
                                   (5, 448, 1024), (16, 512, 512), (17, 1024, 8192),
                                   (33, 192, 512), (64, 256, 2048), (1, 256, 4096),
                                   (2, 16384, 256), (1, 2048, 12288), (12, 1024, 8192)])
def test_residual_linear(M, N, K):
    """Forward on planes and scales packed by the oracle (independent of the GPU packer)."""
    say("residual_linear", M, N, K)
    W = synth.normal_fp32((N, K), 0, 13, N, K, std=0.02)
    x = synth.normal_fp16((M, K), 0, 13, M, K)
    Bo, ao, Br, ar = oracle.residual_binarize(W)
    po = dev(oracle.pack_sign(Bo.astype(np.float32)))
    pr = dev(oracle.pack_sign(Br.astype(np.float32)))
    y = tw.bl_residual_linear(dev(x), po, dev(ao), pr, dev(ar))
    yref = oracle.residual_forward(x, Bo, ao, Br, ar)
    assert_scaled(host(y), yref, oracle.residual_error_scale(x, ao, ar))
    y2 = tw.bl_residual_linear(dev(x), po, dev(ao), pr, dev(ar))
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


def test_residual_end_to_end_beats_one_plane():
    """GPU binarise + forward: the two-plane layer tracks the float layer more closely than
    the first plane alone (the residual's purpose), and matches the oracle."""
    say("residual end to end")
    M, N, K = 4, 512, 1024
    W = synth.normal_fp32((N, K), 0, 14, std=0.02)
    x = synth.normal_fp16((M, K), 0, 14, 1)
    po, ao, pr, ar = tw.bl_residual_binarize(dev(W))
    y = host(tw.bl_residual_linear(dev(x), po, ao, pr, ar))
    Bo, aor, Br, arr = oracle.residual_binarize(W)
    assert_scaled(y, oracle.residual_forward(x, Bo, aor, Br, arr), oracle.residual_error_scale(x, aor, arr))
    yf = x.astype(np.float64) @ W.astype(np.float64).T
    y1 = oracle.residual_forward(x, Bo, aor, Br, np.zeros_like(arr))
    assert np.linalg.norm(y - yf) < 0.75 * np.linalg.norm(y1 - yf)


# ----------------------------------------------------------------------------- workspace hygiene
def test_workspace_left_zero():
    say("workspace zero")
    N, K = 1024, 8192
    codes, packed = _weights(N, K, seed=3)
    x, (q, gamma, rowsum, planes) = _acts(1, K, seed=3)
    beta = dev(np.array([0.5], np.float32))
    tw.bl_bitlinear_gemv(planes, gamma, packed, beta, N, K)
    tw.bl_bitlinear_gemm(q, gamma, packed, beta, N)
    xo, go, ho, Wo = _onebit_inputs(1, 512, 512)
    tw.bl_onebit_linear(dev(xo), dev(go), tw.bl_pack_sign(dev(Wo)), dev(ho))
    tw.bl_residual_linear(dev(xo), *tw.bl_residual_binarize(dev(Wo)))
    torch.cuda.synchronize()
    zero_prefix = 65536 * 4 + 64 * 65536 * 8        # counters + split-K words
    for d, buf in tw._ws.items():
        assert not host(buf[:zero_prefix]).any(), "zero-maintained workspace left dirty"


# ----------------------------------------------------------------------------- whole-stack decode
# Shapes that exercise the work split: one band (N = 64), band counts not a multiple of four,
# one 64-input tile (K = 64), an odd tile count (K = 4160), few groups with long rows (more
# workgroups than group tiles, many workgroups per group), and a wide output.
STACK_SHAPES = [(64, 64), (192, 320), (512, 512), (320, 1024), (1024, 256), (64, 8192),
                (256, 4160), (4096, 1024)]


def _stack_linears(shapes, M, seed):
    """Per linear: host codes, packed weights, beta (scalar or per row), x, y buffer."""
    out = []
    for i, (N, K) in enumerate(shapes):
        codes = synth.ternary_codes(synth.matrix_key(seed, 120, i, N), N, K)
        if i % 2:
            beta = synth.uniform_fp16((N,), 0.01, 0.03, seed, 121, i).astype(np.float32)
        else:
            beta = np.array([synth.BETA_DIRECT], np.float32)
        x = synth.normal_fp16((M, K), seed, 122, i, M)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        out.append(dict(codes=codes, packed=tw.bl_pack_ternary(dev(codes)), beta=beta,
                        dbeta=dev(beta), x=x, dx=dev(x), y=y, N=N, K=K))
    return out


def _stack_oracle(l):
    yref, _, _, _ = oracle.bitlinear_forward(l["x"], l["codes"], l["beta"])
    return yref


def _run_stack(lins, M):
    plan = tw.bl_stack_prepare([(l["dx"], l["packed"], l["dbeta"], l["y"]) for l in lins], M)
    tw.bl_bitlinear_forward_stack(plan, len(lins), M)
    return plan


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_stack_matches_oracle(M):
    say("stack vs oracle", M)
    lins = _stack_linears(STACK_SHAPES, M, seed=M)
    plan = _run_stack(lins, M)
    assert tw.bl_stack_status(plan) == 0
    for l in lins:
        assert_rel(host(l["y"]), _stack_oracle(l))


@pytest.mark.parametrize("M", [1, 2])
def test_stack_equals_separate_calls(M):
    """One persistent launch gives the bits of bl_bitlinear_forward (GEMV path) per linear,
    and repeated launches give the same bits."""
    say("stack vs separate", M)
    lins = _stack_linears(STACK_SHAPES, M, seed=10 + M)
    plan = _run_stack(lins, M)
    first = [host(l["y"]).view(np.uint32).copy() for l in lins]
    for l, f in zip(lins, first):
        y = tw.bl_bitlinear_forward(l["dx"], l["packed"], l["dbeta"], l["N"], path=tw.BL_PATH_GEMV)
        assert np.array_equal(host(y).view(np.uint32), f)
    for l in lins:
        l["y"].fill_(float("nan"))
    tw.bl_bitlinear_forward_stack(plan, len(lins), M)
    for l, f in zip(lins, first):
        assert np.array_equal(host(l["y"]).view(np.uint32), f)
    assert tw.bl_stack_status(plan) == 0


@pytest.mark.parametrize("grid", [1, 3, 8, 37, 300])
def test_stack_small_grids(grid, monkeypatch):
    """Capped grids: workgroups whose share spans several groups and several 64-tile chunks
    (512 x 32768 at 8 workgroups: 128 tiles per share), linears a workgroup has no part of."""
    say("stack grid", grid)
    monkeypatch.setenv("BL_STACK_GRID", str(grid))
    lins = _stack_linears([(512, 32768), (192, 320), (64, 64), (1024, 2048)], 1, seed=20 + grid)
    plan = _run_stack(lins, 1)
    assert tw.bl_stack_status(plan) == 0
    for l in lins:
        assert_rel(host(l["y"]), _stack_oracle(l))


@pytest.mark.parametrize("M", [1, 3])
def test_stack_quantiser_exhaustive(M):
    """The persistent launch quantises every linear's x itself: one linear per M rows of
    the gamma-ladder sweep (every finite fp16 x against every gamma, identity weights,
    beta = 1), q recovered from y and compared with the oracle's to the bit."""
    K = 2048
    packed = tw.bl_pack_ternary(dev(np.eye(K, dtype=np.int8)))
    one = dev(np.array([1.0], np.float32))
    rows = ladder_rows(K)
    xs, lins = [], []
    for r0 in range(0, rows.shape[0], M):
        x = np.zeros((M, K), np.float16)
        chunk = rows[r0:r0 + M]
        x[:chunk.shape[0]] = chunk
        x[chunk.shape[0]:, K - 1] = 1.0
        y = torch.full((M, K), float("nan"), dtype=torch.float32, device=DEV)
        xs.append(x)
        lins.append((dev(x), packed, one, y))
    say("stack quant exhaustive", M, len(lins))
    plan = tw.bl_stack_prepare(lins, M)
    tw.bl_bitlinear_forward_stack(plan, len(lins), M)
    assert tw.bl_stack_status(plan) == 0
    for i, (x, (_, _, _, y)) in enumerate(zip(xs, lins)):
        rq, rg, _ = oracle.quant_act_int8(x)
        scale = (rg / np.float32(127)).astype(np.float32).astype(np.float64)
        q = np.rint(host(y).astype(np.float64) / scale[:, None])
        assert np.array_equal(q, rq.astype(np.float64)), (i, x[:, K - 1])


def test_stack_read_after_write_and_write_after_read():
    """Linear 1 reads, as its fp16 x, the bytes linear 0 writes as fp32 y; linear 2 writes
    its y over linear 0's x. The stack must give the bits of three calls in order."""
    say("stack hazards")
    N0, K0, N1, N2, K2 = 256, 512, 128, 256, 256
    c0 = synth.ternary_codes(synth.matrix_key(0, 123, 0, 0), N0, K0)
    c1 = synth.ternary_codes(synth.matrix_key(0, 123, 1, 0), N1, 2 * N0)
    c2 = synth.ternary_codes(synth.matrix_key(0, 123, 2, 0), N2, K2)
    p0, p1, p2 = (tw.bl_pack_ternary(dev(c)) for c in (c0, c1, c2))
    # x0: a few entries of +-127, so gamma = 127, q = x0 and y0 = acc (beta = 1) are small
    # integers whose fp32 bit patterns read as finite fp16 pairs
    x0 = np.zeros((1, K0), np.float16)
    x0[0, [3, 100, 257, 511]] = [127, -127, 127, 127]
    one = dev(np.array([1.0], np.float32))
    b1 = dev(synth.uniform_fp16((N1,), 0.01, 0.03, 0, 124, 1).astype(np.float32))
    b2 = dev(np.array([0.25], np.float32))
    x2 = synth.normal_fp16((1, K2), 0, 125, 2)

    def buffers():
        buf0 = torch.full((1, N0), float("nan"), dtype=torch.float32, device=DEV)  # y0 = x1
        xb0 = dev(x0)                                                                # x0 = y2
        y1 = torch.full((1, N1), float("nan"), dtype=torch.float32, device=DEV)
        return buf0, xb0, y1

    # separate calls in order
    r0, rx0, ry1 = buffers()
    r0.copy_(tw.bl_bitlinear_forward(rx0, p0, one, N0, path=tw.BL_PATH_GEMV))
    ry1.copy_(tw.bl_bitlinear_forward(r0.view(torch.float16), p1, b1, N1, path=tw.BL_PATH_GEMV))
    rx0.view(torch.float32).copy_(tw.bl_bitlinear_forward(dev(x2), p2, b2, N2, path=tw.BL_PATH_GEMV))
    # one stack
    s0, sx0, sy1 = buffers()
    dx2 = dev(x2)
    plan = tw.bl_stack_prepare([(sx0, p0, one, s0), (s0.view(torch.float16), p1, b1, sy1),
                                (dx2, p2, b2, sx0.view(torch.float32))], 1)
    tw.bl_bitlinear_forward_stack(plan, 3, 1)
    assert tw.bl_stack_status(plan) == 0
    for a, b in ((r0, s0), (ry1, sy1), (rx0, sx0)):
        assert np.array_equal(host(a).view(np.uint16), host(b).view(np.uint16))
    # and against the oracle: y0 is exact, x1 is the fp16 reading of y0's bytes
    acc0 = oracle.acc_exact(x0.astype(np.int8), c0)
    assert np.array_equal(host(s0), acc0.astype(np.float32))
    x1 = host(s0).view(np.float16)
    assert np.isfinite(x1).all()
    y1ref, _, _, _ = oracle.bitlinear_forward(x1, c1, host(b1))
    assert_rel(host(sy1), y1ref)
    y2ref, _, _, _ = oracle.bitlinear_forward(x2, c2, np.float32(0.25))
    assert_rel(host(sx0).view(np.float32), y2ref)


def test_stack_plan_mismatch_sets_status():
    """A launch whose count or M differs from the plan's computes nothing and sets status 1;
    preparing the plan again clears it."""
    say("stack mismatch")
    lins = _stack_linears([(128, 256), (64, 128)], 1, seed=30)
    descs = [(l["dx"], l["packed"], l["dbeta"], l["y"]) for l in lins]
    plan = tw.bl_stack_prepare(descs, 1)
    tw.bl_bitlinear_forward_stack(plan, 3, 1)
    assert tw.bl_stack_status(plan) == 1
    assert all(torch.isnan(l["y"]).all() for l in lins)
    plan2 = tw.bl_stack_prepare(descs, 1)
    tw.bl_bitlinear_forward_stack(plan2, 2, 2)
    assert tw.bl_stack_status(plan2) == 1
    plan3 = tw.bl_stack_prepare(descs, 1)
    tw.bl_bitlinear_forward_stack(plan3, 2, 1)
    assert tw.bl_stack_status(plan3) == 0
    for l in lins:
        assert_rel(host(l["y"]), _stack_oracle(l))


def test_stack_leaves_workspace_zero():
    say("stack workspace zero")
    lins = _stack_linears(STACK_SHAPES[:5], 2, seed=31)
    _run_stack(lins, 2)
    torch.cuda.synchronize()
    zero_prefix = 65536 * 4 + 64 * 65536 * 8        # counters (incl. the arrival counter) + split words
    for d, buf in tw._ws.items():
        assert not host(buf[:zero_prefix]).any(), "zero-maintained workspace left dirty"


# ----------------------------------------------------------------------------- T2-MF64
@pytest.mark.parametrize("N,K", [(64, 64), (192, 320), (1024, 3200)])
def test_pack_and_repack_ternary_mf(N, K):
    say("pack mf", N, K)
    codes = synth.ternary_codes(synth.matrix_key(0, 130, N, K), N, K)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    mf = tw.bl_pack_ternary_mf(dev(codes), n_invalid=bad)
    assert np.array_equal(host(mf), oracle.pack_ternary_mf(codes)) and int(host(bad)[0]) == 0
    mf2 = tw.bl_repack_ternary_mf(tw.bl_pack_ternary(dev(codes)), N, K, n_invalid=bad)
    assert np.array_equal(host(mf2), oracle.pack_ternary_mf(codes)) and int(host(bad)[0]) == 0


def test_mf_invalid_codes():
    say("mf invalid")
    codes = np.zeros((64, 64), dtype=np.int8)
    codes[0, :3] = [2, -5, -1]
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    mf = tw.bl_pack_ternary_mf(dev(codes), n_invalid=bad)
    assert int(host(bad)[0]) == 2
    assert np.array_equal(host(mf), oracle.pack_ternary_mf(codes))
    pn = oracle.pack_ternary(np.zeros((64, 64), dtype=np.int8))
    pn[0] |= 0x01                                   # P and N both set at (0, 0)
    pn[8] |= 0x01
    bad.zero_()
    mf2 = tw.bl_repack_ternary_mf(dev(pn), 64, 64, n_invalid=bad)
    assert int(host(bad)[0]) == 1
    assert np.array_equal(host(mf2), oracle.pack_ternary_mf(np.zeros((64, 64), dtype=np.int8)))


# Up to eight rows over fewer than 512 bands take the four-band kernel with q of a K range
# in LDS: no split (1 x 64 x 64, 1 x 128 x 256, 5 x 192 x 320), split words per output (more
# than eight splits: 4 x 256 x 16384, 64 of them) or per pair of rows (7 x 10240 x 8192 and
# 3 x 8192 x 28672: odd M, the last pair half unused; 8 x 512 x 512, 8 x 8192 x 28672), a
# ragged last group of 511 bands. Otherwise
# the staged-q kernel where four-band groups x row tiles >= 160 (N = 49152, 10240 at
# M = 200) or at most eight K splits meet in split words per pair of rows (64 x 1024 x 8192:
# eight splits; 33 x 4096 x 8192: four, odd M; 64 x 8192 x 28672: the 70B down projection),
# the per-band kernel for more splits (2 x 128 x 39936); 49216 leaves a last group with one
# band; M = 40, 70, 200 ragged
# row tiles; M >= 256 over >= 32 band groups the 48-row tiles (300 = 6 x 48 + 12), with a
# K split past 32768 inputs (256 x 8192 x 33792).
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (1, 128, 256), (5, 192, 320), (8, 512, 512),
                                   (4, 256, 16384), (7, 10240, 8192), (3, 8192, 28672), (8, 32704, 4096),
                                   (33, 4096, 8192), (64, 8192, 28672), (16, 640, 1024),
                                   (17, 384, 448), (33, 256, 640), (64, 1024, 8192),
                                   (100, 256, 640), (2, 128, 39936), (8, 8192, 28672),
                                   (1, 49216, 64), (8, 49152, 256), (40, 49152, 192),
                                   (64, 49152, 320), (70, 49152, 128), (16, 49152, 1024),
                                   (200, 10240, 128), (96, 2560, 256), (300, 8192, 1088),
                                   (256, 8192, 33792)])
def test_gemm_mf_acc_and_output(M, N, K):
    say("gemm mf", M, N, K)
    codes = synth.ternary_codes(synth.matrix_key(0, 131, N, K), N, K)
    if K <= 28672:
        x = synth.normal_fp16((M, K), 0, 132, M, K)
        q, gamma, rowsum, _ = tw.bl_quant_act_int8(dev(x), want_planes=False)
        rq, rg, rrow = oracle.quant_act_int8(x)
        assert np.array_equal(host(rowsum), rrow)
    else:
        # rows longer than the quantiser takes: int8 activations drawn directly (the
        # extremes included), with gamma = 127 and their row sums as the kernel's inputs
        rq = synth.rng(0, 135, M, K).integers(-127, 128, size=(M, K)).astype(np.int8)
        rq[:, :2] = [127, -127]
        rg = np.full(M, 127.0, dtype=np.float32)
        q, gamma = dev(rq), dev(rg)
        rowsum = dev(rq.astype(np.int64).sum(axis=1).astype(np.int32))
    wmf = tw.bl_pack_ternary_mf(dev(codes))
    beta = np.float32(synth.BETA_DIRECT)
    y, acc = tw.bl_bitlinear_gemm_mf(q, gamma, rowsum, wmf, dev(np.array([beta])), N, want_acc=True)
    ref_acc = oracle.acc_exact(rq, codes)
    assert np.array_equal(host(acc), ref_acc)
    assert_rel(host(y), oracle.bitlinear_output(ref_acc, rg, beta))
    y2, _ = tw.bl_bitlinear_gemm_mf(q, gamma, rowsum, wmf, dev(np.array([beta])), N)
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


# Decode through T2-MF64. The fused kernel takes M <= 4, and M <= 16 where K <= 8192 and
# the output has < 512 bands; the other shapes go through quantiser + product (the four-band
# q-in-LDS kernel up to eight rows over < 512 bands: 6 x 8192 x 28672; the staged-q or
# per-band kernels beyond: 12 x 8192 x 28672). Fused: M = 4 over the 70B down shape (eight
# splits, split words per pair of rows), M = 8 over q|k|v. Fused
# shapes: one tile; ragged band groups (inactive waves) with long rows (row loads past 8192
# inputs); the largest K; long K ranges per workgroup (K split in two over wide outputs);
# no K split (>= 512 band groups at M = 1; a 4-tile K at M = 16); ranges past the LDS
# capacity of 16 rows (more splits); every row-tile width 1, 2, 4, 8, 16 with unused rows.
# Routed elsewhere: long or wide shapes at M > 4, and M x N past the split words' capacity.
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (1, 320, 8256), (2, 128, 28672),
                                   (1, 65536, 16384), (1, 131072, 256), (16, 2048, 256),
                                   (16, 32704, 8192), (8, 32704, 8192), (5, 448, 4160),
                                   (13, 192, 2048), (4, 10240, 8192), (3, 65536, 16384),
                                   (8, 65536, 8192), (16, 262208, 4096), (4, 8192, 28672),
                                   (8, 10240, 8192), (6, 8192, 28672), (12, 8192, 28672)])
def test_forward_mf_decode_equals_forward(M, N, K):
    """The fused decode kernel gives the outputs of the unfused T2-PN-64 path to the bit and
    matches the oracle on sampled rows."""
    say("forward mf decode", M, N, K)
    _mf_vs_pn_sampled(M, N, K)


# Prefill-sized M through T2-MF64: 48-row tiles of the staged-q kernel over >= 32 band
# groups (ragged: 300 = 6 x 48 + 12; exactly 32 groups with a 17-tile K, an odd number of
# two-chunk ring turns), the 3B q|k|v and gate|up shapes at M = 512.
@pytest.mark.parametrize("M,N,K", [(300, 16384, 320), (300, 8192, 1088), (512, 9600, 3200),
                                   (512, 17280, 3200)])
def test_forward_mf_prefill_equals_forward(M, N, K):
    say("forward mf prefill", M, N, K)
    _mf_vs_pn_sampled(M, N, K)


def _mf_vs_pn_sampled(M, N, K):
    """T2-MF64 forward bitwise equal to the T2-PN-64 forward on the same GPU-drawn codes, and
    97 sampled output columns against the oracle from codes regenerated on the host."""
    x = synth.normal_fp16((M, K), 0, 135, M, K)
    key = synth.matrix_key(0, 136, N, K)
    codes_d = sgpu.ternary_codes(key, N, K, DEV)     # the GPU twin of synth.ternary_codes
    beta = np.float32(0.0173)
    packed = tw.bl_pack_ternary(codes_d)
    wmf = tw.bl_pack_ternary_mf(codes_d)
    del codes_d
    b = dev(np.array([beta], np.float32))
    y_pn = tw.bl_bitlinear_forward(dev(x), packed, b, N, path=tw.BL_PATH_GEMM)
    y_mf = tw.bl_bitlinear_forward_mf(dev(x), wmf, b, N)
    assert np.array_equal(host(y_pn).view(np.uint32), host(y_mf).view(np.uint32))
    rows = np.unique(np.linspace(0, N - 1, 97).astype(np.int64))
    yref, _, _, _ = oracle.bitlinear_forward(x, synth.ternary_codes(key, N, K, rows=rows), beta)
    assert_rel(host(y_mf)[:, rows], yref)


def _mf_q(x, wmf_eye, K):
    """The fused T2-MF64 decode kernel over an identity weight matrix with beta = 1: y = q *
    fp32(gamma / 127) up to one rounding; recover q (exact: |q| <= 127)."""
    one = dev(np.array([1.0], np.float32))
    y = host(tw.bl_bitlinear_forward_mf(dev(x), wmf_eye, one, K))
    _, rg, _ = oracle.quant_act_int8(x)
    scale = (rg / np.float32(127)).astype(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return y, np.rint(y.astype(np.float64) / scale[:, None])


@pytest.mark.parametrize("M,K", [(1, 8192), (3, 2048), (8, 2048), (16, 4096), (2, 28672)])
def test_forward_mf_decode_quantiser_exhaustive(M, K):
    """Every finite fp16 x against every gamma of the ladder, quantised inside the fused
    T2-MF64 decode kernel, must give the oracle's q to the bit; then degenerate rows."""
    wmf = tw.bl_pack_ternary_mf(dev(np.eye(K, dtype=np.int8)))
    rows = ladder_rows(K)
    say("mf decode quant exhaustive", M, K, rows.shape)
    for r0 in range(0, rows.shape[0], M):
        x = np.zeros((M, K), np.float16)
        chunk = rows[r0:r0 + M]
        x[:chunk.shape[0]] = chunk
        x[chunk.shape[0]:, K - 1] = 1.0
        rq, _, _ = oracle.quant_act_int8(x)
        _, q = _mf_q(x, wmf, K)
        assert np.array_equal(q, rq.astype(np.float64)), (r0, x[:, K - 1])
    # degenerate rows: all zero, one NaN, one inf
    x = synth.normal_fp16((M, K), 0, 95, 1)
    x[0] = 0
    if M > 1:
        x[M - 1, 17] = np.float16(np.nan)
    if M > 2:
        x[1, 5] = np.float16(-np.inf)
    y, q = _mf_q(x, wmf, K)
    rq, rg, _ = oracle.quant_act_int8(x)
    assert np.array_equal(y[0], np.zeros(K, np.float32))
    for m in range(1, M):
        if np.isnan(rg[m]):
            assert np.all(np.isnan(y[m]))
        else:
            assert np.array_equal(q[m], rq[m].astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(8, 512, 512), (32, 320, 1024), (64, 1024, 8192),
                                   (33, 49152, 256), (300, 12800, 256)])
def test_forward_mf_equals_forward(M, N, K):
    """The same weights as T2-MF64 and T2-PN-64 give identical outputs (both kernels sum the
    exact integers and apply one epilogue)."""
    say("forward mf", M, N, K)
    x = synth.normal_fp16((M, K), 0, 133, M, K)
    W = synth.normal_fp32((N, K), 0, 134, N, K, std=0.02)
    packed, beta, _ = tw.bl_ternarize_absmean(dev(W))
    wmf = tw.bl_repack_ternary_mf(packed, N, K)
    y_pn = tw.bl_bitlinear_forward(dev(x), packed, beta, N, path=tw.BL_PATH_GEMM)
    y_mf = tw.bl_bitlinear_forward_mf(dev(x), wmf, beta, N)
    assert np.array_equal(host(y_pn).view(np.uint32), host(y_mf).view(np.uint32))
    codes, rbeta = oracle.ternarize_absmean(W)
    yref, _, _, _ = oracle.bitlinear_forward(x, codes, rbeta)
    assert_rel(host(y_mf), yref)
