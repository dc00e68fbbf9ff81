"""The no-alloc decode entry point (library-owned scratch instead of a workspace) through
the C ABI: two calls in a row, the second smaller, each bitwise equal to
bl_bitlinear_forward on the GEMV path (same kernels, same integers, same epilogue), and the
smaller one against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import ternary_weight_linear_amd as tw
from tests.gpu_util import DEV, assert_rel, dev, host, say

pytestmark = pytest.mark.gpu


def _call(x, packed, beta, N):
    M, K = x.shape
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    st = tw._lib.bl_bitlinear_forward_gemv_noalloc(
        ctypes.c_void_p(x.data_ptr()), M, K, ctypes.c_void_p(packed.data_ptr()),
        ctypes.c_void_p(beta.data_ptr()), beta.numel(), N, ctypes.c_void_p(y.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, tw._lib.bl_status_string(st)
    return y


def test_noalloc_gemv_matches_forward_twice():
    # call 1: 2 x 65536 outputs from 8192 inputs (K split across workgroups, 131072 split
    # words); call 2: 1 x 4096 from 4096 (a deeper split over fewer words)
    cases = [(2, 65536, 8192, 0), (1, 4096, 4096, 1)]
    for M, N, K, seed in cases:
        say("noalloc gemv", M, N, K)
        codes = synth.ternary_codes(synth.matrix_key(seed, 140, N, K), N, K)
        packed = tw.bl_pack_ternary(dev(codes))
        x16 = synth.normal_fp16((M, K), seed, 141, M, K)
        x = dev(x16)
        beta = dev(synth.uniform_fp16((N,), 0.01, 0.03, seed, 142).astype(np.float32))
        y = _call(x, packed, beta, N)
        ref = tw.bl_bitlinear_forward(x, packed, beta, N, path=tw.BL_PATH_GEMV)
        assert np.array_equal(host(y).view(np.uint32), host(ref).view(np.uint32))
        y2 = _call(x, packed, beta, N)                 # the scratch was left zero
        assert np.array_equal(host(y2).view(np.uint32), host(ref).view(np.uint32))
        if N <= 4096:
            yref, _, _, _ = oracle.bitlinear_forward(x16, codes, host(beta))
            assert_rel(host(y), yref)
