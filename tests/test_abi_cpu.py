"""The C ABI without a GPU: the library loads, exports every function the header declares,
and its host-side checks return the documented status before anything is queued.

The pointers passed here are fake addresses; every call below fails a host check, so no
HIP call is ever made with them."""
import ctypes
import os

import pytest

LIB_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "ternary_weight_linear_amd", "libbitlinear.so")

OK, NULL, SHAPE, ALIGN, ALIAS, WS, HIP, ARG, CAPACITY = range(9)


@pytest.fixture(scope="module")
def lib():
    import ternary_weight_linear_amd as tw
    return tw.load_library(LIB_PATH)


def test_exports_every_header_function(lib):
    import ternary_weight_linear_amd as tw
    names = tw.header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/libbitlinear.h but not exported"


def test_status_strings_and_version(lib):
    for s in range(9):
        assert lib.bl_status_string(s) and lib.bl_status_string(s) != b"unknown status"
    assert lib.bl_status_string(99) == b"unknown status"
    assert lib.bl_version() >= 10000
    assert lib.bl_last_error() == b""


def test_size_queries(lib):
    assert lib.bl_ternary_packed_bytes(4096, 4096) == 4096 * 4096 // 4
    assert lib.bl_ternary_packed_bytes(28672, 8192) == 28672 * 8192 // 4
    assert lib.bl_ternary_packed_bytes(100, 64) == 0          # N % 64
    assert lib.bl_sign_packed_bytes(4096, 4096) == 2097152
    assert lib.bl_sign_packed_bytes(64, 192) == 0             # K % 128
    assert lib.bl_act_planes_bytes(3, 640) == 3 * 640
    ws = lib.bl_workspace_bytes(512, 8640, 3200)
    assert ws >= 512 * 8640 * 4 and ws % 256 == 0
    assert lib.bl_workspace_bytes(0, 64, 64) == 0


def test_workspace_sizes_over_shapes(lib):
    """The host-side launch plans behind bl_workspace_bytes hold for every batch size,
    including the decode sizes whose sign-plane plan splits K to fit LDS and the prefill
    sizes that plan never takes."""
    for M in (1, 2, 3, 4, 5, 16, 17, 64, 512, 4096):
        for N in (64, 4096, 16384, 28672):
            for K in (128, 4096, 12288, 65536):
                ws = lib.bl_workspace_bytes(M, N, K)
                assert ws > 0 and ws % 256 == 0, (M, N, K)


def _p(v):
    return ctypes.c_void_p(v)


A = 0x100000          # fake, 256-aligned addresses far apart
B = 0x40000000
C = 0x80000000
D = 0xC0000000


def test_pack_checks(lib):
    assert lib.bl_pack_ternary(None, 64, 64, _p(B), None, None) == NULL
    assert lib.bl_pack_ternary(_p(A), 64, 96, _p(B), None, None) == SHAPE
    assert lib.bl_pack_ternary(_p(A), 0, 64, _p(B), None, None) == SHAPE
    assert lib.bl_pack_ternary(_p(A + 1), 64, 64, _p(B), None, None) == ALIGN
    assert lib.bl_pack_ternary(_p(A), 64, 64, _p(A + 64), None, None) == ALIAS
    assert lib.bl_pack_sign(_p(A), 64, 64, _p(B), None) == SHAPE
    assert lib.bl_unpack_sign(_p(A), 64, 128, None, None) == NULL
    assert lib.bl_unpack_ternary(_p(A), 64, 64, _p(A + 512), None, None) == ALIAS


def test_quant_checks(lib):
    assert lib.bl_quant_act_int8(_p(A), 2, 64, None, _p(C), None, None, None) == NULL
    assert lib.bl_quant_act_int8(_p(A), 2, 100, _p(B), _p(C), None, None, None) == SHAPE
    assert lib.bl_quant_act_int8(_p(A), 2, 64, _p(A + 128), _p(C), None, None, None) == ALIAS
    assert lib.bl_quant_act_int8(_p(A), 2, 64, _p(B), _p(B + 64), None, None, None) == ALIAS


def test_product_checks(lib):
    M, N, K = 1, 128, 256
    wsb = lib.bl_workspace_bytes(M, N, K)
    ok = dict(planes=_p(A), gamma=_p(A + 65536), w=_p(B), beta=_p(B + 1 << 20), y=_p(C), ws=_p(D))
    def gemv(**kw):
        a = {**ok, **kw}
        return lib.bl_bitlinear_gemv(a["planes"], a["gamma"], kw.get("M", M), K, a["w"], a["beta"],
                                     kw.get("beta_len", 1), kw.get("N", N), a["y"], a["ws"],
                                     kw.get("wsb", wsb), None)
    assert gemv(planes=None) == NULL
    assert gemv(N=100) == SHAPE
    assert gemv(M=5) == SHAPE
    assert gemv(beta_len=7) == ARG
    assert gemv(wsb=16) == WS
    assert gemv(ws=None) == WS
    assert gemv(ws=_p(D + 16)) == ALIGN
    assert gemv(w=_p(B + 4)) == ALIGN
    assert gemv(y=_p(B + 64)) == ALIAS
    assert lib.bl_bitlinear_acc_i32(_p(A), None, M, K, _p(B), N, _p(C), 9, _p(D), wsb, None) == ARG
    assert lib.bl_bitlinear_acc_i32(None, None, M, K, _p(B), N, _p(C), 2, _p(D), wsb, None) == NULL
    assert lib.bl_bitlinear_forward(_p(A), 1, 64, _p(B), _p(C), 1, 64, _p(C), 5, _p(D),
                                    lib.bl_workspace_bytes(1, 64, 64), None) == ARG
    assert lib.bl_onebit_linear(_p(A), _p(A + 4096), _p(B), _p(B + 8192), 1, 64, 192, _p(C), _p(D),
                                1 << 20, None) == SHAPE
    assert lib.bl_ternarize_absmean(_p(A), 64, 64, None, None, _p(C), _p(D), 1 << 24, None) == NULL
    assert lib.bl_ternarize_absmean(_p(A), 1 << 17, 1 << 16, None, _p(B), _p(C), _p(D), 1 << 24,
                                    None) == SHAPE
    svb = lib.bl_workspace_bytes(1, 64, 128)
    assert lib.bl_svid_rank1(_p(A), 64, 128, 0, _p(B), _p(C), _p(C + 4096), None, _p(D), svb, None) == ARG
    assert lib.bl_svid_rank1(_p(A), 64, 64, 4, _p(B), _p(C), _p(C + 4096), None, _p(D), svb, None) == SHAPE
    assert lib.bl_svid_rank1(_p(A), 64, 128, 4, _p(B), _p(C), _p(C + 64), None, _p(D), svb, None) == ALIAS
    assert lib.bl_svid_rank1(_p(A), 64, 128, 4, _p(B), _p(C), _p(C + 4096), None, _p(D), 64, None) == WS


def test_residual_checks(lib):
    N, K = 128, 256
    KB = K // 128
    ab = N * KB * 4
    pb = N * K // 8
    assert lib.bl_residual_binarize(None, N, K, _p(B), _p(C), _p(B + pb), _p(C + ab), None) == NULL
    assert lib.bl_residual_binarize(_p(A), N, 192, _p(B), _p(C), _p(B + pb), _p(C + ab), None) == SHAPE
    assert lib.bl_residual_binarize(_p(A), 96, K, _p(B), _p(C), _p(B + pb), _p(C + ab), None) == SHAPE
    assert lib.bl_residual_binarize(_p(A), N, K, _p(B + 8), _p(C), _p(B + pb), _p(C + ab), None) == ALIGN
    assert lib.bl_residual_binarize(_p(A), N, K, _p(B), _p(C + 2), _p(B + pb), _p(C + ab), None) == ALIGN
    assert lib.bl_residual_binarize(_p(A), N, K, _p(B), _p(C), _p(B + 16), _p(C + ab), None) == ALIAS
    assert lib.bl_residual_binarize(_p(A), N, K, _p(B), _p(C), _p(B + pb), _p(C + 4), None) == ALIAS
    assert lib.bl_residual_binarize(_p(A), N, K, _p(A + 64), _p(C), _p(B + pb), _p(C + ab), None) == ALIAS
    M = 3
    wsb = lib.bl_workspace_bytes(M, N, K)

    def lin(**kw):
        a = dict(x=_p(A), po=_p(B), ao=_p(B + pb), pr=_p(B + 2 * pb), ar=_p(B + 2 * pb + ab),
                 M=M, N=N, K=K, y=_p(C), ws=_p(D), wsb=wsb)
        a.update(kw)
        return lib.bl_residual_linear(a["x"], a["po"], a["ao"], a["pr"], a["ar"], a["M"], a["N"],
                                      a["K"], a["y"], a["ws"], a["wsb"], None)
    assert lin(ar=None) == NULL
    assert lin(K=64) == SHAPE
    assert lin(M=1048561) == SHAPE
    assert lin(K=(1 << 26) + 128) == SHAPE
    assert lin(x=_p(A + 2)) == ALIGN
    assert lin(ao=_p(B + pb + 1)) == ALIGN
    assert lin(wsb=1024) == WS
    assert lin(y=_p(B + pb)) == ALIAS
    assert lin(y=_p(D + 4096)) == ALIAS
    assert lib.bl_onebit_linear(_p(A + 8), _p(A + 4096), _p(B), _p(B + 8192), 1, 64, 128, _p(C), _p(D),
                                lib.bl_workspace_bytes(1, 64, 128), None) == ALIGN


def test_stack_checks(lib):
    import ternary_weight_linear_amd as tw
    assert lib.bl_stack_plan_bytes(320) == 64 + 64 * 320
    assert lib.bl_stack_plan_bytes(0) == 0 and lib.bl_stack_plan_bytes(4097) == 0
    M = 2
    # two linears: [1024 x 512] then [256 x 1024]; buffers at distinct fake addresses
    shapes = [(1024, 512), (256, 1024)]

    def descs(over=None):
        arr = (tw.bl_linear_desc * 2)()
        for i, (N, K) in enumerate(shapes):
            arr[i] = tw.bl_linear_desc(A + i * 0x100000, B + i * 0x1000000, C + i * 0x1000,
                                       D + i * 0x100000, 1, N, K, 0)
        for (i, f), v in (over or {}).items():
            setattr(arr[i], f, v)
        return arr

    plan = D + 0x10000000
    pb = lib.bl_stack_plan_bytes(2)

    def prep(arr, count=2, m=M, p=plan, nbytes=pb):
        return lib.bl_stack_prepare(ctypes.cast(arr, ctypes.c_void_p), count, m, _p(p), nbytes, None)

    assert lib.bl_stack_prepare(None, 2, M, _p(plan), pb, None) == NULL
    assert prep(descs(), p=0) == NULL
    assert prep(descs({(1, "beta"): None})) == NULL
    assert prep(descs(), count=0) == SHAPE
    assert prep(descs(), count=4097) == SHAPE
    assert prep(descs(), m=5) == SHAPE
    assert prep(descs(), nbytes=pb - 1) == ARG
    assert prep(descs(), p=plan + 8) == ALIGN
    assert prep(descs({(0, "N"): 100})) == SHAPE                 # N % 64
    assert prep(descs({(1, "K"): 65536 + 64})) == SHAPE          # K > 65536
    assert prep(descs({(0, "N"): 4194304, (0, "y"): 0x200000000})) == SHAPE   # M * N > 2^22
    assert prep(descs({(1, "beta_len"): 7})) == ARG
    assert prep(descs({(0, "reserved"): 1})) == ARG
    assert prep(descs({(0, "x"): A + 2})) == ALIGN
    assert prep(descs({(1, "wpacked"): B + 8})) == ALIGN
    assert prep(descs({(0, "y"): A + 512})) == ALIAS              # y over its own x
    assert prep(descs({(1, "y"): B + 64})) == ALIAS               # y over a weight
    assert prep(descs({(0, "y"): C + 0x1000})) == ALIAS           # y over another beta
    assert prep(descs({(1, "y"): D + 1024})) == ALIAS             # y over another y
    assert prep(descs({(0, "y"): plan - 4096})) == ALIAS          # y over the plan
    wsb = lib.bl_workspace_bytes(M, 64, 128)
    assert lib.bl_bitlinear_forward_stack(None, 2, M, _p(A), wsb, None) == NULL
    assert lib.bl_bitlinear_forward_stack(_p(plan), 0, M, _p(A), wsb, None) == SHAPE
    assert lib.bl_bitlinear_forward_stack(_p(plan), 2, 0, _p(A), wsb, None) == SHAPE
    assert lib.bl_bitlinear_forward_stack(_p(plan + 4), 2, M, _p(A), wsb, None) == ALIGN
    assert lib.bl_bitlinear_forward_stack(_p(plan), 2, M, None, wsb, None) == WS
    assert lib.bl_bitlinear_forward_stack(_p(plan), 2, M, _p(A), 4096, None) == WS
    assert lib.bl_bitlinear_forward_stack(_p(plan), 2, M, _p(A + 16), wsb, None) == ALIGN
    assert lib.bl_stack_status(None, None) < 0


def test_mf_checks(lib):
    N, K, M = 128, 256, 8
    pb = N * K // 4
    # packers
    assert lib.bl_pack_ternary_mf(None, N, K, _p(B), None, None) == NULL
    assert lib.bl_pack_ternary_mf(_p(A), 100, K, _p(B), None, None) == SHAPE
    assert lib.bl_pack_ternary_mf(_p(A), N, 96, _p(B), None, None) == SHAPE
    assert lib.bl_pack_ternary_mf(_p(A + 4), N, K, _p(B), None, None) == ALIGN
    assert lib.bl_pack_ternary_mf(_p(A), N, K, _p(A + 64), None, None) == ALIAS
    assert lib.bl_repack_ternary_mf(_p(A), N, K, None, None, None) == NULL
    assert lib.bl_repack_ternary_mf(_p(A), N, K, _p(A + 256), None, None) == ALIAS
    assert lib.bl_repack_ternary_mf(_p(A), N, K, _p(B + 8), None, None) == ALIGN
    wsb = lib.bl_workspace_bytes(M, N, K)

    def gemm(**kw):
        a = dict(q=_p(A), g=_p(A + 0x10000), r=_p(A + 0x20000), M=M, K=K, w=_p(B), b=_p(A + 0x30000),
                 bl=1, N=N, y=_p(C), acc=None, ws=_p(D), wsb=wsb)
        a.update(kw)
        return lib.bl_bitlinear_gemm_mf(a["q"], a["g"], a["r"], a["M"], a["K"], a["w"], a["b"], a["bl"],
                                         a["N"], a["y"], a["acc"], a["ws"], a["wsb"], None)
    assert gemm(r=None) == NULL
    assert gemm(y=None, acc=None) == NULL
    assert gemm(g=None) == NULL
    assert gemm(N=96) == SHAPE
    assert gemm(K=65536 + 64) == SHAPE
    assert gemm(M=1 << 16, K=1 << 15) == SHAPE            # M * K >= 2^31
    assert gemm(bl=3) == ARG
    assert gemm(q=_p(A + 8)) == ALIGN
    assert gemm(wsb=1024) == WS
    assert gemm(y=_p(B + 64)) == ALIAS                    # output over the weights
    assert gemm(y=None, acc=_p(A + 0x20000)) == ALIAS     # acc over rowsum
    assert gemm(acc=_p(C + 16)) == ALIAS                  # y and acc overlap

    def fwd(**kw):
        a = dict(x=_p(A), M=M, K=K, w=_p(B), b=_p(C), bl=1, N=N, y=_p(D + 0x10000000), ws=_p(D), wsb=wsb)
        a.update(kw)
        return lib.bl_bitlinear_forward_mf(a["x"], a["M"], a["K"], a["w"], a["b"], a["bl"], a["N"],
                                           a["y"], a["ws"], a["wsb"], None)
    assert fwd(x=None) == NULL
    assert fwd(K=28672 + 64) == SHAPE
    assert fwd(x=_p(A + 2)) == ALIGN
    assert fwd(wsb=100) == WS
    assert fwd(y=_p(A + 16)) == ALIAS


def test_noalloc_gemv_checks(lib):
    """The no-alloc decode entry point rejects bad arguments, and shapes beyond its scratch
    (M * N > 262144), before touching the GPU."""
    f = lib.bl_bitlinear_forward_gemv_noalloc
    K, N = 256, 1024
    assert f(None, 1, K, _p(B), _p(C), 1, N, _p(D), None) == NULL
    assert f(_p(A), 5, K, _p(B), _p(C), 1, N, _p(D), None) == SHAPE          # M > 4
    assert f(_p(A), 1, 100, _p(B), _p(C), 1, N, _p(D), None) == SHAPE        # K % 64
    assert f(_p(A), 1, 28736, _p(B), _p(C), 1, N, _p(D), None) == SHAPE      # K > 28672
    assert f(_p(A), 4, K, _p(B), _p(C), 1, 65600, _p(D), None) == CAPACITY   # M * N > 2^18
    assert f(_p(A), 1, K, _p(B), _p(C), 1, 262208, _p(D), None) == CAPACITY
    assert f(_p(A), 1, K, _p(B), None, 1, N, _p(D), None) == NULL
    assert f(_p(A), 1, K, _p(B), _p(C), 7, N, _p(D), None) == ARG            # beta_len
    assert f(_p(A + 2), 1, K, _p(B), _p(C), 1, N, _p(D), None) == ALIGN
    assert f(_p(A), 1, K, _p(B), _p(C), 1, N, _p(A + 64), None) == ALIAS     # y over x
    assert f(_p(A), 1, K, _p(B), _p(C), 1, N, _p(B + 128), None) == ALIAS    # y over weights
