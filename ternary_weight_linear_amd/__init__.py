"""Python binding of libbitlinear: BitNet b1.58 ternary, OneBit sign-only and
residual-binarised linear layers on MI355X (gfx950).

Every function here only marshals arguments: it checks tensor dtypes, devices and
contiguity, allocates outputs with torch (device memory is PyTorch's job) and calls the
C entry point of the same name on the current HIP stream. All arithmetic happens in the
library's HIP kernels. Importing this module fails loudly if the library is not built.

See include/libbitlinear.h for the contract of each call (shapes, layouts, errors).
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbitlinear.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "libbitlinear.h")

BL_PATH_AUTO, BL_PATH_GEMV, BL_PATH_GEMM = 0, 1, 2


class BitLinearError(RuntimeError):
    def __init__(self, status: int, where: str, lib):
        msg = lib.bl_status_string(status).decode()
        extra = lib.bl_last_error().decode() if status == 6 else ""
        super().__init__(f"{where}: status {status} ({msg}){': ' + extra if extra else ''}")
        self.status = status


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SIGS = {
    "bl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bl_last_error": (ctypes.c_char_p, []),
    "bl_version": (ctypes.c_int, []),
    "bl_ternary_packed_bytes": (_SZ, [_I64, _I64]),
    "bl_sign_packed_bytes": (_SZ, [_I64, _I64]),
    "bl_act_planes_bytes": (_SZ, [_I64, _I64]),
    "bl_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "bl_workspace_clear": (ctypes.c_int, [_P, _SZ, _P]),
    "bl_ternarize_absmean": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "bl_pack_ternary": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "bl_unpack_ternary": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "bl_pack_sign": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "bl_unpack_sign": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "bl_quant_act_int8": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "bl_bitlinear_gemv": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "bl_bitlinear_gemm": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "bl_bitlinear_acc_i32": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, ctypes.c_int, _P, _SZ, _P]),
    "bl_bitlinear_forward": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, _I64, _P, ctypes.c_int, _P, _SZ, _P]),
    "bl_onebit_linear": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "bl_svid_rank1": (ctypes.c_int, [_P, _I64, _I64, ctypes.c_int, _P, _P, _P, _P, _P, _SZ, _P]),
    "bl_residual_binarize": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _P]),
    "bl_residual_linear": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "bl_pack_ternary_mf": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "bl_repack_ternary_mf": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "bl_bitlinear_gemm_mf": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "bl_bitlinear_forward_mf": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "bl_stack_plan_bytes": (_SZ, [_I64]),
    "bl_stack_prepare": (ctypes.c_int, [_P, _I64, _I64, _P, _SZ, _P]),
    "bl_bitlinear_forward_stack": (ctypes.c_int, [_P, _I64, _I64, _P, _SZ, _P]),
    "bl_stack_status": (ctypes.c_int, [_P, _P]),
    "bl_bitlinear_forward_gemv_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _I64, _I64, _P, _P]),
}


class bl_linear_desc(ctypes.Structure):
    """One linear of a stack plan (the C struct of the same name)."""
    _fields_ = [("x", _P), ("wpacked", _P), ("beta", _P), ("y", _P),
                ("beta_len", _I64), ("N", _I64), ("K", _I64), ("reserved", _I64)]


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/libbitlinear.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bl_[a-z0-9_]+)\s*\(", text)))


def load_library(path: str = LIB_PATH):
    """dlopen libbitlinear.so and attach the C signatures. Raises if it is not built."""
    if not os.path.exists(path):
        raise ImportError(f"libbitlinear is not built ({path} missing); run "
                          "`python ternary_weight_linear_amd/build.py` or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        if not hasattr(lib, name):
            raise ImportError(f"{path} lacks {name}: the library is stale; rebuild it with "
                              "`python ternary_weight_linear_amd/build.py`")
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def _check(status: int, where: str):
    if status != 0:
        raise BitLinearError(status, where, _lib)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {devs}")
    d = devs.pop()
    if d.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {d}")
    return d


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _half_bits(t, name):
    _need(t, torch.float16, name)
    return t


# ------------------------------------------------------------------------------------------
# workspace: one zero-filled buffer per device, grown on demand, kept zero by the library
# ------------------------------------------------------------------------------------------
_ws_lock = threading.Lock()
_ws = {}


def workspace(device, nbytes: int):
    """A zero-filled device buffer of at least nbytes for `device` (cached, grown on demand).
    Calls that share it must be ordered on one stream, as the C contract requires."""
    device = torch.device(device)
    with _ws_lock:
        buf = _ws.get(device)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            _ws[device] = buf
        return buf


def _ws_for(device, M, N, K):
    nbytes = _lib.bl_workspace_bytes(M, N, K)
    if nbytes == 0:
        raise ValueError(f"invalid shape M={M} N={N} K={K}")
    buf = workspace(device, nbytes)
    return buf, buf.numel()


# ------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------
def bl_ternary_packed_bytes(N: int, K: int) -> int:
    return _lib.bl_ternary_packed_bytes(N, K)


def bl_sign_packed_bytes(N: int, K: int) -> int:
    return _lib.bl_sign_packed_bytes(N, K)


def bl_act_planes_bytes(M: int, K: int) -> int:
    return _lib.bl_act_planes_bytes(M, K)


def bl_workspace_bytes(M: int, N: int, K: int) -> int:
    return _lib.bl_workspace_bytes(M, N, K)


def bl_ternarize_absmean(W, want_codes: bool = False):
    """fp32 W [N, K] -> (packed uint8 [N*K/4], beta fp32 [1], codes int8 [N, K] or None)."""
    _need(W, torch.float32, "W")
    d = _dev(W)
    N, K = W.shape
    packed = torch.empty(max(_lib.bl_ternary_packed_bytes(N, K), 1), dtype=torch.uint8, device=d)
    beta = torch.empty(1, dtype=torch.float32, device=d)
    codes = torch.empty((N, K), dtype=torch.int8, device=d) if want_codes else None
    ws, wsb = _ws_for(d, 1, N, K)
    _check(_lib.bl_ternarize_absmean(_ptr(W), N, K, _ptr(codes), _ptr(packed), _ptr(beta),
                                     _ptr(ws), wsb, _stream(d)), "bl_ternarize_absmean")
    return packed, beta, codes


def bl_pack_ternary(codes, n_invalid=None):
    """int8 codes [N, K] -> uint8 T2-PN-64 [N*K/4]. n_invalid: optional int32 [1] counter."""
    _need(codes, torch.int8, "codes")
    d = _dev(codes, n_invalid)
    N, K = codes.shape
    out = torch.empty(max(_lib.bl_ternary_packed_bytes(N, K), 1), dtype=torch.uint8, device=d)
    _check(_lib.bl_pack_ternary(_ptr(codes), N, K, _ptr(out), _ptr(n_invalid), _stream(d)),
           "bl_pack_ternary")
    return out


def bl_unpack_ternary(packed, N: int, K: int, n_invalid=None):
    _need(packed, torch.uint8, "packed")
    d = _dev(packed, n_invalid)
    out = torch.empty((N, K), dtype=torch.int8, device=d)
    _check(_lib.bl_unpack_ternary(_ptr(packed), N, K, _ptr(out), _ptr(n_invalid), _stream(d)),
           "bl_unpack_ternary")
    return out


def bl_pack_sign(W):
    """fp32 W [N, K] -> uint8 S1-128 [N*K/8] (bit set iff W < 0)."""
    _need(W, torch.float32, "W")
    d = _dev(W)
    N, K = W.shape
    out = torch.empty(max(_lib.bl_sign_packed_bytes(N, K), 1), dtype=torch.uint8, device=d)
    _check(_lib.bl_pack_sign(_ptr(W), N, K, _ptr(out), _stream(d)), "bl_pack_sign")
    return out


def bl_unpack_sign(packed, N: int, K: int):
    _need(packed, torch.uint8, "packed")
    d = _dev(packed)
    out = torch.empty((N, K), dtype=torch.int8, device=d)
    _check(_lib.bl_unpack_sign(_ptr(packed), N, K, _ptr(out), _stream(d)), "bl_unpack_sign")
    return out


def bl_quant_act_int8(x, want_q: bool = True, want_rowsum: bool = True, want_planes: bool = True):
    """fp16 x [M, K] -> (q int8 [M, K] | None, gamma fp32 [M], rowsum int32 [M] | None,
    planes uint32 [M, K/64, 16] | None)."""
    _half_bits(x, "x")
    d = _dev(x)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=d) if want_q else None
    gamma = torch.empty(M, dtype=torch.float32, device=d)
    rowsum = torch.empty(M, dtype=torch.int32, device=d) if want_rowsum else None
    planes = torch.empty((M, K // 64, 16), dtype=torch.int32, device=d) if want_planes else None
    _check(_lib.bl_quant_act_int8(_ptr(x), M, K, _ptr(q), _ptr(gamma), _ptr(rowsum), _ptr(planes),
                                  _stream(d)), "bl_quant_act_int8")
    return q, gamma, rowsum, planes


def _beta_len(beta, N):
    _need(beta, torch.float32, "beta")
    return beta.numel()


def bl_bitlinear_gemv(planes, gamma, wpacked, beta, N: int, K: int, out=None):
    """Add-only GEMV (M <= 4): y fp32 [M, N]."""
    _need(planes, torch.int32, "planes")
    _need(gamma, torch.float32, "gamma")
    _need(wpacked, torch.uint8, "wpacked")
    d = _dev(planes, gamma, wpacked, beta)
    M = gamma.numel()
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_bitlinear_gemv(_ptr(planes), _ptr(gamma), M, K, _ptr(wpacked), _ptr(beta),
                                  _beta_len(beta, N), N, _ptr(y), _ptr(ws), wsb, _stream(d)),
           "bl_bitlinear_gemv")
    return y


def bl_bitlinear_gemm(q, gamma, wpacked, beta, N: int, out=None):
    """int8-MFMA GEMM: y fp32 [M, N]."""
    _need(q, torch.int8, "q")
    _need(gamma, torch.float32, "gamma")
    _need(wpacked, torch.uint8, "wpacked")
    d = _dev(q, gamma, wpacked, beta)
    M, K = q.shape
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_bitlinear_gemm(_ptr(q), _ptr(gamma), M, K, _ptr(wpacked), _ptr(beta),
                                  _beta_len(beta, N), N, _ptr(y), _ptr(ws), wsb, _stream(d)),
           "bl_bitlinear_gemm")
    return y


def bl_bitlinear_acc_i32(wpacked, N: int, K: int, q=None, planes=None, M: int | None = None,
                         path: int = BL_PATH_AUTO):
    """Raw int32 accumulators [M, N] of the chosen kernel path."""
    _need(wpacked, torch.uint8, "wpacked")
    if q is not None:
        _need(q, torch.int8, "q")
    if planes is not None:
        _need(planes, torch.int32, "planes")
    d = _dev(wpacked, q, planes)
    if M is None:
        M = q.shape[0] if q is not None else planes.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_bitlinear_acc_i32(_ptr(q), _ptr(planes), M, K, _ptr(wpacked), N, _ptr(acc), path,
                                     _ptr(ws), wsb, _stream(d)), "bl_bitlinear_acc_i32")
    return acc


def bl_bitlinear_forward(x, wpacked, beta, N: int, path: int = BL_PATH_AUTO, out=None):
    """fp16 x [M, K] -> y fp32 [M, N]: quantise + GEMV/GEMM + rescale."""
    _half_bits(x, "x")
    _need(wpacked, torch.uint8, "wpacked")
    d = _dev(x, wpacked, beta)
    M, K = x.shape
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_bitlinear_forward(_ptr(x), M, K, _ptr(wpacked), _ptr(beta), _beta_len(beta, N),
                                     N, _ptr(y), path, _ptr(ws), wsb, _stream(d)),
           "bl_bitlinear_forward")
    return y


def bl_onebit_linear(x, g, spacked, h, out=None):
    """OneBit layer: fp16 x [M, K], g fp16 [K], S1-128 signs, h fp16 [N] -> y fp32 [M, N]."""
    _half_bits(x, "x")
    _half_bits(g, "g")
    _half_bits(h, "h")
    _need(spacked, torch.uint8, "spacked")
    d = _dev(x, g, spacked, h)
    M, K = x.shape
    N = h.numel()
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_onebit_linear(_ptr(x), _ptr(g), _ptr(spacked), _ptr(h), M, N, K, _ptr(y),
                                 _ptr(ws), wsb, _stream(d)), "bl_onebit_linear")
    return y


def bl_svid_rank1(W, iters: int = 20):
    """SVID init from fp32 W [N, K]: (S1-128 signs uint8 [N*K/8], g fp16 [K], h fp16 [N], sigma fp32 [1])."""
    _need(W, torch.float32, "W")
    d = _dev(W)
    N, K = W.shape
    spacked = torch.empty(max(_lib.bl_sign_packed_bytes(N, K), 1), dtype=torch.uint8, device=d)
    g = torch.empty(K, dtype=torch.float16, device=d)
    h = torch.empty(N, dtype=torch.float16, device=d)
    sigma = torch.empty(1, dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, 1, N, K)
    _check(_lib.bl_svid_rank1(_ptr(W), N, K, iters, _ptr(spacked), _ptr(g), _ptr(h), _ptr(sigma),
                              _ptr(ws), wsb, _stream(d)), "bl_svid_rank1")
    return spacked, g, h, sigma


def bl_residual_binarize(W):
    """Residual binarisation of fp32 W [N, K]: (planes_o uint8 [N*K/8], alpha_o fp32 [N, K/128],
    planes_r uint8 [N*K/8], alpha_r fp32 [N, K/128])."""
    _need(W, torch.float32, "W")
    d = _dev(W)
    N, K = W.shape
    nb = max(_lib.bl_sign_packed_bytes(N, K), 1)
    po = torch.empty(nb, dtype=torch.uint8, device=d)
    pr = torch.empty(nb, dtype=torch.uint8, device=d)
    ao = torch.empty((N, max(K // 128, 1)), dtype=torch.float32, device=d)
    ar = torch.empty((N, max(K // 128, 1)), dtype=torch.float32, device=d)
    _check(_lib.bl_residual_binarize(_ptr(W), N, K, _ptr(po), _ptr(ao), _ptr(pr), _ptr(ar),
                                     _stream(d)), "bl_residual_binarize")
    return po, ao, pr, ar


def bl_residual_linear(x, planes_o, alpha_o, planes_r, alpha_r, out=None):
    """Residual-binarised layer: fp16 x [M, K] and the outputs of bl_residual_binarize
    -> y fp32 [M, N]."""
    _half_bits(x, "x")
    _need(planes_o, torch.uint8, "planes_o")
    _need(planes_r, torch.uint8, "planes_r")
    _need(alpha_o, torch.float32, "alpha_o")
    _need(alpha_r, torch.float32, "alpha_r")
    d = _dev(x, planes_o, alpha_o, planes_r, alpha_r)
    M, K = x.shape
    N = alpha_o.shape[0]
    if alpha_o.shape != (N, K // 128) or alpha_r.shape != (N, K // 128):
        raise ValueError(f"alpha_o/alpha_r must be [N, K/128] = [{N}, {K // 128}]")
    if planes_o.numel() != N * K // 8 or planes_r.numel() != N * K // 8:
        raise ValueError(f"planes must hold N*K/8 = {N * K // 8} bytes")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_residual_linear(_ptr(x), _ptr(planes_o), _ptr(alpha_o), _ptr(planes_r),
                                   _ptr(alpha_r), M, N, K, _ptr(y), _ptr(ws), wsb, _stream(d)),
           "bl_residual_linear")
    return y


def bl_pack_ternary_mf(codes, n_invalid=None):
    """int8 codes [N, K] -> T2-MF64 uint8 [N*K/4] (the matrix-core layout)."""
    _need(codes, torch.int8, "codes")
    d = _dev(codes)
    N, K = codes.shape
    packed = torch.empty(max(_lib.bl_ternary_packed_bytes(N, K), 1), dtype=torch.uint8, device=d)
    _check(_lib.bl_pack_ternary_mf(_ptr(codes), N, K, _ptr(packed), _ptr(n_invalid), _stream(d)),
           "bl_pack_ternary_mf")
    return packed


def bl_repack_ternary_mf(t2pn, N: int, K: int, out=None, n_invalid=None):
    """T2-PN-64 uint8 [N*K/4] -> T2-MF64 uint8 [N*K/4] (same weights)."""
    _need(t2pn, torch.uint8, "t2pn")
    d = _dev(t2pn)
    mf = out if out is not None else torch.empty(max(_lib.bl_ternary_packed_bytes(N, K), 1),
                                                 dtype=torch.uint8, device=d)
    _check(_lib.bl_repack_ternary_mf(_ptr(t2pn), N, K, _ptr(mf), _ptr(n_invalid), _stream(d)),
           "bl_repack_ternary_mf")
    return mf


def bl_bitlinear_gemm_mf(q, gamma, rowsum, wmf, beta, N: int, want_y: bool = True,
                         want_acc: bool = False):
    """int8 q [M, K], gamma fp32 [M], rowsum int32 [M], T2-MF64 weights -> (y fp32 [M, N] or
    None, acc int32 [M, N] or None)."""
    _need(q, torch.int8, "q")
    _need(rowsum, torch.int32, "rowsum")
    _need(wmf, torch.uint8, "wmf")
    d = _dev(q, rowsum, wmf)
    M, K = q.shape
    y = torch.empty((M, N), dtype=torch.float32, device=d) if want_y else None
    acc = torch.empty((M, N), dtype=torch.int32, device=d) if want_acc else None
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_bitlinear_gemm_mf(_ptr(q), _ptr(gamma), _ptr(rowsum), M, K, _ptr(wmf),
                                     _ptr(beta), _beta_len(beta, N) if beta is not None else 1, N,
                                     _ptr(y), _ptr(acc), _ptr(ws), wsb, _stream(d)),
           "bl_bitlinear_gemm_mf")
    return y, acc


def bl_bitlinear_forward_mf(x, wmf, beta, N: int, out=None):
    """fp16 x [M, K] -> y fp32 [M, N] from T2-MF64 weights: one fused quantise + matrix-core
    launch at decode sizes (see the header), else quantiser + matrix-core product."""
    _half_bits(x, "x")
    _need(wmf, torch.uint8, "wmf")
    d = _dev(x, wmf, beta)
    M, K = x.shape
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=d)
    ws, wsb = _ws_for(d, M, N, K)
    _check(_lib.bl_bitlinear_forward_mf(_ptr(x), M, K, _ptr(wmf), _ptr(beta), _beta_len(beta, N),
                                        N, _ptr(y), _ptr(ws), wsb, _stream(d)),
           "bl_bitlinear_forward_mf")
    return y


def bl_bitlinear_forward_gemv_noalloc(x, wpacked, beta, out):
    """fp16 x [M, K] -> out fp32 [M, N] (caller-allocated): the GEMV path of
    bl_bitlinear_forward with the library's own scratch instead of a workspace; nothing is
    allocated by this call. 1 <= M <= 4, M * N <= 262144."""
    _half_bits(x, "x")
    _need(wpacked, torch.uint8, "wpacked")
    _need(out, torch.float32, "out")
    d = _dev(x, wpacked, beta, out)
    M, K = x.shape
    N = out.shape[1]
    _check(_lib.bl_bitlinear_forward_gemv_noalloc(_ptr(x), M, K, _ptr(wpacked), _ptr(beta),
                                                  _beta_len(beta, N), N, _ptr(out), _stream(d)),
           "bl_bitlinear_forward_gemv_noalloc")
    return out


def bl_stack_plan_bytes(count: int) -> int:
    return _lib.bl_stack_plan_bytes(count)


def bl_stack_prepare(linears, M: int, descs_only: bool = False):
    """Device plan (uint8 tensor) for a list of linears, each a tuple
    (x fp16 [M, K], wpacked uint8 T2-PN-64, beta fp32 [1] or [N], y fp32 [M, N]).
    The plan keeps raw pointers: the tensors must stay alive (and in place) while it is used.
    descs_only=True returns the ctypes descriptor array instead (no device work)."""
    if not linears:
        raise ValueError("a stack needs at least one linear")
    arr = (bl_linear_desc * len(linears))()
    tensors = []
    for i, (x, wpacked, beta, y) in enumerate(linears):
        _half_bits(x, f"linears[{i}].x")
        _need(wpacked, torch.uint8, f"linears[{i}].wpacked")
        _need(beta, torch.float32, f"linears[{i}].beta")
        _need(y, torch.float32, f"linears[{i}].y")
        if x.dim() != 2 or y.dim() != 2 or x.shape[0] != M or y.shape[0] != M:
            raise ValueError(f"linears[{i}]: x and y must be [M, *] with M = {M}")
        N, K = y.shape[1], x.shape[1]
        arr[i] = bl_linear_desc(x.data_ptr(), wpacked.data_ptr(), beta.data_ptr(), y.data_ptr(),
                                _beta_len(beta, N), N, K, 0)
        tensors += [x, wpacked, beta, y]
    if descs_only:
        return arr
    d = _dev(*tensors)
    nbytes = _lib.bl_stack_plan_bytes(len(linears))
    if nbytes == 0:
        raise ValueError(f"a stack holds 1 .. 4096 linears, got {len(linears)}")
    plan = torch.empty(nbytes, dtype=torch.uint8, device=d)
    _check(_lib.bl_stack_prepare(ctypes.cast(arr, _P), len(linears), M, _ptr(plan), nbytes,
                                 _stream(d)), "bl_stack_prepare")
    return plan


def bl_bitlinear_forward_stack(plan, count: int, M: int):
    """Run every linear of `plan` in order in one persistent launch (outputs land in the
    y tensors the plan was prepared with)."""
    _need(plan, torch.uint8, "plan")
    d = _dev(plan)
    ws, wsb = _ws_for(d, M, 64, 128)
    _check(_lib.bl_bitlinear_forward_stack(_ptr(plan), count, M, _ptr(ws), wsb, _stream(d)),
           "bl_bitlinear_forward_stack")


def bl_stack_status(plan) -> int:
    """Device status word of a plan (synchronises the current stream)."""
    d = _dev(plan)
    st = _lib.bl_stack_status(_ptr(plan), _stream(d))
    if st < 0:
        raise BitLinearError(6, "bl_stack_status", _lib)
    return st


__all__ = [n for n in list(globals()) if n.startswith("bl_")] + [
    "BitLinearError", "workspace", "load_library", "header_functions", "LIB_PATH",
    "BL_PATH_AUTO", "BL_PATH_GEMV", "BL_PATH_GEMM"]
