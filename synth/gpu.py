"""GPU side of the counter-based ternary code generator (see synth.ternary_codes).

Used where a matrix is too large to draw on the host (the 70B-shaped stack). Loads
synth/libblsynth.so, built together with libbitlinear."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libblsynth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} missing; build with `python ternary_weight_linear_amd/build.py`")
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.syn_ternary_codes.restype = ctypes.c_int
        _lib.syn_ternary_codes.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
    return _lib


def ternary_codes(key: int, N: int, K: int, device, row0: int = 0, rows: int | None = None, out=None):
    """int8 codes of rows row0..row0+rows-1 of an [N, K] matrix, on `device`."""
    lib = _load()
    rows = N - row0 if rows is None else rows
    if out is None:
        out = torch.empty((rows, K), dtype=torch.int8, device=device)
    st = lib.syn_ternary_codes(ctypes.c_void_p(out.data_ptr()), rows, K, ctypes.c_uint64(key), row0,
                               ctypes.c_void_p(torch.cuda.current_stream(out.device).cuda_stream))
    if st != 0:
        raise RuntimeError(f"syn_ternary_codes failed: {st}")
    return out
