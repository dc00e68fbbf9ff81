"""Helpers shared by the GPU parity tests (host <-> device copies, tolerance checks)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    """Name the case about to run on the GPU (flushed, so a crash still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_rel(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = 1e-3):
    """Elementwise |y - ref| <= tol * |ref|; where ref == 0 the GPU value must be 0."""
    y_gpu = y_gpu.astype(np.float64)
    err = np.abs(y_gpu - y_ref)
    bad = err > tol * np.abs(y_ref)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements out of tolerance, first at {tuple(i)}: "
                             f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r}")
    return float((err / np.where(y_ref == 0, 1, np.abs(y_ref))).max()) if y_ref.size else 0.0


def assert_scaled(y_gpu: np.ndarray, y_ref: np.ndarray, scale: np.ndarray, tol: float = 1e-3):
    """|y - ref| <= tol * scale (the OneBit componentwise error scale)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = err > tol * scale
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements out of tolerance, first at {tuple(i)}: "
                             f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} scale={scale[tuple(i)]!r}")
    return float((err / scale).max())


def gamma_ladder() -> np.ndarray:
    """fp16 row maxima for the exhaustive quantiser sweeps (>= 64 values): every power of two
    of a spread of binades with its neighbours one ulp below and above (the subnormal range
    included, where an ulp is 2^-24), the largest subnormal and the extremes, and mantissas
    spread over [1, 2) in a few binades. Sorted and unique."""
    vals = []
    for p in (-24, -23, -20, -17, -15, -14, -13, -10, -7, -4, -1, 0, 1, 2, 3, 4, 6, 7, 8, 10,
              12, 14, 15):
        b = np.float16(2.0 ** p)
        vals += [b, np.nextafter(b, np.float16(0)), np.nextafter(b, np.float16(np.inf))]
    vals += [np.float16(v) for v in (65504, 127.0, 3.14, 0.0999, 6.1e-5, 1023 * 2.0 ** -24,
                                     1.5 * 2.0 ** -14, 100.0, 1.0 / 3.0, 7.7, 254.0, 1e4)]
    for e, j in ((-9, 3), (-2, 11), (0, 19), (5, 27), (9, 31), (13, 7), (1, 1021), (-6, 513)):
        vals.append(np.float16((1 + j / 1024) * 2.0 ** e))
    v = np.unique(np.array([x for x in vals if x > 0], dtype=np.float16))
    assert v.size >= 64
    return v


def finite_fp16() -> np.ndarray:
    """Every finite fp16 value (63,488 of them, both zeros included)."""
    all16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return all16[np.isfinite(all16)]
