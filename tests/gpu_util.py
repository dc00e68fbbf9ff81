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
