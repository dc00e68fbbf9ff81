"""Seeded synthetic inputs for the BitLinear / OneBit linear layers.

This module only draws inputs. It holds none of the layers' arithmetic
(no quantisation, packing, accumulation or scaling), so both the CPU oracle
and the HIP path can consume its output without sharing any method code.

Two kinds of generator live here:

* NumPy draws (``PCG64`` seeded from a ``SeedSequence`` of integer keys) for
  anything the host can hold: fp16 activations, fp32 weights, fp16 value
  vectors, outlier-channel masks.
* A counter-based ternary code generator built on SplitMix64 (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014). Code
  ``(n, k)`` of a matrix is ``splitmix64_output(key, n*K + k + 1) mod 3 - 1``,
  so any row of any matrix can be regenerated alone. ``synth/csrc/synth.hip``
  implements the same published definition on the GPU for matrices too large
  to draw on the host; the two are checked against each other in the tests.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_KEY_MUL = 1_000_003


def rng(seed: int, *keys: int) -> np.random.Generator:
    """NumPy generator for one (seed, keys...) stream."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, keys)])))


def normal_fp16(shape, seed: int, *keys: int, std: float = 1.0) -> np.ndarray:
    """fp16 array drawn from N(0, std^2): drawn in fp64, rounded to fp16 (RNE)."""
    return (rng(seed, *keys).standard_normal(shape) * std).astype(np.float16)


def normal_fp32(shape, seed: int, *keys: int, std: float = 1.0) -> np.ndarray:
    """fp32 array drawn from N(0, std^2): drawn in fp64, rounded to fp32 (RNE)."""
    return (rng(seed, *keys).standard_normal(shape) * std).astype(np.float32)


def uniform_fp16(shape, lo: float, hi: float, seed: int, *keys: int) -> np.ndarray:
    """fp16 array drawn from U(lo, hi): drawn in fp64, rounded to fp16 (RNE)."""
    return rng(seed, *keys).uniform(lo, hi, shape).astype(np.float16)


def with_outlier_channels(x16: np.ndarray, frac: float, factor: float, seed: int, *keys: int):
    """Scale round(frac*K) columns of x (chosen without replacement, the same
    columns for every row) by `factor`; the product is formed in fp64 and
    rounded back to fp16. Returns (x, sorted column indices)."""
    K = x16.shape[-1]
    n = int(round(frac * K))
    cols = np.sort(rng(seed, *keys).choice(K, size=n, replace=False))
    out = x16.astype(np.float64)
    out[..., cols] *= factor
    return out.astype(np.float16), cols


def matrix_key(seed: int, config: int, layer: int, matrix: int) -> int:
    """64-bit key of one synthetic weight matrix (wraps modulo 2^64)."""
    k = int(seed)
    for v in (config, layer, matrix):
        k = (k * _KEY_MUL + int(v)) & 0xFFFFFFFFFFFFFFFF
    return k


def splitmix64(key: int, counter: np.ndarray) -> np.ndarray:
    """The counter-th output (counter >= 1) of SplitMix64 seeded with `key`:
    state = key + counter * golden_gamma, then the published finaliser."""
    with np.errstate(over="ignore"):
        z = np.uint64(key) + counter.astype(np.uint64) * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def ternary_codes(key: int, N: int, K: int, rows=None) -> np.ndarray:
    """Counter-based ternary codes in {-1, 0, +1}, each with probability ~1/3.

    Returns int8 [len(rows), K] (all N rows when `rows` is None)."""
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    ctr = rows[:, None] * np.int64(K) + np.arange(K, dtype=np.int64)[None, :] + 1
    return (splitmix64(key, ctr) % np.uint64(3)).astype(np.int8) - np.int8(1)


# --------------------------------------------------------------------------------------
# The five workloads (shapes are out x in, i.e. N x K). Each entry lists the linears of
# one layer: (name, N, K).
# --------------------------------------------------------------------------------------
LLAMA7B_LINEARS = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                   ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
LLAMA3B_LINEARS = [("q", 3200, 3200), ("k", 3200, 3200), ("v", 3200, 3200), ("o", 3200, 3200),
                   ("gate", 8640, 3200), ("up", 8640, 3200), ("down", 3200, 8640)]
LLAMA70B_LINEARS = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
                    ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]
LLAMA70B_LAYERS = 80
# Per-tensor scale used where codes are drawn directly instead of from a float matrix: the
# expected mean |W| of N(0, 0.02^2), i.e. 0.02*sqrt(2/pi), rounded to fp32.
BETA_DIRECT = np.float32(0.02 * np.sqrt(2.0 / np.pi))
