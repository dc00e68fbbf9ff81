"""Packed weight and activation layouts, written element by element from their spec.

ORACLE — test infrastructure only (see the package docstring).

The pages fix only the information content: ternary weights carry log2(3) ~ 1.58
bits and were measured with a 2-bit kernel ([b158], "BitNet b1.58 介绍" and the
latency/memory paragraph of "实验及结果"); OneBit keeps one bit per weight
([onebit], "1. 新的1bit结构", Fig. 3 and the 4096x4096 storage count). The bit
layouts below are this library's own choice; the same text is in the C header.

T2-PN-64 (ternary, 2 bits/weight). N % 64 == 0, K % 64 == 0.
  Tile (tn, tk) = rows 64tn..64tn+63, inputs 64tk..64tk+63, 1024 bytes at byte
  (tn*(K/64) + tk)*1024. Row r of a tile = bytes 16r..16r+15 = four little-endian
  uint32 words [P0, P1, N0, N1]. Word X_h covers k = 64tk + 32h + c, c in 0..31;
  input c = 4j + i sits at bit 8i + j (byte i, bit j). P bit set iff w = +1,
  N bit set iff w = -1; both clear iff w = 0; both set is invalid.

X8-64 (activation bit planes of int8 q, used by the add-only GEMV).
  For row m and 64-input tile t: 16 uint32 words at word (m*(K/64) + t)*16.
  Word 2b + h holds bit b (two's complement, b = 0..7) of q[m, 64t + 32h + c],
  with c = 4j + i at bit 8i + j, the same order as T2-PN-64.

T2-MF64 (ternary, 2 bits/weight, for int8 matrix-core operands). N % 64 == 0,
  K % 64 == 0. Tiles as T2-PN-64 (64 rows x 64 inputs, 1024 bytes, same order), read
  as 256 little-endian uint32 words. Tile row r = 16f + u (f, u: 0..3, 0..15) and tile
  input c = 16g + 4j + i (g, j, i: 0..3) sit in word 4*(16g + u) + j at bits 8i + 2f
  and 8i + 2f + 1. For f = 0, 1, 2 the field holds the code w + 1 (0, 1, 2; 3 is
  invalid); for f = 3 it holds w in two's complement (00 = 0, 01 = +1, 11 = -1; 10 is
  invalid). Masking word j with 0x03030303 << 2f leaves, in byte i, 4^f (w + 1) for
  f < 3 and, read as a signed byte, 64 w for f = 3.

S1-128 (sign, 1 bit/weight). N % 64 == 0, K % 128 == 0.
  Tile (tn, tk) = rows 64tn.., inputs 128tk.., 1024 bytes at byte
  (tn*(K/128) + tk)*1024, read as 256 little-endian uint32 words. Tile row
  r = 16f + u (f, u: 0..3, 0..15) and tile input c = 32s + 8g + 2q + e
  (s, g, q: 0..3; e: 0..1) sit in word 4*(16g + u) + f at bit 16e + 4s + q.
  Bit set iff the weight is -1.
"""
from __future__ import annotations

import numpy as np


def ternary_packed_bytes(N: int, K: int) -> int:
    return N * K // 4


def sign_packed_bytes(N: int, K: int) -> int:
    return N * K // 8


def _t2_byte_and_bit(N: int, K: int):
    """Byte offset of the P flag of every (n, k), the bit within that byte, and the
    offset to add for the N flag -- straight from the T2-PN-64 text."""
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    tn, r = n // 64, n % 64
    tk, kk = k // 64, k % 64
    h, c = kk // 32, kk % 32
    i, j = c % 4, c // 4                      # c = 4j + i  ->  bit 8i + j of the word
    word_p = (tn * (K // 64) + tk) * 1024 + 16 * r + 4 * h
    byte_p = word_p + i                       # bit 8i + j of a little-endian word = byte i, bit j
    return byte_p, np.broadcast_to(j, byte_p.shape), 8


def pack_ternary(codes: np.ndarray, count_invalid: bool = False):
    """int8 codes [N, K] -> uint8 T2-PN-64 bytes [N*K/4].

    A code other than -1/0/+1 packs as 0 and is counted as invalid (the count is
    returned when `count_invalid`). Parity: pinned by hand-worked bytes, the round
    trip and word invariants in the CPU tests."""
    codes = np.asarray(codes)
    N, K = codes.shape
    assert N % 64 == 0 and K % 64 == 0, "T2-PN-64 needs N % 64 == 0 and K % 64 == 0"
    out = np.zeros(ternary_packed_bytes(N, K), dtype=np.uint8)
    byte_p, bit, n_off = _t2_byte_and_bit(N, K)
    bitval = (1 << bit).astype(np.uint8)
    plus, minus = codes == 1, codes == -1
    np.bitwise_or.at(out, byte_p[plus], bitval[plus])
    np.bitwise_or.at(out, (byte_p + n_off)[minus], bitval[minus])
    if count_invalid:
        return out, int(np.count_nonzero(~(plus | minus | (codes == 0))))
    return out


def unpack_ternary(packed: np.ndarray, N: int, K: int, count_invalid: bool = False):
    """T2-PN-64 bytes -> int8 codes [N, K]. A (P, N) = (1, 1) pair decodes to 0 and
    is counted as invalid."""
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    assert packed.size == ternary_packed_bytes(N, K)
    byte_p, bit, n_off = _t2_byte_and_bit(N, K)
    p = (packed[byte_p] >> bit.astype(np.uint8)) & 1
    m = (packed[byte_p + n_off] >> bit.astype(np.uint8)) & 1
    bad = (p == 1) & (m == 1)
    codes = (p.astype(np.int8) - m.astype(np.int8))
    codes[bad] = 0
    if count_invalid:
        return codes, int(np.count_nonzero(bad))
    return codes


def _mf_byte_and_shift(N: int, K: int):
    """Byte offset of the 2-bit field of every (n, k), its shift within that byte and its
    fragment f (which fixes the field's encoding), straight from the T2-MF64 text."""
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    tn, r = n // 64, n % 64
    tk, c = k // 64, k % 64
    f, u = r // 16, r % 16
    g, j, i = c // 16, (c // 4) % 4, c % 4
    word = 4 * (16 * g + u) + j
    wbit = 8 * i + 2 * f
    byte = (tn * (K // 64) + tk) * 1024 + 4 * word + wbit // 8
    return byte, np.broadcast_to(wbit % 8, byte.shape), np.broadcast_to(f, byte.shape)


def pack_ternary_mf(codes: np.ndarray, count_invalid: bool = False):
    """int8 codes [N, K] -> uint8 T2-MF64 bytes [N*K/4]: field w + 1 (rows 16f + u of a
    tile with f < 3) or w in two's complement (f = 3).

    A code other than -1/0/+1 packs as w = 0 and is counted as invalid.
    Parity: pinned by hand-worked bytes, the round trip, agreement with T2-PN-64 and the
    operand identity in the CPU tests."""
    codes = np.asarray(codes)
    N, K = codes.shape
    assert N % 64 == 0 and K % 64 == 0, "T2-MF64 needs N % 64 == 0 and K % 64 == 0"
    valid = (codes == 1) | (codes == 0) | (codes == -1)
    w = np.where(valid, codes.astype(np.int64), 0)
    byte, shift, f = _mf_byte_and_shift(N, K)
    field = np.where(f < 3, w + 1, w & 3)
    out = np.zeros(ternary_packed_bytes(N, K), dtype=np.uint8)
    np.bitwise_or.at(out, byte.ravel(), (field << shift).astype(np.uint8).ravel())
    if count_invalid:
        return out, int(np.count_nonzero(~valid))
    return out


def unpack_ternary_mf(packed: np.ndarray, N: int, K: int, count_invalid: bool = False):
    """T2-MF64 bytes -> int8 codes [N, K]. An invalid field (3 for f < 3, 2 for f = 3)
    decodes to 0 and is counted."""
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    assert packed.size == ternary_packed_bytes(N, K)
    byte, shift, f = _mf_byte_and_shift(N, K)
    c = ((packed[byte] >> shift.astype(np.uint8)) & 3).astype(np.int64)
    bad = np.where(f < 3, c == 3, c == 2)
    w = np.where(f < 3, c - 1, np.where(c == 3, -1, c))
    codes = np.where(bad, 0, w).astype(np.int8)
    if count_invalid:
        return codes, int(np.count_nonzero(bad))
    return codes


def _s1_byte_and_bit(N: int, K: int):
    n = np.arange(N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    tn, r = n // 64, n % 64
    tk, c = k // 128, k % 128
    f, u = r // 16, r % 16
    s, g, q, e = c // 32, (c // 8) % 4, (c // 2) % 4, c % 2
    word = 4 * (16 * g + u) + f
    wbit = 16 * e + 4 * s + q
    byte = (tn * (K // 128) + tk) * 1024 + 4 * word + wbit // 8
    return byte, np.broadcast_to(wbit % 8, byte.shape)


def pack_sign(W: np.ndarray) -> np.ndarray:
    """Float weights [N, K] -> uint8 S1-128 bytes [N*K/8]; bit set iff W < 0.

    Reading (the pages keep only Sign(W), [onebit] "3. 通过知识蒸馏迁移原模型能力"):
    one bit cannot hold a zero, so +0, -0 and NaN all map to +1 (bit clear).
    Parity: pinned by worked bytes, the round trip and the 4096x4096 storage count."""
    W = np.asarray(W)
    N, K = W.shape
    assert N % 64 == 0 and K % 128 == 0, "S1-128 needs N % 64 == 0 and K % 128 == 0"
    out = np.zeros(sign_packed_bytes(N, K), dtype=np.uint8)
    byte, bit = _s1_byte_and_bit(N, K)
    neg = W < 0
    np.bitwise_or.at(out, byte[neg], (1 << bit[neg]).astype(np.uint8))
    return out


def unpack_sign(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """S1-128 bytes -> int8 signs [N, K] in {-1, +1}."""
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    assert packed.size == sign_packed_bytes(N, K)
    byte, bit = _s1_byte_and_bit(N, K)
    neg = (packed[byte] >> bit.astype(np.uint8)) & 1
    return (1 - 2 * neg.astype(np.int16)).astype(np.int8)


def act_planes(q: np.ndarray) -> np.ndarray:
    """int8 activations [M, K] -> uint32 X8-64 bit planes [M, K/64, 16]."""
    q = np.asarray(q, dtype=np.int8)
    M, K = q.shape
    assert K % 64 == 0
    u = q.view(np.uint8).astype(np.uint32).reshape(M, K // 64, 2, 32)   # [m, t, h, c]
    c = np.arange(32)
    shift = (8 * (c % 4) + c // 4).astype(np.uint32)                     # c = 4j+i -> bit 8i+j
    out = np.zeros((M, K // 64, 16), dtype=np.uint32)
    for b in range(8):
        bits = (u >> np.uint32(b)) & np.uint32(1)                      # [m, t, h, c]
        word = np.bitwise_or.reduce(bits << shift, axis=-1)             # [m, t, h]
        out[:, :, 2 * b] = word[:, :, 0]
        out[:, :, 2 * b + 1] = word[:, :, 1]
    return out
