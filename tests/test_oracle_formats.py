"""Pins for the oracle's packed layouts (CPU only).

The layouts are this library's own; the pins are hand-worked bytes from the
layout text, round trips, word invariants, and the add-only identity that ties
the weight layout to the activation bit planes."""
import numpy as np
import pytest

import oracle
import synth


def _words(packed):
    return np.asarray(packed, dtype=np.uint8).view("<u4")


# ----------------------------------------------------------------------------- T2-PN-64
@pytest.mark.parametrize("n,k,code,byte,value", [
    (0, 0, +1, 0, 0x01),      # P0 of row 0, c = 0 -> bit 0
    (0, 4, +1, 0, 0x02),      # c = 4 = 4*1 + 0 -> bit 1
    (0, 1, -1, 9, 0x01),      # N0 starts at byte 8; c = 1 -> bit 8 -> byte 9 bit 0
    (0, 31, -1, 11, 0x80),    # c = 31 = 4*7 + 3 -> bit 31 of N0 -> byte 11 bit 7
    (1, 33, +1, 21, 0x01),    # row 1 at byte 16; P1 at +4; c = 1 -> byte 21 bit 0
    (63, 63, +1, 16 * 63 + 7, 0x80),   # row 63, P1, c = 31 -> bit 31 -> byte 7 of the row
    (0, 64, +1, 1024, 0x01),  # tile (0, 1)
    (64, 0, -1, 2048 + 8, 0x01),  # tile (1, 0) with K = 128 -> byte 2 * 1024
])
def test_t2_worked_bytes(n, k, code, byte, value):
    codes = np.zeros((128, 128), dtype=np.int8)
    codes[n, k] = code
    packed = oracle.pack_ternary(codes)
    expect = np.zeros_like(packed)
    expect[byte] = value
    assert np.array_equal(packed, expect)


def test_t2_round_trip_and_invariants():
    codes = synth.ternary_codes(synth.matrix_key(0, 99, 0, 0), 192, 320)
    packed = oracle.pack_ternary(codes)
    assert packed.size == 192 * 320 // 4 == oracle.ternary_packed_bytes(192, 320)
    assert np.array_equal(oracle.unpack_ternary(packed, 192, 320), codes)
    w = _words(packed).reshape(-1, 4)                  # [P0, P1, N0, N1] per tile row
    assert not np.any(w[:, 0] & w[:, 2]) and not np.any(w[:, 1] & w[:, 3])
    pop = lambda a: int(sum(bin(int(v)).count("1") for v in a.ravel()))
    assert pop(w[:, :2]) == int(np.count_nonzero(codes == 1))
    assert pop(w[:, 2:]) == int(np.count_nonzero(codes == -1))


def test_t2_all_plus_row():
    codes = np.zeros((64, 64), dtype=np.int8)
    codes[5] = 1
    w = _words(oracle.pack_ternary(codes)).reshape(64, 4)
    assert list(w[5]) == [0xFFFFFFFF, 0xFFFFFFFF, 0, 0]
    assert not np.any(np.delete(w, 5, axis=0))


def test_t2_invalid_codes():
    codes = np.zeros((64, 64), dtype=np.int8)
    codes[0, :3] = [2, -5, 1]
    packed, bad = oracle.pack_ternary(codes, count_invalid=True)
    assert bad == 2
    back = oracle.unpack_ternary(packed, 64, 64)
    assert list(back[0, :3]) == [0, 0, 1]
    # a (P, N) = (1, 1) pair is invalid on unpack and decodes to 0
    packed = packed.copy()
    packed[0] |= 0x01
    packed[8] |= 0x01
    codes2, bad2 = oracle.unpack_ternary(packed, 64, 64, count_invalid=True)
    assert bad2 == 1 and codes2[0, 0] == 0


# ----------------------------------------------------------------------------- T2-MF64
# Hand-worked from the layout text on a 128 x 128 matrix whose other weights make every
# field zero (-1 in rows 16f + u with f < 3, field w + 1 = 0; 0 in rows with f = 3, field
# w = 0): row r = 16f + u, input c = 16g + 4j + i -> word 4(16g + u) + j, byte i of the
# word, shift 2f; the field is w + 1 for f < 3 and w in two's complement for f = 3.
def _mf_background():
    codes = np.full((128, 128), -1, dtype=np.int8)
    codes[(np.arange(128) % 64) >= 48, :] = 0
    return codes


@pytest.mark.parametrize("n,k,code,byte,value", [
    (0, 0, 1, 0, 0x02),          # word 0, byte 0, shift 0, field 2
    (0, 1, 0, 1, 0x01),          # i = 1 -> byte 1, field 1
    (0, 4, 1, 4, 0x02),          # j = 1 -> word 1
    (0, 15, 1, 15, 0x02),        # j = 3, i = 3 -> word 3, byte 3
    (0, 16, 0, 256, 0x01),       # g = 1 -> word 64
    (1, 0, 1, 16, 0x02),         # u = 1 -> word 4
    (16, 0, 0, 0, 0x04),         # f = 1 -> shift 2, field 1
    (32, 0, 1, 0, 0x20),         # f = 2 -> shift 4, field 2
    (48, 0, 1, 0, 0x40),         # f = 3 -> shift 6, field 01 (w = +1)
    (48, 0, -1, 0, 0xC0),        # f = 3, field 11 (w = -1)
    (63, 63, -1, 1023, 0xC0),    # u = 15, g = 3, j = 3, i = 3: word 255, byte 3
    (0, 64, 1, 1024, 0x02),      # second k tile
    (64, 0, 0, 2048, 0x01),      # second row band: tile (1, 0)
    (127, 127, 1, 4095, 0x40),   # tile (1, 1), word 255, byte 3, f = 3
])
def test_mf_worked_bytes(n, k, code, byte, value):
    codes = _mf_background()
    codes[n, k] = code
    packed = oracle.pack_ternary_mf(codes)
    expect = np.zeros_like(packed)
    expect[byte] = value
    assert np.array_equal(packed, expect)


def test_mf_layout_is_a_bijection():
    from oracle.formats import _mf_byte_and_shift
    byte, shift, f = _mf_byte_and_shift(128, 192)
    slots = byte.astype(np.int64) * 8 + shift
    assert np.unique(slots).size == 128 * 192
    assert slots.min() == 0 and byte.max() == 128 * 192 // 4 - 1 and np.all(shift % 2 == 0)
    assert np.array_equal(shift, 2 * f)


def test_mf_round_trip_and_agreement_with_t2():
    codes = synth.ternary_codes(synth.matrix_key(0, 99, 1, 0), 192, 320)
    mf = oracle.pack_ternary_mf(codes)
    assert mf.size == oracle.ternary_packed_bytes(192, 320)
    assert np.array_equal(oracle.unpack_ternary_mf(mf, 192, 320), codes)
    pn = oracle.pack_ternary(codes)
    assert np.array_equal(oracle.unpack_ternary(pn, 192, 320), oracle.unpack_ternary_mf(mf, 192, 320))
    # no field holds an invalid value (3 at shifts 0, 2, 4; 2 at shift 6)
    w = _words(mf)
    for s in range(0, 32, 2):
        fld = (w >> s) & 3
        assert not np.any(fld == (2 if s % 8 == 6 else 3))


def test_mf_operand_extraction():
    """The use the layout is cut for: in record 16g + u of a tile, word j masked with
    0x03030303 << 2f holds, in byte i, 4^f (w + 1) (f < 3) or, as a signed byte, 64 w
    (f = 3), for w of row 16f + u, input 16g + 4j + i."""
    codes = synth.ternary_codes(synth.matrix_key(0, 99, 2, 0), 64, 64)
    w = _words(oracle.pack_ternary_mf(codes)).reshape(64, 4)     # [record, j]
    for g in range(4):
        for u in range(16):
            for f in range(4):
                for j in range(4):
                    d = int(w[16 * g + u, j]) & (0x03030303 << (2 * f))
                    got = [int(np.int8(np.uint8((d >> (8 * i)) & 0xFF))) for i in range(4)]
                    wt = [int(codes[16 * f + u, 16 * g + 4 * j + i]) for i in range(4)]
                    want = [(4 ** f) * (x + 1) for x in wt] if f < 3 else [64 * x for x in wt]
                    assert got == want


def test_mf_operand_dot_identity():
    """Summing q times the masked bytes over a tile row, shifting right by 2f and taking
    away sum q for f < 3 gives sum q w exactly (what the kernels' epilogues do)."""
    rng = np.random.default_rng(5)
    codes = synth.ternary_codes(synth.matrix_key(0, 99, 3, 0), 64, 64)
    q = rng.integers(-127, 128, size=64)
    w = _words(oracle.pack_ternary_mf(codes)).reshape(64, 4)
    for f in range(4):
        for u in range(16):
            s = 0
            for g in range(4):
                for j in range(4):
                    d = int(w[16 * g + u, j]) & (0x03030303 << (2 * f))
                    for i in range(4):
                        s += int(q[16 * g + 4 * j + i]) * int(np.int8(np.uint8((d >> (8 * i)) & 0xFF)))
            assert s % (4 ** f) == 0
            v = (s >> (2 * f)) - (int(q.sum()) if f < 3 else 0)
            assert v == int(np.dot(q, codes[16 * f + u].astype(np.int64)))


def test_mf_invalid_codes():
    codes = np.zeros((64, 64), dtype=np.int8)
    codes[0, :3] = [2, -5, -1]
    codes[48, :3] = [3, 1, -1]
    packed, bad = oracle.pack_ternary_mf(codes, count_invalid=True)
    assert bad == 3
    back = oracle.unpack_ternary_mf(packed, 64, 64)
    assert list(back[0, :3]) == [0, 0, -1] and list(back[48, :3]) == [0, 1, -1]
    packed = packed.copy()
    packed[0] |= 0x03                                  # field 3 at (0, 0): f = 0
    packed[0] = (packed[0] & 0x3F) | 0x80              # field 10 at (48, 0): f = 3
    back, bad2 = oracle.unpack_ternary_mf(packed, 64, 64, count_invalid=True)
    assert bad2 == 2 and back[0, 0] == 0 and back[48, 0] == 0


# ----------------------------------------------------------------------------- S1-128
@pytest.mark.parametrize("n,k,byte,value", [
    (0, 0, 0, 0x01),        # r = 0, c = 0 -> word 0, bit 0
    (0, 1, 2, 0x01),        # e = 1 -> bit 16 -> byte 2 bit 0
    (0, 2, 0, 0x02),        # q = 1 -> bit 1
    (0, 32, 0, 0x10),       # s = 1 -> bit 4
    (0, 8, 256, 0x01),      # g = 1 -> word 64 -> byte 256
    (1, 0, 16, 0x01),       # u = 1 -> word 4 -> byte 16
    (16, 0, 4, 0x01),       # f = 1 -> word 1 -> byte 4
    (0, 127, 771, 0x80),    # c = 96 + 24 + 6 + 1 -> word 192, bit 31 -> byte 771 bit 7
    (63, 127, 1023, 0x80),  # f = 3, u = 15 -> word 255, bit 31
    (0, 128, 1024, 0x01),   # tile (0, 1)
    (64, 0, 2048, 0x01),    # tile (1, 0) of a 128 x 256 matrix
])
def test_s1_worked_bytes(n, k, byte, value):
    W = np.ones((128, 256), dtype=np.float32)
    W[n, k] = -0.25
    packed = oracle.pack_sign(W)
    expect = np.zeros_like(packed)
    expect[byte] = value
    assert np.array_equal(packed, expect)


def test_s1_layout_is_a_bijection():
    """Every (row, input) of a tile gets its own bit: the 64 x 128 one-hot matrices pack to
    64 * 128 distinct single-bit patterns covering all 8192 bits of the tile."""
    byte, bit = oracle.formats._s1_byte_and_bit(64, 128)
    pos = (byte * 8 + bit).ravel()
    assert np.array_equal(np.sort(pos), np.arange(8192))


def test_s1_round_trip_and_zero_reading():
    W = synth.normal_fp32((128, 384), 0, 98, 1)
    W[0, :4] = [0.0, -0.0, np.nan, -np.inf]
    S = oracle.unpack_sign(oracle.pack_sign(W), 128, 384)
    expect = np.where(W < 0, -1, 1)
    assert np.array_equal(S, expect)
    assert list(S[0, :4]) == [1, 1, 1, -1]
    assert oracle.pack_sign(W).size == 128 * 384 // 8


# ----------------------------------------------------------------------------- X8-64 planes
def test_planes_worked_bits():
    q = np.zeros((1, 64), dtype=np.int8)
    q[0, 0] = 1
    q[0, 5] = -128            # 0x80: plane 7 only; c = 5 = 4*1 + 1 -> bit 9
    q[0, 40] = 3              # h = 1, c = 8 = 4*2 + 0 -> bit 2; planes 0 and 1
    X = oracle.act_planes(q)[0, 0]
    expect = np.zeros(16, dtype=np.uint32)
    expect[2 * 0 + 0] |= 1 << 0
    expect[2 * 7 + 0] |= 1 << 9
    expect[2 * 0 + 1] |= 1 << 2
    expect[2 * 1 + 1] |= 1 << 2
    assert np.array_equal(X, expect)


def _popcount32(a):
    a = a.astype(np.uint64)
    c = np.zeros_like(a)
    for b in range(32):
        c += (a >> np.uint64(b)) & np.uint64(1)
    return c.astype(np.int64)


def test_add_only_identity_ties_layouts_together():
    """sum_b c_b * popcount((P & X_b) | (N & ~X_b)) + popcount(N) == sum_k w_k q_k,
    with c_b = 2^b (b < 7) and c_7 = -128: the identity the add-only GEMV evaluates.
    A wrong bit order in either the weight layout or the planes breaks it."""
    M, N, K = 3, 64, 192
    rg = synth.rng(0, 97)
    q = rg.integers(-128, 128, size=(M, K)).astype(np.int8)
    codes = synth.ternary_codes(synth.matrix_key(0, 97, 0, 1), N, K)
    w = _words(oracle.pack_ternary(codes)).reshape(N // 64, K // 64, 64, 4)   # [tn, tk, r, word]
    X = oracle.act_planes(q)                                                  # [m, t, 16]
    cb = [1, 2, 4, 8, 16, 32, 64, -128]
    acc = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for t in range(K // 64):
            P = w[0, t, :, 0:2]
            Nn = w[0, t, :, 2:4]
            for b in range(8):
                xb = X[m, t, 2 * b: 2 * b + 2][None, :]
                sel = (P & xb) | (Nn & ~xb)
                acc[m] += cb[b] * _popcount32(sel).sum(axis=1)
            acc[m] += _popcount32(Nn).sum(axis=1)
    brute = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for n in range(N):
            brute[m, n] = sum(int(codes[n, k]) * int(q[m, k]) for k in range(K))
    assert np.array_equal(acc, brute)
