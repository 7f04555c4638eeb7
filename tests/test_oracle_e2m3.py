"""Pins of the oracle's FP6 E2M3 storage of int4-grid codes.

The encoding is the FP6 E2M3 element of the OCP Microscaling Formats (MX)
v1.0 specification (1 sign, 2 exponent bits with bias 1, 3 mantissa bits, no
infinity or NaN); the pins are the values that specification lists for it,
a brute-force bit packing built with Python integers, and closed forms.
"""

import numpy as np
import pytest

import oracle


def test_e2m3_characteristic_values():
    # the specification's table for E2M3: max normal 7.5, min normal 1.0,
    # max subnormal 0.875, min subnormal 0.125, signed zero
    assert oracle.e2m3_value(0b011111) == 7.5
    assert oracle.e2m3_value(0b001000) == 1.0
    assert oracle.e2m3_value(0b000111) == 0.875
    assert oracle.e2m3_value(0b000001) == 0.125
    assert oracle.e2m3_value(0b000000) == 0.0
    v = oracle.e2m3_value(0b100000)
    assert v == 0.0 and np.signbit(v)
    assert oracle.e2m3_value(0b111111) == -7.5


def test_e2m3_value_order_and_sign():
    pos = [oracle.e2m3_value(c) for c in range(32)]
    assert all(b > a for a, b in zip(pos, pos[1:])), "positive codes increase with the code"
    for c in range(32):
        assert oracle.e2m3_value(c | 0x20) == -pos[c]
    # spacing: 1/8 up to 2, 1/4 up to 4, 1/2 up to 7.5
    assert np.allclose(np.diff(pos[:16]), 0.125)
    assert np.allclose(np.diff(pos[16:24]), 0.25)
    assert np.allclose(np.diff(pos[24:32]), 0.5)


def test_e2m3_int_grid_codes():
    for v in range(-7, 8):
        c = oracle.e2m3_code_of_int(v)
        assert oracle.e2m3_value(c) == v
        if v:
            assert oracle.e2m3_code_of_int(-v) == c ^ 0x20
    # worked by hand: 3 = 2 * 1.5 (exponent field 2, mantissa 4), 5 = 4 * 1.25, 7 = 4 * 1.75
    assert oracle.e2m3_code_of_int(3) == 0b010100
    assert oracle.e2m3_code_of_int(5) == 0b011010
    assert oracle.e2m3_code_of_int(7) == 0b011110
    assert oracle.e2m3_code_of_int(-1) == 0b101000
    with pytest.raises(ValueError):
        oracle.e2m3_code_of_int(-8)


def test_pack_e2m3_byte_layout():
    # code j at bits 6j .. 6j+5, little-endian
    assert oracle.pack_e2m3(np.array([1, 0, 0, 0])).tolist() == [0x08, 0x00, 0x00]
    assert oracle.pack_e2m3(np.array([0, 1, 0, 0])).tolist() == [0x00, 0x02, 0x00]
    assert oracle.pack_e2m3(np.array([0, 0, 0, -1])).tolist() == [0x00, 0x00, 0xA0]
    assert oracle.pack_e2m3(np.array([0, 0, 7, 0])).tolist() == [0x00, 0xE0, 0x01]


def test_pack_e2m3_brute_force():
    rng = np.random.default_rng(11)
    for k in (4, 8, 32, 128, 260):
        q = rng.integers(-7, 8, size=(5, k))
        got = oracle.pack_e2m3(q)
        assert got.shape == (5, k * 3 // 4) and got.dtype == np.uint8
        for r in range(5):
            word = 0
            for j in range(k):
                word |= oracle.e2m3_code_of_int(int(q[r, j])) << (6 * j)
            assert bytes(got[r]) == word.to_bytes(k * 3 // 4, "little")
        assert np.array_equal(oracle.unpack_e2m3(got), q)


def test_pack_e2m3_rejects():
    with pytest.raises(ValueError):
        oracle.pack_e2m3(np.zeros(6, dtype=np.int64))
    with pytest.raises(ValueError):
        oracle.pack_e2m3(np.full(4, -8))


def test_e2m3_fp32_dot_product_exact():
    # the largest |sum| the GEMM meets (k < 2^17, all codes +-7) stays below
    # 2^24, so a float32 running sum of E2M3 products is the integer sum
    k = 131072 - 128
    a = oracle.unpack_e2m3(oracle.pack_e2m3(np.full(k, 7))).astype(np.float32)
    b = oracle.unpack_e2m3(oracle.pack_e2m3(np.full(k, -7))).astype(np.float32)
    acc = np.float32(0)
    for chunk in range(0, k, 4096):
        acc = np.float32(acc + np.sum(a[chunk:chunk + 4096] * b[chunk:chunk + 4096], dtype=np.float32))
    assert int(acc) == -49 * k
    assert abs(49 * k) < 2 ** 24
