"""Pins for the oracle's H32 transform and int8 activation quantizer (no GPU).

H32: the Sylvester Walsh-Hadamard matrix, H[i][j] = (-1)^popcount(i&j)
(soothill.io, "DeepSeek V4 Flash 0731 on evox3", introduction and table "The
optimization ladder", name H32 rotations but give no formula; the identities
below are properties of the textbook matrix). Quantizer: hand-worked blocks,
the rounding bound and exact rational checks of the fp32 steps.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import hadamard, quant


def f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def test_hadamard_orthogonal():
    H = hadamard.hadamard_matrix(32)
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=np.int64))
    assert np.array_equal(H, H.T)


def test_fwht_equals_matrix_product_on_integers():
    H = hadamard.hadamard_matrix(32)
    g = np.random.default_rng(0)
    v = g.integers(-1000, 1000, size=(50, 32))
    got = hadamard.fwht32(v.astype(np.float32))   # small integers: exact in fp32
    assert np.array_equal(got.astype(np.int64), v @ H.T)


def test_fwht_involution_and_unit_vectors():
    g = np.random.default_rng(1)
    v = g.integers(-100, 100, size=(10, 32)).astype(np.float32)
    assert np.array_equal(hadamard.fwht32(hadamard.fwht32(v)), 32 * v)
    e0 = np.zeros(32, np.float32)
    e0[0] = 1
    assert np.array_equal(hadamard.fwht32(e0), np.ones(32, np.float32))
    one = np.ones(32, np.float32)
    assert np.array_equal(hadamard.fwht32(one), 32 * e0)


def test_fwht_butterfly_order_in_fp32():
    """With a large and a small value the fp32 result depends on the order of the
    additions; this vector's expected output was worked by hand from the
    butterfly h = 1, 2, 4, 8, 16."""
    v = np.zeros(32, np.float32)
    v[0] = 2.0 ** 24
    v[1] = 1.0
    v[2] = 1.0
    # h=1: (v0,v1) -> (2^24+1 -> 2^24 (tie to even), 2^24-1); (v2,v3) -> (1, 1)
    # h=2: v0 = 2^24 + 1 -> 2^24; v2 = 2^24 - 1; v1 = (2^24-1) + 1 = 2^24; v3 = 2^24-1-1
    # h>=4: partners are zero, values copy to both halves
    out = hadamard.fwht32(v)
    exp4 = np.array([2.0 ** 24, 2.0 ** 24, 2.0 ** 24 - 1, 2.0 ** 24 - 2], np.float32)
    assert np.array_equal(out[:4], exp4)
    assert np.array_equal(out.reshape(8, 4), np.tile(exp4, (8, 1)))


def test_inv_sqrt32_is_nearest_binary32():
    c = quant.INV_SQRT32
    assert f32_bits(c) == 0x3E3504F3
    # exact check: 1/32 lies between (c - u/2)^2 and (c + u/2)^2, u = ulp(c)
    cf = Fraction(float(c))
    u = Fraction(2) ** (-26)            # c in [2^-3, 2^-2): ulp = 2^-3 * 2^-23
    assert (cf - u / 2) ** 2 < Fraction(1, 32) < (cf + u / 2) ** 2


def test_hand_worked_blocks():
    v = np.zeros(32, np.float32)
    v[:6] = [127.0, -63.5, 0.25, 0.5, 1.5, 2.5]
    q, d = quant.quantize_act(v)
    assert d[0] == 1.0
    assert list(q[:6]) == [127, -64, 0, 0, 2, 2]          # half to even
    v = np.zeros(32, np.float32)
    v[:5] = [254.0, 3.0, 5.0, 1.0, -1.0]
    q, d = quant.quantize_act(v)
    assert d[0] == 2.0 and list(q[:5]) == [127, 2, 2, 0, 0]
    q, d = quant.quantize_act(np.zeros(64, np.float32))
    assert np.all(d == 0) and np.all(q == 0)


def test_underflowing_block_is_zero():
    """A block whose scale amax/127 is zero or subnormal is stored as zero
    (1/d would overflow); a block whose scale is exactly 2^-126 is kept."""
    v = np.zeros(64, np.float32)
    v[:32] = np.float32(1e-38) * (np.arange(32) - 16)
    v[32] = np.float32(127 * 2.0 ** -126)
    v[33] = np.float32(-0.5 * 127 * 2.0 ** -126)
    q, d = quant.quantize_act(v)
    assert d[0] == 0 and np.all(q[:32] == 0)
    assert d[1] == np.float32(2.0 ** -126)
    assert q[32] == 127 and q[33] == -64                   # -63.5 -> -64 (half to even)


def test_scale_steps_exact_rational():
    """d and 1/d are the correctly rounded binary32 values, checked with exact
    rationals on the binary32 grid around them."""
    g = np.random.default_rng(2)
    x = (g.standard_normal(32 * 200) * g.uniform(0.01, 100, 32 * 200)).astype(np.float32)
    q, d = quant.quantize_act(x)
    amax = np.abs(x.reshape(-1, 32)).max(axis=1)
    for a, dd in zip(amax, d):
        exact = Fraction(float(a)) / 127
        lo = Fraction(float(np.nextafter(dd, np.float32(0))))
        hi = Fraction(float(np.nextafter(dd, np.float32(np.inf))))
        df = Fraction(float(dd))
        assert abs(exact - df) <= abs(exact - lo) and abs(exact - df) <= abs(exact - hi)


def test_rounding_bound_and_extremes():
    g = np.random.default_rng(3)
    x = g.standard_normal(32 * 500).astype(np.float32)
    q, d = quant.quantize_act(x)
    xb = x.reshape(-1, 32).astype(np.float64)
    qb = q.reshape(-1, 32).astype(np.float64)
    err = np.abs(xb - qb * d[:, None])
    assert np.all(err <= d[:, None] * (0.5 + 1e-6))
    am = np.argmax(np.abs(xb), axis=1)
    assert np.all(np.abs(qb[np.arange(len(am)), am]) == 127)


def test_rotation_then_scale_order():
    """rot=1 equals rot=0 applied to fl32(fl32(H v) * c), for integer v (H v exact)."""
    H = hadamard.hadamard_matrix(32)
    g = np.random.default_rng(4)
    v = g.integers(-50, 50, size=(20, 32))
    q1, d1 = quant.quantize_act(v.astype(np.float32).ravel(), rot=1)
    hv = (v @ H.T).astype(np.float32) * quant.INV_SQRT32
    q0, d0 = quant.quantize_act(hv.astype(np.float32).ravel(), rot=0)
    assert np.array_equal(q1, q0) and np.array_equal(d1, d0)
    # ones -> 32 e0 -> only element 0 nonzero
    q, d = quant.quantize_act(np.ones(32, np.float32), rot=1)
    assert q[0] == 127 and np.all(q[1:] == 0)
    assert d[0] == np.float32(np.float32(32.0) * quant.INV_SQRT32) / np.float32(127)


def test_rot_flag_validated():
    with pytest.raises(ValueError):
        quant.quantize_act(np.zeros(32, np.float32), rot=2)
