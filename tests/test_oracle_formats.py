"""Pins for the oracle's block formats (no GPU).

Byte budgets: lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
AMD Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128 GB"
(32-weight blocks; FP2 10 bytes = 2.50 bpw; FP3 3.50 bpw; FP4 4.25 bpw).
Bit positions: hand-worked golden blocks in tests/golden/blocks.json.
FP4 special case: OCP Microscaling (MX) v1.0 FP4 E2M1 element decoding.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blocks.json")


@pytest.mark.parametrize("fmt,bpw", [(2, 2.50), (3, 3.50), (4, 4.25)])
def test_block_bytes_match_page_bpw(fmt, bpw):
    assert formats.block_bytes(fmt) * 8 / 32 == bpw
    assert formats.block_bytes(2) == 10
    # tensor bytes = rows * K/32 * block bytes (2048 x 4096 FP2 = 2,621,440 B)
    assert formats.row_bytes(2, 4096) * 2048 == 2_621_440
    assert formats.row_bytes(3, 2048) * 4096 == 3_670_016


def _rule(rule, j):
    return eval(rule, {}, {"j": j})  # rules are fixed strings from the golden file


def test_golden_blocks():
    blocks = json.load(open(GOLDEN))["blocks"]
    assert len(blocks) >= 9
    for b in blocks:
        fmt = b["fmt"]
        codes = np.array([[_rule(b["rule"], j) for j in range(32)]], dtype=np.uint8)
        sbytes = bytes.fromhex(b["scale"])
        if fmt == 4:
            scales = np.array([[sbytes[0]]], dtype=np.uint8)
        else:
            scales = np.array([[sbytes[0] | (sbytes[1] << 8)]], dtype=np.uint16)
        packed = formats.pack(fmt, codes, scales)
        want = bytes.fromhex(b["bytes"].replace(" ", ""))
        assert packed.tobytes() == want, (b["rule"], packed.tobytes().hex(), want.hex())
        c2, s2 = formats.unpack(fmt, packed, 32)
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_code_bits_are_a_bijection(fmt):
    """Each (weight, code bit) lands on exactly one packed bit, all distinct,
    covering the whole code region; the scale region is untouched."""
    bits = formats.BITS[fmt]
    code_bytes = formats.LO_BYTES[fmt] + formats.HI_BYTES[fmt]
    seen = set()
    for j in range(32):
        for bit in range(bits):
            codes = np.zeros((1, 32), dtype=np.uint8)
            codes[0, j] = 1 << bit
            scales = np.zeros((1, 1), dtype=np.uint8 if fmt == 4 else np.uint16)
            p = formats.pack(fmt, codes, scales)[0]
            on = np.unpackbits(p, bitorder="little").nonzero()[0]
            assert len(on) == 1
            assert on[0] < code_bytes * 8
            seen.add(int(on[0]))
    assert len(seen) == 32 * bits == code_bytes * 8


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_exhaustive_position_value_roundtrip(fmt):
    """Every code value at every position survives pack/unpack, with a random
    background in the other positions."""
    g = np.random.default_rng(1)
    n = 1 << formats.BITS[fmt]
    for j in range(32):
        codes = g.integers(0, n, size=(n, 32), dtype=np.uint8)
        codes[:, j] = np.arange(n)
        scales = (g.integers(0, 255, size=(n, 1), dtype=np.uint8) if fmt == 4
                  else g.integers(0, 0x7C00, size=(n, 1), dtype=np.uint16))
        c2, s2 = formats.unpack(fmt, formats.pack(fmt, codes, scales), 32)
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("fmt,rows,k", [(2, 7, 256), (3, 5, 2048), (4, 3, 512)])
def test_random_roundtrip_and_row_layout(fmt, rows, k):
    g = np.random.default_rng(2)
    codes = g.integers(0, 1 << formats.BITS[fmt], size=(rows, k), dtype=np.uint8)
    nb = k // 32
    scales = (g.integers(0, 255, size=(rows, nb), dtype=np.uint8) if fmt == 4
              else g.integers(0, 0x7C00, size=(rows, nb), dtype=np.uint16))
    p = formats.pack(fmt, codes, scales)
    assert p.shape == (rows, nb * formats.block_bytes(fmt))
    c2, s2 = formats.unpack(fmt, p, k)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # row-planar: a row packed alone equals that row of the whole tensor, and the
    # scales sit at the end of the row in block order
    r = rows // 2
    assert np.array_equal(formats.pack(fmt, codes[r:r + 1], scales[r:r + 1])[0], p[r])
    if fmt == 4:
        assert np.array_equal(p[r, -nb:], scales[r])
    else:
        tail = p[r, -2 * nb:].reshape(nb, 2)
        assert np.array_equal(tail[:, 0] | (tail[:, 1].astype(np.uint16) << 8), scales[r])


def test_fp16_scale_values_match_struct():
    bits = np.array([0x0000, 0x3C00, 0xC000, 0x0001, 0x3555, 0x7BFF, 0x2E66], dtype=np.uint16)
    got = formats.scale_values(2, bits)
    for b, v in zip(bits, got):
        assert v == struct.unpack("<e", struct.pack("<H", int(b)))[0]


def test_e8m0_scale_values():
    e = np.array([0, 1, 120, 126, 127, 128, 254], dtype=np.uint8)
    got = formats.scale_values(4, e)
    for ei, v in zip(e, got):
        assert Fraction(v) == Fraction(2) ** (int(ei) - 127)


def test_invalid_scales_rejected():
    codes = np.zeros((1, 32), dtype=np.uint8)
    with pytest.raises(ValueError):
        formats.pack(4, codes, np.array([[255]], dtype=np.uint8))
    with pytest.raises(ValueError):
        formats.pack(2, codes, np.array([[0x7C00]], dtype=np.uint16))   # +inf
    with pytest.raises(ValueError):
        formats.pack(3, codes, np.array([[0xFE00]], dtype=np.uint16))   # nan
    with pytest.raises(ValueError):
        formats.pack(2, np.full((1, 32), 4, dtype=np.uint8), np.zeros((1, 1), np.uint16))


def _e2m1(code):
    """OCP MX v1.0 FP4 E2M1 element: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0.5 * m)."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m))


def test_fp4_reduces_to_ocp_mxfp4():
    """A ROCmFP4 block whose codebook is 2x the E2M1 value set and whose E8M0
    byte is e-1 dequantizes exactly as an MXFP4 block with shared exponent e."""
    cb = np.array([int(2 * _e2m1(c)) for c in range(16)], dtype=np.int8)
    g = np.random.default_rng(3)
    codes = g.integers(0, 16, size=(4, 64), dtype=np.uint8)
    e = g.integers(100, 150, size=(4, 2), dtype=np.uint8)
    w = formats.dequant(4, codes, e - 1, cb)
    for r in range(4):
        for k in range(64):
            mx = math.ldexp(1.0, int(e[r, k // 32]) - 127) * _e2m1(int(codes[r, k]))
            assert w[r, k] == mx


def test_dequant_matches_elementwise_definition():
    g = np.random.default_rng(4)
    for fmt in (2, 3, 4):
        codes = g.integers(0, 1 << fmt, size=(3, 64), dtype=np.uint8)
        scales = (g.integers(110, 140, size=(3, 2), dtype=np.uint8) if fmt == 4
                  else np.float16(g.uniform(0.01, 0.1, (3, 2))).view(np.uint16))
        cb = g.integers(-128, 128, size=1 << fmt, dtype=np.int8)
        w = formats.dequant(fmt, codes, scales, cb)
        for r in range(3):
            for k in range(64):
                if fmt == 4:
                    s = 2.0 ** (int(scales[r, k // 32]) - 127)
                else:
                    s = struct.unpack("<e", struct.pack("<H", int(scales[r, k // 32])))[0]
                assert w[r, k] == s * int(cb[codes[r, k]])
