"""ROCmFP2 / FP3 / FP4 block formats: pack, unpack, dequantize (oracle).

[Strix-284B] fixes the block (32 weights) and the byte budget: FP2 10 bytes
(2.50 bpw), FP3 3.50 bpw -> 14 bytes, FP4 4.25 bpw -> 17 bytes. The bit
positions below are this repository's reading (the pages print none):

* 2-bit plane, 8 bytes: code of weight j at byte 4*(j>>4) + (j&3), bit 2*((j>>2)&3).
* FP3 = 2-bit plane of the low two code bits + a 4-byte plane of bit 2:
  byte (j&3), bit (j>>2).
* FP4 nibble plane, 16 bytes: code of weight j at byte 4*(j>>3) + (j&3),
  bit 4*((j>>2)&1).
* Scales: fp16 little-endian (FP2, FP3); E8M0 byte e -> 2^(e-127), e = 255
  invalid (FP4).
* Row-planar rows: all code planes (block-major), then FP3 high planes, then
  all scales.

Everything is written with explicit per-weight loops over the 32 positions of a
block (vectorised across rows and blocks only) so that each rule can be read
off directly.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
BLOCK_BYTES = {2: 10, 3: 14, 4: 17}
LO_BYTES = {2: 8, 3: 8, 4: 16}     # code plane bytes per block
HI_BYTES = {2: 0, 3: 4, 4: 0}      # FP3 bit-2 plane bytes per block
SCALE_BYTES = {2: 2, 3: 2, 4: 1}
BITS = {2: 2, 3: 3, 4: 4}


def block_bytes(fmt: int) -> int:
    return BLOCK_BYTES[fmt]


def row_bytes(fmt: int, k: int) -> int:
    assert k % BLOCK == 0
    return (k // BLOCK) * BLOCK_BYTES[fmt]


def _lo_position(fmt: int, j: int):
    """(byte, bit) of weight j's code (FP2/FP4) or its low two bits (FP3)."""
    if fmt in (2, 3):
        return 4 * (j >> 4) + (j & 3), 2 * ((j >> 2) & 3)
    return 4 * (j >> 3) + (j & 3), 4 * ((j >> 2) & 1)


def _hi_position(j: int):
    """(byte, bit) of bit 2 of weight j's FP3 code in the 4-byte high plane."""
    return j & 3, j >> 2


def pack(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes uint8 [rows, K] (< 2^bits), scales [rows, K/32] (uint16 fp16 bits or
    uint8 E8M0) -> packed uint8 [rows, row_bytes]."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, k = codes.shape
    nb = k // BLOCK
    bits = BITS[fmt]
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range")
    c = codes.reshape(rows, nb, BLOCK).astype(np.uint32)
    lo = np.zeros((rows, nb, LO_BYTES[fmt]), dtype=np.uint32)
    hi = np.zeros((rows, nb, HI_BYTES[fmt]), dtype=np.uint32)
    lo_mask = 0xF if fmt == 4 else 0x3
    for j in range(BLOCK):
        byte, bit = _lo_position(fmt, j)
        lo[:, :, byte] |= (c[:, :, j] & lo_mask) << bit
        if fmt == 3:
            hbyte, hbit = _hi_position(j)
            hi[:, :, hbyte] |= ((c[:, :, j] >> 2) & 1) << hbit
    parts = [lo.astype(np.uint8).reshape(rows, -1)]
    if fmt == 3:
        parts.append(hi.astype(np.uint8).reshape(rows, -1))
    if fmt == 4:
        s = np.asarray(scales, dtype=np.uint8).reshape(rows, nb)
        if np.any(s == 255):
            raise ValueError("E8M0 scale 0xFF is invalid")
        parts.append(s)
    else:
        s = np.asarray(scales, dtype=np.uint16).reshape(rows, nb)
        if np.any((s & 0x7C00) == 0x7C00):
            raise ValueError("non-finite fp16 scale")
        # little-endian bytes of each fp16
        sb = np.stack([s & 0xFF, s >> 8], axis=-1).astype(np.uint8).reshape(rows, -1)
        parts.append(sb)
    out = np.concatenate(parts, axis=1)
    assert out.shape[1] == row_bytes(fmt, k)
    return out


def unpack(fmt: int, packed: np.ndarray, k: int):
    """packed uint8 [rows, row_bytes] -> (codes uint8 [rows, K], scales)."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    nb = k // BLOCK
    assert packed.shape[1] == row_bytes(fmt, k)
    off = 0
    lo = packed[:, off:off + nb * LO_BYTES[fmt]].reshape(rows, nb, LO_BYTES[fmt]).astype(np.uint32)
    off += nb * LO_BYTES[fmt]
    hi = None
    if fmt == 3:
        hi = packed[:, off:off + nb * 4].reshape(rows, nb, 4).astype(np.uint32)
        off += nb * 4
    codes = np.zeros((rows, nb, BLOCK), dtype=np.uint32)
    lo_mask = 0xF if fmt == 4 else 0x3
    for j in range(BLOCK):
        byte, bit = _lo_position(fmt, j)
        v = (lo[:, :, byte] >> bit) & lo_mask
        if fmt == 3:
            hbyte, hbit = _hi_position(j)
            v |= ((hi[:, :, hbyte] >> hbit) & 1) << 2
        codes[:, :, j] = v
    if fmt == 4:
        scales = packed[:, off:off + nb].copy()
    else:
        sb = packed[:, off:off + 2 * nb].reshape(rows, nb, 2).astype(np.uint16)
        scales = (sb[:, :, 0] | (sb[:, :, 1] << 8)).astype(np.uint16)
    return codes.reshape(rows, k).astype(np.uint8), scales


def scale_values(fmt: int, scales: np.ndarray) -> np.ndarray:
    """Scale values in fp64: fp16 for FP2/FP3, 2^(e-127) for FP4 E8M0."""
    if fmt == 4:
        e = np.asarray(scales, dtype=np.int64)
        if np.any(e == 255):
            raise ValueError("E8M0 scale 0xFF is invalid")
        return np.ldexp(1.0, e - 127)
    return np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant(fmt: int, codes: np.ndarray, scales: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """w[r, k] = scale[r, k/32] * C[code[r, k]] in fp64 (exact: an fp16 or power
    of two times an int8)."""
    codes = np.asarray(codes)
    rows, k = codes.shape
    cbv = np.asarray(cb, dtype=np.int8).astype(np.float64)
    s = scale_values(fmt, scales)                       # [rows, nb]
    w = cbv[codes.astype(np.int64)].reshape(rows, k // BLOCK, BLOCK)
    return (w * s[:, :, None]).reshape(rows, k)
