"""Float -> ROCmFPX weight quantization with one codebook per matrix (oracle).

TEST INFRASTRUCTURE: the slow, plain reference that the HIP quantizer is
checked against; only the tests, the smoke check and the benchmark's CPU
baseline use it.

[0731-Strix] section "How the model fits on AMD Strix Halo": the expert
weights are stored with learned codebooks, one per expert. [Strix-284B] section
"ROCmFPX: fitting 284B weights into 128 GB": 32-weight blocks, each with a small
scale. The pages print no fitting procedure; this repository's reading (block
absmax scale, Lloyd's 1-D k-means on the scale-normalized weights in integer
units of 1/256, nearest-entry codes) is written out below in the order of the
format specification's weight-quantization section (steps Q1..Q6).
"""
from __future__ import annotations

import numpy as np

from . import formats

BLOCK = 32


def block_scales(fmt: int, w: np.ndarray):
    """Q1. w float32 [..., K] -> (stored scale, d float32) per 32-block.

    FP2/FP3 store fp16 bits h = fp16_rne(fl32(amax / 127)), saturated to 65504;
    FP4 stores E8M0 e with 2^(e-127) the least power of two >= fl32(amax / 127),
    clamped to 1..254 (e = 0 only for an all-zero block)."""
    w = np.asarray(w, dtype=np.float32)
    blocks = w.reshape(*w.shape[:-1], w.shape[-1] // BLOCK, BLOCK)
    a = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    t = (a / np.float32(127.0)).astype(np.float32)
    if fmt in (2, 3):
        with np.errstate(over="ignore"):
            h = t.astype(np.float16)                       # round to nearest even
        h = np.where(t >= np.float32(65520.0), np.float16(65504.0), h)
        return h.view(np.uint16), h.astype(np.float32)
    # FP4: t = m * 2^x with m in [0.5, 1); t is a power of two exactly when m = 0.5
    m, x = np.frexp(t.astype(np.float64))
    k = np.where(m == 0.5, x - 1, x)                       # least k with 2^k >= t
    e = np.where(t > 0, np.clip(127 + k, 1, 254), 0).astype(np.int64)
    d = np.ldexp(np.float64(1.0), e - 127).astype(np.float32)   # exact (2^-127 is an fp32 subnormal)
    return e.astype(np.uint8), d


def normalized(w: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Q2. v = clamp(rne(fl32(w / d) * 256), -32767, 32767), 0 where d = 0 (an
    all-zero block, amax = 0, gives v = 0 in every format).
    w float32 [..., K], d float32 [..., K/32] -> int64 [..., K]."""
    w = np.asarray(w, dtype=np.float32)
    blocks = w.reshape(*w.shape[:-1], w.shape[-1] // BLOCK, BLOCK)
    dd = np.asarray(d, dtype=np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (blocks / dd).astype(np.float32)               # IEEE fp32 division
    s = (r * np.float32(256.0)).astype(np.float32)         # exact: a power of two
    v = np.clip(np.rint(np.where(dd == 0, np.float32(0.0), s)), -32767, 32767).astype(np.int64)
    return v.reshape(w.shape)


def initial_centroids(bits: int) -> np.ndarray:
    """Q3 start: the midpoints of 2^bits equal cells over [-127, 127], in units of 1/256."""
    n = 1 << bits
    return np.array([32512 * (2 * i + 1) // n - 32512 for i in range(n)], dtype=np.int64)


def nearest(v: np.ndarray, c: np.ndarray) -> np.ndarray:
    """argmin_i |v - c_i|, ties to the lower i (a later entry must be strictly nearer)."""
    best = np.abs(v - c[0])
    idx = np.zeros(v.shape, dtype=np.int64)
    for i in range(1, len(c)):
        di = np.abs(v - c[i])
        closer = di < best
        idx[closer] = i
        best = np.where(closer, di, best)
    return idx


def lloyd(v: np.ndarray, bits: int, iters: int) -> np.ndarray:
    """Q3. Lloyd's iterations on the integers v of one matrix; returns the centroids."""
    v = np.asarray(v, dtype=np.int64).ravel()
    c = initial_centroids(bits)
    for _ in range(iters):
        a = nearest(v, c)
        new = c.copy()
        for i in range(len(c)):
            members = v[a == i]
            n_i = np.int64(members.size)
            if n_i > 0:
                s_i = np.int64(members.sum(dtype=np.int64))
                new[i] = (2 * s_i + n_i) // (2 * n_i)      # floor division: mean rounded half up
        c = new
    return c


def codebook(c: np.ndarray) -> np.ndarray:
    """Q4. C_i = clamp(floor((c_i + 128) / 256), -127, 127) as int8."""
    return np.clip((np.asarray(c, dtype=np.int64) + 128) // 256, -127, 127).astype(np.int8)


def quantize(fmt: int, w: np.ndarray, iters: int):
    """Q1..Q6 for n matrices w float32 [n, rows, K].

    Returns (packed uint8 [n, rows, row_bytes], codebooks int8 [n, 2^bits],
    codes uint8 [n, rows, K], stored scales [n, rows, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, rows, k = w.shape
    bits = formats.BITS[fmt]
    packed = np.zeros((n, rows, formats.row_bytes(fmt, k)), dtype=np.uint8)
    cbs = np.zeros((n, 1 << bits), dtype=np.int8)
    codes = np.zeros((n, rows, k), dtype=np.uint8)
    scales = None
    for m in range(n):
        sc, d = block_scales(fmt, w[m])
        v = normalized(w[m], d)
        C = codebook(lloyd(v, bits, iters))
        cm = nearest(v.ravel(), 256 * C.astype(np.int64)).reshape(rows, k).astype(np.uint8)
        packed[m] = formats.pack(fmt, cm, sc)
        cbs[m] = C
        codes[m] = cm
        if scales is None:
            scales = np.zeros((n,) + sc.shape, dtype=sc.dtype)
        scales[m] = sc
    return packed, cbs, codes, scales


def dequantize(fmt: int, packed: np.ndarray, cb: np.ndarray, k: int) -> np.ndarray:
    """d * C[code] of one packed matrix [rows, row_bytes], in fp64."""
    codes, sc = formats.unpack(fmt, packed, k)
    return formats.dequant(fmt, codes, sc, cb)
