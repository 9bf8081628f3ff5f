"""Per-block integer partial sums and block-quantized rows (oracle).

[Strix-284B] (section "ROCmFPX: fitting 284B weights into 128 GB"): codes
index a small codebook and the expanded int8 weights feed integer dot products
against the quantized activations. Definitions used here:

* P[r, b] = sum_{j<32} C[code[r, 32b+j]] * q[32b+j] in exact integers (int64);
* y[r]    = sum_b scale[r, b] * d[b] * P[r, b] in fp64.
"""
from __future__ import annotations

import numpy as np

from .formats import scale_values
from .quant import quantize_act

BLOCK = 32


def block_dots(codes: np.ndarray, cb: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """codes uint8 [rows, K], cb int8 [2^bits], xq int8 [K] -> P int64 [rows, K/32]."""
    codes = np.asarray(codes)
    rows, k = codes.shape
    w = np.asarray(cb, dtype=np.int8).astype(np.int64)[codes.astype(np.int64)]
    xv = np.asarray(xq, dtype=np.int8).astype(np.int64).reshape(k // BLOCK, BLOCK)
    return (w.reshape(rows, k // BLOCK, BLOCK) * xv[None]).sum(axis=2)


def rows_from_blocks(fmt: int, scales: np.ndarray, d: np.ndarray, P: np.ndarray) -> np.ndarray:
    """y[r] = sum_b scale[r,b] * d[b] * P[r,b] in fp64."""
    s = scale_values(fmt, scales)
    return (s * np.asarray(d, dtype=np.float64)[None, :] * P.astype(np.float64)).sum(axis=1)


def matvec(fmt: int, codes, scales, cb, x: np.ndarray, rot: int = 0):
    """Quantize each column of x (fp32 [ncols, K]) and apply the block-quantized
    matrix. Returns (y fp64 [ncols, rows], xq int8 [ncols, K], d fp32 [ncols, K/32])."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float32))
    xq, d = quantize_act(x, rot)
    ys = []
    for c in range(x.shape[0]):
        P = block_dots(codes, cb, xq[c])
        ys.append(rows_from_blocks(fmt, scales, d[c], P))
    return np.stack(ys), xq, d
