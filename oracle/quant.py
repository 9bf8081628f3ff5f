"""int8 per-32-block activation quantization (oracle).

[Strix-284B] (section "ROCmFPX: fitting 284B weights into 128 GB") says the
expanded weights feed integer dot products; the activation side is int8 per
32-weight block with an fp32 absmax scale. Reading used here, every step in
IEEE binary32 with round-to-nearest-even and in this order (no fused
multiply-add):

1. optional H32: v <- FWHT32(v), then v_i <- v_i * c, c = fp32 nearest 1/sqrt(32);
2. amax = max |v_i|;
3. d = amax / 127;
4. if d < 2^-126 (zero or subnormal, where 1/d would overflow) the block is
   stored as d = 0, q = 0; otherwise id = 1 / d;
5. q_i = clamp(rint(v_i * id), -127, 127), rint = round half to even.
"""
from __future__ import annotations

import numpy as np

from .hadamard import fwht32

BLOCK = 32
# binary32 nearest to 1/sqrt(32): the fp64 quotient is within an fp64 ulp of the
# exact value, far from any binary32 rounding boundary (checked exactly by the
# tests with rational arithmetic).
INV_SQRT32 = np.float32(1.0 / np.sqrt(np.float64(32.0)))


def quantize_act(x: np.ndarray, rot: int = 0):
    """x fp32 [..., K] -> (q int8 [..., K], d fp32 [..., K/32])."""
    if rot not in (0, 1):
        raise ValueError("rotation flag must be 0 or 1")
    x = np.asarray(x, dtype=np.float32)
    k = x.shape[-1]
    assert k % BLOCK == 0
    v = x.reshape(*x.shape[:-1], k // BLOCK, BLOCK).copy()
    if rot == 1:
        v = fwht32(v)
        v = (v * INV_SQRT32).astype(np.float32)
    amax = np.max(np.abs(v), axis=-1)                              # exact
    d = (amax / np.float32(127.0)).astype(np.float32)              # IEEE division
    normal = d >= np.float32(2.0 ** -126)
    d = np.where(normal, d, np.float32(0.0)).astype(np.float32)
    inv = np.where(normal, np.float32(1.0) / np.where(normal, d, np.float32(1.0)),
                   np.float32(0.0)).astype(np.float32)
    t = (v * inv[..., None]).astype(np.float32)                    # fp32 product
    q = np.clip(np.rint(t), -127, 127).astype(np.int8)             # half to even
    return q.reshape(x.shape), d


def dequant_act(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """d_b * q_i in fp64 (exact)."""
    q = np.asarray(q, dtype=np.float64)
    k = q.shape[-1]
    return (q.reshape(*q.shape[:-1], k // BLOCK, BLOCK)
            * np.asarray(d, dtype=np.float64)[..., None]).reshape(q.shape)
