"""H32: 32-point Walsh-Hadamard transform (oracle).

[evox3] (introduction; table "The optimization ladder") names "H32 rotations"
on the 3.5-bit expert tensors and a fused / shared H32 input, without a
definition. Reading used here: the unnormalised Sylvester matrix in natural
order, H[i][j] = (-1)^popcount(i & j), applied to each 32-element activation
block in fp32 by the in-place butterfly for h = 1, 2, 4, 8, 16 with
(a, b) -> (a + b, a - b); the 1/sqrt(32) normalisation is a separate fp32
multiply done by the activation quantizer.
"""
from __future__ import annotations

import numpy as np

N = 32


def hadamard_matrix(n: int = N) -> np.ndarray:
    """Integer Sylvester matrix from its entry formula (used only by tests)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pop % 2 == 0, 1, -1).astype(np.int64)


def fwht32(v: np.ndarray) -> np.ndarray:
    """Butterfly FWHT over the last axis (length 32), in the dtype of ``v``
    (fp32 for the quantizer). Returns a new array."""
    v = np.array(v, copy=True)
    assert v.shape[-1] == N
    h = 1
    while h < N:
        for j in range(N):
            if j & h:
                continue
            a = v[..., j].copy()
            b = v[..., j + h].copy()
            v[..., j] = a + b
            v[..., j + h] = a - b
        h *= 2
    return v
