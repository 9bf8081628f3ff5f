"""MoE router: fp64 logits in a fixed summation order, top-k, softmax (oracle).

[0731-Strix] (section "Run with Lucebox Engine") gives 256 experts with six
routed per token; the pages give no router arithmetic beyond dedicated TOP_K /
ARGSORT kernels ([Strix-284B], section "Decode: up to 32 tok/s"). Reading
used here, chosen so that a GPU can reproduce the ids bit for bit:

1. s_b = sequential fp64 sum over i = 0..31 of f64(W[e, 32b+i]) * f64(x[32b+i])
   (products are exact in fp64);
2. pad s to a power of two with +0.0, then the stride-halving tree
   s_j <- s_j + s_{j+n} for n = P/2, ..., 1;
3. logit_e = s_0 + bias_e;
4. the k largest logits, ties to the lower id, returned in ascending id order;
5. g = softmax over the k selected logits (max-subtracted, fp64, sum in
   ascending id order).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def _next_pow2(n: int) -> int:
    p = 1
    while p < n:
        p *= 2
    return p


def logits(w_bits: np.ndarray, x: np.ndarray, bias=None, chunk: int = 256) -> np.ndarray:
    """w_bits uint16 fp16 [E, H], x fp32 [T, H] -> logits fp64 [T, E]."""
    w = np.asarray(w_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    x = np.atleast_2d(np.asarray(x, dtype=np.float32)).astype(np.float64)
    E, H = w.shape
    T = x.shape[0]
    nb = H // BLOCK
    P = _next_pow2(nb)
    # position-major copies: wT[i, e, b] = W[e, 32b+i], xT[i, t, b] = x[t, 32b+i]
    wT = np.ascontiguousarray(w.reshape(E, nb, BLOCK).transpose(2, 0, 1))
    out = np.empty((T, E), dtype=np.float64)
    for t0 in range(0, T, chunk):
        xT = np.ascontiguousarray(x[t0:t0 + chunk].reshape(-1, nb, BLOCK).transpose(2, 0, 1))
        tc = xT.shape[1]
        s = np.zeros((tc, E, P), dtype=np.float64)
        tmp = np.empty((tc, E, nb), dtype=np.float64)
        for i in range(BLOCK):                       # sequential inside a block
            np.multiply(xT[i][:, None, :], wT[i][None, :, :], out=tmp)
            s[:, :, :nb] += tmp
        n = P // 2
        while n >= 1:                                # stride-halving tree
            s[:, :, :n] = s[:, :, :n] + s[:, :, n:2 * n]
            n //= 2
        out[t0:t0 + tc] = s[:, :, 0]
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out


def select(lg: np.ndarray, topk: int):
    """Top-k ids per row (ties -> lower id) in ascending id order, and the
    softmax weights over the selected logits."""
    lg = np.atleast_2d(lg)
    T, E = lg.shape
    assert 1 <= topk <= E
    idx = np.empty((T, topk), dtype=np.int32)
    g = np.empty((T, topk), dtype=np.float64)
    for t in range(T):
        order = np.argsort(-lg[t], kind="stable")     # stable: equal -> lower id first
        sel = np.sort(order[:topk])
        idx[t] = sel
        v = lg[t, sel]
        m = v.max()
        ex = np.exp(v - m)
        tot = 0.0
        for val in ex:                                 # ascending id order
            tot += val
        g[t] = ex / tot
    return idx, g


def route(w_bits, x, bias=None, topk: int = 6):
    """-> (idx int32 [T, k] ascending, g fp64 [T, k], logits fp64 [T, E])."""
    lg = logits(w_bits, x, bias)
    idx, g = select(lg, topk)
    return idx, g, lg
