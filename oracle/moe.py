"""Top-k SwiGLU MoE layer over block-quantized experts (oracle).

[Strix-284B] (section "ROCmFPX: fitting 284B weights into 128 GB") and
[0731-Strix] (section "How the model fits on AMD Strix Halo"): routed-expert
gate and up matrices in the 2.5-bit format (FP2), down projections in the
3.5-bit format (FP3), each expert with its own codebooks. [evox3] (table "The
optimization ladder"): the input rotation is shared, i.e. applied once per
activation block and reused by every expert; prefill batches all tokens of a
layer. Definitions used here, per token:

  x^  = Act(x, rot_gateup)                      (once, shared by all experts)
  gt  = Row(W_gate[e], x^),  ut = Row(W_up[e], x^)
  a   = fl32( gt / (1 + exp(-gt)) * ut )        (SwiGLU, fp64 then fp32)
  h^  = Act(a, rot_down)
  y_e = Row(W_down[e], h^)
  out = sum over the selected e in ascending id of g_e * y_e   (fp64)

``q`` decode columns and prefill tokens are independent tokens; grouping tokens
by expert (``moe_grouped``) is a re-association of the same sums, evaluated
with fp64 BLAS on exactly dequantized operands (every product is exact in fp64;
only the fp64 summation order differs from the per-block form).

An expert tensor is obtained from ``get(name, e) -> (fmt, codes, scales, cb)``
with name in {"gate", "up", "down"}.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np

from .dots import block_dots, rows_from_blocks
from .formats import dequant
from .quant import dequant_act, quantize_act
from .router import route

Getter = Callable[[str, int], tuple]


@dataclasses.dataclass
class Layer:
    hidden: int
    inter: int
    n_experts: int
    topk: int
    w_router: np.ndarray            # uint16 fp16 bits [E, hidden]
    get: Getter
    bias: Optional[np.ndarray] = None
    rot_gateup: int = 0
    rot_down: int = 0


def swiglu(gt: np.ndarray, ut: np.ndarray) -> np.ndarray:
    """fl32(g / (1 + exp(-g)) * u) from fp64 g, u."""
    gt = np.asarray(gt, dtype=np.float64)
    with np.errstate(over="ignore"):
        a = gt / (1.0 + np.exp(-gt)) * np.asarray(ut, dtype=np.float64)
    return a.astype(np.float32)


def _rows(get: Getter, name: str, e: int, xq: np.ndarray, dx: np.ndarray) -> np.ndarray:
    fmt, codes, scales, cb = get(name, e)
    return rows_from_blocks(fmt, scales, dx, block_dots(codes, cb, xq))


def expert_ffn(L: Layer, e: int, xq: np.ndarray, dx: np.ndarray):
    """One expert on one quantized token. Returns (y fp64 [hidden], a fp32,
    hq int8, dh fp32)."""
    gt = _rows(L.get, "gate", e, xq, dx)
    ut = _rows(L.get, "up", e, xq, dx)
    a = swiglu(gt, ut)
    hq, dh = quantize_act(a, L.rot_down)
    y = _rows(L.get, "down", e, hq, dh)
    return y, a, hq, dh


def moe_tokens(L: Layer, x: np.ndarray):
    """Per-token definition. x fp32 [T, hidden] -> (out fp64 [T, hidden], idx, g)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float32))
    idx, g, _ = route(L.w_router, x, L.bias, L.topk)
    xq, dx = quantize_act(x, L.rot_gateup)
    out = np.zeros((x.shape[0], L.hidden), dtype=np.float64)
    for t in range(x.shape[0]):
        for s in range(L.topk):                       # idx is ascending
            y, _, _, _ = expert_ffn(L, int(idx[t, s]), xq[t], dx[t])
            out[t] += g[t, s] * y
    return out, idx, g


def moe_grouped(L: Layer, x: np.ndarray, routing=None):
    """Same result as ``moe_tokens`` (up to fp64 summation order), computed per
    expert over all of its tokens with fp64 GEMMs of exactly dequantized
    operands. x fp32 [T, hidden] -> (out fp64 [T, hidden], idx, g)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float32))
    T = x.shape[0]
    if routing is None:
        idx, g, _ = route(L.w_router, x, L.bias, L.topk)
    else:
        idx, g = routing
    xq, dx = quantize_act(x, L.rot_gateup)
    out = np.zeros((T, L.hidden), dtype=np.float64)
    for e in range(L.n_experts):                     # ascending id
        tok, slot = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        xd = dequant_act(xq[tok], dx[tok])          # [n_e, hidden]
        fg, cg, sg, bg = L.get("gate", e)
        fu, cu, su, bu = L.get("up", e)
        gt = xd @ dequant(fg, cg, sg, bg).T          # [n_e, inter]
        ut = xd @ dequant(fu, cu, su, bu).T
        a = swiglu(gt, ut)
        hq, dh = quantize_act(a, L.rot_down)
        fd, cd, sd, bd = L.get("down", e)
        y = dequant_act(hq, dh) @ dequant(fd, cd, sd, bd).T   # [n_e, hidden]
        out[tok] += g[tok, slot][:, None] * y
    return out, idx, g


def rel_l2(y: np.ndarray, ref: np.ndarray) -> float:
    """||y - ref||_2 / ||ref||_2 over the whole array, in fp64."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    return float(num / den) if den > 0 else float(num)
