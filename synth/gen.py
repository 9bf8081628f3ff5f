"""Seeded input generators (PCG64 via numpy), one function per workload.

Every array is drawn on the host from ``numpy.random.default_rng`` seeded with a
``SeedSequence([seed, stream, ...])`` so that any single expert's tensors can be
regenerated without drawing the others. Both the CPU oracle and the HIP path
consume exactly these arrays; each side packs, quantizes and computes on its
own.

Workload shapes (the ROCmFPX block formats and the MoE layer they serve are
described on lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on AMD
Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128 GB"):

* ``fp2_matvec``      FP2 512x256 matvec, one 4-entry codebook, batch 1.
* ``LayerSpec.full``  hidden 4096, 256 routed experts, inter 2048, top-6;
                      gate/up FP2, down FP3.
* ``dense_mix``       FP4 4096x16384 + FP3 4096x2048 with H32 on its input.

Distributions: codes uniform over all 2^bits values; fp16 scales U(0.01, 0.1)
rounded to nearest-even fp16; E8M0 bytes uniform in 120..123; codebooks uniform
integers in [-127, 127]; router weights fp16 N(0, 0.02); tokens fp32 N(0, 1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "rng", "uniform_codes", "fp16_scales", "e8m0_scales", "codebook",
    "MatvecCase", "fp2_matvec", "matvec_case", "LayerSpec", "ExpertTensor",
    "expert_tensor", "router_weights", "tokens", "zipf_bias", "q4_group",
    "dense_mix", "float_matrices", "STREAM",
]

# Stream ids keep the draws of different tensors independent of each other.
STREAM = {
    "gate": 11, "up": 12, "down": 13, "router": 14, "tokens": 15, "q4": 16,
    "matvec": 17, "dense_fp4": 18, "dense_fp3": 19, "dense_x": 20,
    "float_w": 21,
}


def rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), *map(int, stream)]))


def uniform_codes(g: np.random.Generator, shape, bits: int) -> np.ndarray:
    """Codes uniform over 0 .. 2^bits - 1, uint8."""
    return g.integers(0, 1 << bits, size=shape, dtype=np.uint8)


def fp16_scales(g: np.random.Generator, shape, lo=0.01, hi=0.1) -> np.ndarray:
    """U(lo, hi) rounded to fp16 (round-to-nearest-even); returned as raw uint16 bits."""
    return g.uniform(lo, hi, size=shape).astype(np.float16).view(np.uint16)


def e8m0_scales(g: np.random.Generator, shape, lo=120, hi=123) -> np.ndarray:
    """E8M0 exponent bytes uniform in lo..hi inclusive."""
    return g.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def codebook(g: np.random.Generator, n: int) -> np.ndarray:
    return g.integers(-127, 128, size=n, dtype=np.int8)


@dataclasses.dataclass
class MatvecCase:
    fmt: int            # 2, 3 or 4 (ROCmFP2 / FP3 / FP4)
    rows: int
    k: int
    codes: np.ndarray   # uint8 [rows, k]
    scales: np.ndarray  # uint16 fp16 bits [rows, k/32] (FP2/FP3) or uint8 E8M0 (FP4)
    cb: np.ndarray      # int8 [2^fmt]
    x: np.ndarray       # fp32 [ncols, k]
    rot: int = 0


def matvec_case(fmt: int, rows: int, k: int, ncols: int = 1, seed: int = 0,
                rot: int = 0, stream: int = STREAM["matvec"]) -> MatvecCase:
    """One block-quantized weight matrix plus ``ncols`` N(0,1) activation columns.

    Draw order: codes, scales, codebook, x.
    """
    assert k % 32 == 0
    g = rng(seed, stream, fmt, rows, k)
    codes = uniform_codes(g, (rows, k), fmt)
    if fmt == 4:
        scales = e8m0_scales(g, (rows, k // 32))
    else:
        scales = fp16_scales(g, (rows, k // 32))
    cb = codebook(g, 1 << fmt)
    x = g.standard_normal((ncols, k), dtype=np.float32)
    return MatvecCase(fmt, rows, k, codes, scales, cb, x, rot)


def fp2_matvec(seed: int = 0) -> MatvecCase:
    """FP2 512x256 (rows x K), fp16 scales U(0.01, 0.1), one 4-entry codebook, batch 1."""
    return matvec_case(2, 512, 256, 1, seed)


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    hidden: int
    inter: int
    n_experts: int
    topk: int
    fmt_gate: int = 2
    fmt_up: int = 2
    fmt_down: int = 3
    rot_gateup: int = 0
    rot_down: int = 0

    @staticmethod
    def full(**kw) -> "LayerSpec":
        """hidden 4096, 256 routed experts, inter 2048, top-6, gate/up FP2, down FP3."""
        return LayerSpec(4096, 2048, 256, 6, **kw)

    @staticmethod
    def tiny(**kw) -> "LayerSpec":
        """A small layer of the same structure for fast tests."""
        d = dict(hidden=256, inter=256, n_experts=8, topk=2)
        d.update(kw)
        return LayerSpec(**d)

    def shape(self, tensor: str):
        """(rows, K, format) of one expert's tensor."""
        if tensor == "gate":
            return self.inter, self.hidden, self.fmt_gate
        if tensor == "up":
            return self.inter, self.hidden, self.fmt_up
        if tensor == "down":
            return self.hidden, self.inter, self.fmt_down
        raise KeyError(tensor)


@dataclasses.dataclass
class ExpertTensor:
    fmt: int
    codes: np.ndarray   # uint8 [rows, K]
    scales: np.ndarray  # uint16 fp16 bits or uint8 E8M0 [rows, K/32]
    cb: np.ndarray      # int8 [2^fmt]


def expert_tensor(spec: LayerSpec, tensor: str, e: int, seed: int = 0) -> ExpertTensor:
    """Expert ``e``'s tensor (gate / up / down). Draw order: codes, scales, codebook."""
    rows, k, fmt = spec.shape(tensor)
    g = rng(seed, STREAM[tensor], e)
    codes = uniform_codes(g, (rows, k), fmt)
    scales = e8m0_scales(g, (rows, k // 32)) if fmt == 4 else fp16_scales(g, (rows, k // 32))
    cb = codebook(g, 1 << fmt)
    return ExpertTensor(fmt, codes, scales, cb)


def router_weights(spec: LayerSpec, seed: int = 0, sigma: float = 0.02) -> np.ndarray:
    """fp16 N(0, sigma) router matrix [E][hidden], returned as raw uint16 bits."""
    g = rng(seed, STREAM["router"])
    w = g.normal(0.0, sigma, size=(spec.n_experts, spec.hidden))
    return w.astype(np.float16).view(np.uint16)


def tokens(n: int, hidden: int, seed: int = 0, stream: int = 0) -> np.ndarray:
    """fp32 N(0, 1) tokens [n][hidden]."""
    g = rng(seed, STREAM["tokens"], stream)
    return g.standard_normal((n, hidden), dtype=np.float32)


def zipf_bias(n_experts: int, s: float = 1.1) -> np.ndarray:
    """Per-expert logit offset -s*ln(e+1) (fp64): adds a Zipf(s)-shaped skew to the
    expert load when added to the router logits."""
    return np.array([-s * math.log(e + 1.0) for e in range(n_experts)], dtype=np.float64)


def q4_group(hidden: int, seed: int = 0, variant: int = 0, rho: float = 0.98) -> np.ndarray:
    """Four correlated tokens: x0 ~ N(0,1), x_t = rho*x0 + sqrt(1-rho^2)*z_t (t=1..3).

    Correlated tokens share most of their routed experts. ``variant`` selects the
    sub-seed; callers redraw with the next variant until their overlap criterion
    holds.
    """
    g = rng(seed, STREAM["q4"], variant)
    x0 = g.standard_normal(hidden)
    out = [x0]
    c = math.sqrt(1.0 - rho * rho)
    for _ in range(3):
        out.append(rho * x0 + c * g.standard_normal(hidden))
    return np.stack(out).astype(np.float32)


def dense_mix(ncols: int = 1, seed: int = 0):
    """FP4 4096x16384 (E8M0 bytes U{120..123}, 16-entry codebook) and FP3
    4096x2048 (fp16 scales, 8-entry codebook, H32 on its input), with ``ncols``
    N(0,1) columns each."""
    fp4 = matvec_case(4, 4096, 16384, ncols, seed, rot=0, stream=STREAM["dense_fp4"])
    fp3 = matvec_case(3, 4096, 2048, ncols, seed, rot=1, stream=STREAM["dense_fp3"])
    return fp4, fp3


def float_matrices(n: int, rows: int, k: int, seed: int = 0, sigma: float = 0.02,
                   outlier_frac: float = 1e-3) -> np.ndarray:
    """fp32 weights [n, rows, k] to quantize: N(0, sigma) with a fraction of
    outliers drawn N(0, 10 sigma) (heavy-tailed like trained projection weights);
    matrix m is drawn from its own stream, so any one can be regenerated alone."""
    out = np.empty((n, rows, k), dtype=np.float32)
    for m in range(n):
        g = rng(seed, STREAM["float_w"], m, rows, k)
        w = g.standard_normal((rows, k)) * sigma
        mask = g.random((rows, k)) < outlier_frac
        w[mask] *= 10.0
        out[m] = w.astype(np.float32)
    return out
