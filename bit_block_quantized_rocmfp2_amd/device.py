"""Device-resident layers and matrices built from seeded synthetic inputs.

Packing goes through the library's host packer (``qmoe_pack``); torch provides
device memory only. The expert tensors of a layer are laid out expert-major,
each expert's rows back to back (row-planar rows), exactly as the C ABI expects.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

from . import _binding as B


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray, device="cuda"):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def pack_experts(spec, name: str, seed: int = 0, device="cuda", workers: int = 0):
    """One projection ("gate", "up" or "down") of every expert of a layer, packed
    in the spec's format and copied to the GPU: (packed bytes, codebooks)."""
    from synth import gen
    torch = _torch()
    E = spec.n_experts
    rows, k, fmt = spec.shape(name)
    row_bytes = B.qmoe_packed_bytes(fmt, 1, k)
    host = np.empty((E, rows * row_bytes), dtype=np.uint8)
    cb = np.empty((E, 1 << fmt), dtype=np.int8)

    def work(e):
        t = gen.expert_tensor(spec, name, e, seed)
        host[e] = B.qmoe_pack(fmt, t.codes, t.scales).reshape(-1)
        cb[e] = t.cb

    nw = workers or min(16, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(nw) as ex:
        list(ex.map(work, range(E)))
    packed = torch.from_numpy(host.reshape(-1)).to(device)
    del host
    return packed, torch.from_numpy(cb.reshape(-1)).to(device)


class DeviceLayer:
    """All experts of one MoE layer packed and copied to the GPU."""

    def __init__(self, spec, seed: int = 0, bias=None, device="cuda", workers: int = 0):
        from synth import gen
        torch = _torch()
        self.spec = spec
        self.seed = seed
        tensors = {}
        cbs = {}
        for name in ("gate", "up", "down"):
            tensors[name], cbs[name] = pack_experts(spec, name, seed, device, workers)
        self.gate, self.up, self.down = tensors["gate"], tensors["up"], tensors["down"]
        self.cb_gate, self.cb_up, self.cb_down = cbs["gate"], cbs["up"], cbs["down"]
        self.w_router_host = gen.router_weights(spec, seed)
        self.w_router = to_device(self.w_router_host, device)
        self.bias_host = None if bias is None else np.asarray(bias, dtype=np.float64)
        self.bias = None if bias is None else torch.from_numpy(self.bias_host).to(device)
        self.desc = B.make_layer(spec.hidden, spec.inter, spec.n_experts, spec.topk, spec.fmt_gate, spec.fmt_up,
                                 spec.fmt_down, spec.rot_gateup, spec.rot_down, self.w_router, self.bias,
                                 self.gate, self.up, self.down, self.cb_gate, self.cb_up, self.cb_down)
        B.qmoe_layer_check(self.desc)

    def packed_bytes_per_expert(self) -> int:
        s = self.spec
        return (B.qmoe_packed_bytes(s.fmt_gate, s.inter, s.hidden) + B.qmoe_packed_bytes(s.fmt_up, s.inter, s.hidden)
                + B.qmoe_packed_bytes(s.fmt_down, s.hidden, s.inter))

    def workspace(self, max_tokens: int, device="cuda"):
        torch = _torch()
        n = B.qmoe_workspace_bytes(self.desc, max_tokens)
        return torch.zeros(n, dtype=torch.uint8, device=device)


class DeviceMatrix:
    """One packed block-quantized matrix (plus its codebook) on the GPU."""

    def __init__(self, case, device="cuda"):
        torch = _torch()
        self.case = case
        self.fmt, self.rows, self.k = case.fmt, case.rows, case.k
        self.w = torch.from_numpy(B.qmoe_pack(case.fmt, case.codes, case.scales).reshape(-1)).to(device)
        self.cb = torch.from_numpy(np.ascontiguousarray(case.cb)).to(device)

    def workspace(self, ncols: int, device="cuda"):
        torch = _torch()
        return torch.zeros(B.qmoe_matvec_workspace_bytes(self.k, ncols), dtype=torch.uint8, device=device)
