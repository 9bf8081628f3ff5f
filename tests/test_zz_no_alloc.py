"""The decode entry point that allocates nothing (qmoe_decode_layer_noalloc),
through the C ABI: its outputs equal those of qmoe_decode_layer (the same
kernels on a caller workspace) bit for bit, on two calls in a row on the
library's one built-in scratch array, the second with a smaller input (fewer
tokens of a smaller layer), so that it runs on what the first call left
behind. A layer whose decode workspace exceeds the array is refused before any
launch."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import bit_block_quantized_rocmfp2_amd as qm  # noqa: E402
from bit_block_quantized_rocmfp2_amd import _binding as B  # noqa: E402
from oracle import moe  # noqa: E402
from synth import gen  # noqa: E402


def with_workspace(dl, x):
    xd = qm.device.to_device(x)
    out = torch.empty_like(xd)
    ws = torch.full((qm.qmoe_workspace_bytes(dl.desc, x.shape[0]),), 0x5A, dtype=torch.uint8, device="cuda")
    qm.qmoe_decode_layer(dl.desc, xd, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def without_allocation(dl, x):
    xd = qm.device.to_device(x)
    out = torch.full_like(xd, float("nan"))
    st = B.LIB.qmoe_decode_layer_noalloc(ctypes.byref(dl.desc), xd.data_ptr(), x.shape[0], out.data_ptr(),
                                         torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.LIB.qmoe_last_error().decode()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_workspace_entry_point():
    big = gen.LayerSpec(hidden=1024, inter=1024, n_experts=32, topk=6, rot_down=1)
    small = gen.LayerSpec.tiny()
    dl_big = qm.device.DeviceLayer(big, seed=3)
    dl_small = qm.device.DeviceLayer(small, seed=4)
    x4 = gen.tokens(4, big.hidden, seed=31)
    x1 = gen.tokens(1, small.hidden, seed=32)
    ref4 = with_workspace(dl_big, x4)
    ref1 = with_workspace(dl_small, x1)
    got4 = without_allocation(dl_big, x4)        # first call: q=4 on the larger layer
    got1 = without_allocation(dl_small, x1)      # second call: q=1 on the smaller layer
    assert np.array_equal(got4, ref4)
    assert np.array_equal(got1, ref1)
    # and the reference itself is right (the oracle, within the layer bar)
    cache = {}

    def get(name, e):
        if (name, e) not in cache:
            t = gen.expert_tensor(small, name, e, 4)
            cache[(name, e)] = (t.fmt, t.codes, t.scales, t.cb)
        return cache[(name, e)]

    L = moe.Layer(small.hidden, small.inter, small.n_experts, small.topk, dl_small.w_router_host, get)
    ref, _, _ = moe.moe_tokens(L, x1)
    assert moe.rel_l2(got1, ref) < 1e-3


def test_noalloc_refuses_oversized_layer():
    # 128 decode slots x inter 32768 int8 = 4 MiB of SwiGLU outputs alone: more
    # than the built-in array; refused on the host (the buffers are never read)
    assert qm.LIB.qmoe_decode_noalloc_max_bytes() == 4 << 20
    spec = gen.LayerSpec(hidden=256, inter=32768, n_experts=1, topk=1)

    def alloc(n, dt=np.uint8):                 # 16-byte aligned host buffer
        a = np.zeros(n + 64, dt)
        off = ((-a.ctypes.data) % 16) // a.itemsize
        return a[off:off + n]

    bufs = {}
    for name in ("gate", "up", "down"):
        rows, k, fmt = spec.shape(name)
        bufs[name] = alloc(qm.qmoe_packed_bytes(fmt, rows, k))
        bufs["cb_" + name] = alloc(1 << fmt).view(np.int8)
    wr = alloc(spec.hidden, np.uint16)
    L = qm.make_layer(spec.hidden, spec.inter, 1, 1, 2, 2, 3, 0, 0, wr, None, bufs["gate"], bufs["up"], bufs["down"],
                      bufs["cb_gate"], bufs["cb_up"], bufs["cb_down"])
    qm.qmoe_layer_check(L)
    x = torch.zeros((1, spec.hidden), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    st = B.LIB.qmoe_decode_layer_noalloc(ctypes.byref(L), x.data_ptr(), 1, out.data_ptr(), None)
    assert st == -6, st
    assert "scratch" in B.LIB.qmoe_last_error().decode()
