"""Host-side tests of the C ABI (no GPU, no kernel launches).

* the shared library loads and exports every function declared in include/qmoe.h;
* qmoe_pack is byte-identical to the oracle's packer (they share no code) and
  reproduces the hand-worked golden blocks;
* every argument error is reported on the host before any launch, with the
  codebook classes of lucebox.com "Lucebox × Geometric: DeepSeek V4 Flash 0731
  reaches 32.7 tok/s on AMD Strix Halo", section "Lucebox Engine integration
  with Geometric" (missing, truncated, mismatched).
"""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import bit_block_quantized_rocmfp2_amd as qm
from bit_block_quantized_rocmfp2_amd import _binding as B
from oracle import formats
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 16
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(qmoe_[a-z_]+)\b", out))
    for n in names:
        assert n in exported, n
        assert hasattr(B.LIB, n)
    assert set(B.EXPORTED) == set(names)


def test_prefill_small_default_matches_header():
    hdr = open(HEADER).read()
    m = re.search(r"#define QMOE_PREFILL_SMALL_DEFAULT (\d+)", hdr)
    assert m and int(m.group(1)) == qm.PREFILL_SMALL_DEFAULT


def test_block_and_packed_bytes():
    assert [qm.qmoe_block_bytes(f) for f in (2, 3, 4)] == [10, 14, 17]
    assert qm.qmoe_block_bytes(5) == 0
    assert qm.qmoe_packed_bytes(2, 2048, 4096) == 2_621_440
    assert qm.qmoe_packed_bytes(3, 4096, 2048) == 3_670_016
    assert qm.qmoe_packed_bytes(4, 4096, 16384) == 35_651_584
    assert qm.qmoe_packed_bytes(2, 4, 33) == 0


@pytest.mark.parametrize("fmt,rows,k", [(2, 9, 256), (3, 5, 512), (4, 3, 1024), (2, 1, 32), (3, 2, 96)])
def test_pack_byte_identical_to_oracle(fmt, rows, k):
    c = gen.matvec_case(fmt, rows, k, seed=11)
    a = qm.qmoe_pack(fmt, c.codes, c.scales)
    b = formats.pack(fmt, c.codes, c.scales)
    assert a.tobytes() == b.tobytes()
    codes, scales = qm.qmoe_unpack(fmt, a, rows, k)
    assert np.array_equal(codes, c.codes) and np.array_equal(scales, c.scales)


def test_pack_golden_blocks():
    blocks = json.load(open(os.path.join(ROOT, "tests", "golden", "blocks.json")))["blocks"]
    for b in blocks:
        codes = np.array([[eval(b["rule"], {}, {"j": j}) for j in range(32)]], dtype=np.uint8)
        sb = bytes.fromhex(b["scale"])
        scales = (np.array([[sb[0]]], np.uint8) if b["fmt"] == 4
                  else np.array([[sb[0] | (sb[1] << 8)]], np.uint16))
        got = qm.qmoe_pack(b["fmt"], codes, scales).tobytes()
        assert got == bytes.fromhex(b["bytes"].replace(" ", "")), b["rule"]


def test_pack_errors():
    z = np.zeros((1, 32), np.uint8)
    with pytest.raises(qm.QmoeError) as e:
        qm.qmoe_pack(2, np.full((1, 32), 4, np.uint8), np.zeros((1, 1), np.uint16))
    assert e.value.status == -1
    with pytest.raises(qm.QmoeError) as e:
        qm.qmoe_pack(2, z, np.array([[0x7C00]], np.uint16))
    assert e.value.status == -5
    with pytest.raises(qm.QmoeError) as e:
        qm.qmoe_pack(4, z, np.array([[0xFF]], np.uint8))
    assert e.value.status == -5
    out = np.zeros(20, np.uint8)
    st = B.LIB.qmoe_pack(2, 1, 33, z.ctypes.data, z.ctypes.data, out.ctypes.data, out.nbytes)
    assert st == -2
    st = B.LIB.qmoe_pack(7, 1, 32, z.ctypes.data, z.ctypes.data, out.ctypes.data, out.nbytes)
    assert st == -3
    st = B.LIB.qmoe_pack(2, 1, 32, z.ctypes.data, z.ctypes.data, out.ctypes.data, 9)
    assert st == -8
    assert "out_bytes" in B.LIB.qmoe_last_error().decode()


# --------------------------------------------------------------- layer descriptor checks

def host_layer(spec=None, **over):
    """Descriptor over host numpy buffers (never dereferenced by the check)."""
    spec = spec or gen.LayerSpec.tiny()
    E = spec.n_experts
    bufs = {}

    def alloc(n, dt=np.uint8):
        a = np.zeros(n + 64, dt)
        off = (-a.ctypes.data) % 16
        return a[off:off + n]

    for name in ("gate", "up", "down"):
        rows, k, fmt = spec.shape(name)
        bufs[name] = alloc(E * qm.qmoe_packed_bytes(fmt, rows, k))
        bufs["cb_" + name] = alloc(E << fmt).view(np.int8)
    bufs["w_router"] = alloc(E * spec.hidden * 2).view(np.uint16)
    bufs.update(over)
    d = dict(hidden=spec.hidden, inter=spec.inter, n_experts=E, topk=spec.topk, fmt_gate=spec.fmt_gate,
             fmt_up=spec.fmt_up, fmt_down=spec.fmt_down, rot_gateup=spec.rot_gateup, rot_down=spec.rot_down)
    for k in list(d):
        if k in over:
            d[k] = over[k]
    L = qm.make_layer(d["hidden"], d["inter"], d["n_experts"], d["topk"], d["fmt_gate"], d["fmt_up"], d["fmt_down"],
                      d["rot_gateup"], d["rot_down"], bufs["w_router"], None, bufs["gate"], bufs["up"],
                      bufs["down"], bufs["cb_gate"], bufs["cb_up"], bufs["cb_down"])
    return L, bufs


def status_of(L):
    return B.LIB.qmoe_layer_check(ctypes.byref(L))


def test_layer_check_ok_and_workspace():
    L, _ = host_layer()
    assert status_of(L) == 0
    lay = qm.qmoe_workspace_layout(L, 4)
    offs = [lay[k] for k in ("xq", "dx", "idx", "gw", "logits", "plan", "hq", "dh", "group", "ypair")]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay["total"] == qm.qmoe_workspace_bytes(L, 4) > lay["ypair"]
    full = gen.LayerSpec.full()
    Lf, _ = host_layer(full)
    assert qm.qmoe_workspace_bytes(Lf, 8192) > 8192 * 6 * 4096 * 4


def test_layer_check_codebook_classes():
    spec = gen.LayerSpec.tiny()
    L, b = host_layer()
    L.cb_down = None
    assert status_of(L) == -4 and "missing" in B.LIB.qmoe_last_error().decode()
    L, b = host_layer(cb_up=np.zeros(spec.n_experts * 4 - 1, np.int8))
    assert status_of(L) == -4 and "truncated" in B.LIB.qmoe_last_error().decode()
    # an FP3 (8-entry) codebook given for the FP2 gate tensor
    L, b = host_layer(cb_gate=np.zeros(spec.n_experts * 8, np.int8))
    assert status_of(L) == -4 and "mismatched" in B.LIB.qmoe_last_error().decode()


def test_layer_check_alignment():
    """The kernels read router rows in 16-byte pieces, codebooks as dwords and the
    bias as fp64: misaligned pointers are refused on the host."""
    L, b = host_layer()
    assert status_of(L) == 0
    L.w_router += 8
    assert status_of(L) == -1 and "router" in B.LIB.qmoe_last_error().decode()
    L, b = host_layer()
    L.cb_up += 2
    assert status_of(L) == -1 and "codebook" in B.LIB.qmoe_last_error().decode()
    L, b = host_layer()
    bias = np.zeros(gen.LayerSpec.tiny().n_experts + 1, np.float64)
    L.router_bias = bias.ctypes.data + 4
    assert status_of(L) == -1 and "bias" in B.LIB.qmoe_last_error().decode()
    L.router_bias = bias.ctypes.data
    assert status_of(L) == 0


def test_layer_check_shapes_formats_sizes():
    assert status_of(host_layer(rot_down=2)[0]) == -3          # unsupported rotation refused up front
    assert status_of(host_layer(rot_gateup=-1)[0]) == -3
    assert status_of(host_layer(fmt_up=3)[0]) == -3            # gate/up formats must match
    assert status_of(host_layer(fmt_down=5)[0]) == -3
    assert status_of(host_layer(topk=9)[0]) == -2
    assert status_of(host_layer(topk=0)[0]) == -2
    spec = gen.LayerSpec.tiny()
    assert status_of(host_layer(topk=spec.n_experts + 1)[0]) == -2
    assert status_of(host_layer(n_experts=0)[0]) == -2
    L, b = host_layer(gate=np.zeros(16, np.uint8))
    assert status_of(L) == -8
    L, b = host_layer()
    L.up = None
    assert status_of(L) == -1
    L, b = host_layer()
    L.w_router_bytes = 2
    assert status_of(L) == -8
    # K=96 FP2 rows are 30 bytes: not 16-byte rows
    odd = gen.LayerSpec.tiny(hidden=96)
    L, b = host_layer(odd)
    assert status_of(L) == -2 and "multiple of 16" in B.LIB.qmoe_last_error().decode()


def test_launch_entry_points_reject_before_launch():
    L, b = host_layer()
    ws = np.zeros(16, np.uint8)
    x = np.zeros((4, 256), np.float32)
    out = np.zeros_like(x)
    st = B.LIB.qmoe_decode_layer(ctypes.byref(L), x.ctypes.data, 5, out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -2
    st = B.LIB.qmoe_decode_layer(ctypes.byref(L), x.ctypes.data, 1, out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -6
    st = B.LIB.qmoe_decode_layer(ctypes.byref(L), x.ctypes.data, 1, out.ctypes.data, None, 0, None)
    assert st == -6
    st = B.LIB.qmoe_decode_layer_mfma(ctypes.byref(L), x.ctypes.data, 5, out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -2
    st = B.LIB.qmoe_decode_layer_mfma(ctypes.byref(L), x.ctypes.data, 1, out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -6
    st = B.LIB.qmoe_quant_act(x.ctypes.data, 4, 256, 2, out.ctypes.data, out.ctypes.data, None)
    assert st == -3
    st = B.LIB.qmoe_quant_act(x.ctypes.data, 4, 100, 0, out.ctypes.data, out.ctypes.data, None)
    assert st == -2
    w = np.zeros(1024, np.uint8)
    cb = np.zeros(16, np.int8)
    st = B.LIB.qmoe_matvec(2, 8, 256, w.ctypes.data, w.nbytes, cb.ctypes.data, 0, x.ctypes.data, 5,
                           out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -2                                            # ncols
    st = B.LIB.qmoe_matvec(2, 8, 256, w.ctypes.data, 10, cb.ctypes.data, 0, x.ctypes.data, 1,
                           out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -8                                            # weights truncated
    st = B.LIB.qmoe_matvec(2, 8, 256, w.ctypes.data, w.nbytes, None, 0, x.ctypes.data, 1,
                           out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -4                                            # missing codebook
    st = B.LIB.qmoe_block_dots(3, 8, 100, w.ctypes.data, w.nbytes, cb.ctypes.data, x.ctypes.data,
                               out.ctypes.data, None)
    assert st == -2
    st = B.LIB.qmoe_prefill_layer(ctypes.byref(L), x.ctypes.data, 4, out.ctypes.data, ws.ctypes.data, 16, None)
    assert st == -6


def test_quantize_rejects_bad_arguments_before_launch():
    """Argument errors of qmoe_quantize are reported on the host, before any
    device work (host pointers stand in: nothing is launched on these paths)."""
    w = np.zeros((1, 4, 256), dtype=np.float32)
    out = np.zeros((1, 4, 80), dtype=np.uint8)
    cb = np.zeros((1, 4), dtype=np.int8)
    ws = np.zeros(qm.qmoe_quantize_workspace_bytes(1, 4, 256) + 256, dtype=np.uint8)
    wsa = ws[(-ws.ctypes.data) % 256:]                     # 256-byte aligned view
    L = B.LIB

    def call(fmt=2, n=1, rows=4, k=256, wp=w, iters=4, o=out, ob=None, c=cb, wsp=wsa, wsb=None):
        return L.qmoe_quantize(fmt, n, rows, k, B._ptr(wp), iters, B._ptr(o), o.nbytes if ob is None else ob,
                               B._ptr(c), B._ptr(wsp), wsp.nbytes if wsb is None else wsb, None)
    assert call(fmt=5) == -3                               # unknown format
    assert call(k=96) == -2                                # row not a multiple of 16 bytes
    assert call(k=100) == -2                               # not a multiple of 32
    assert call(iters=65) == -2 and call(iters=-1) == -2
    assert call(n=0) == -2
    assert call(wp=None) == -1
    assert call(ob=10) == -8                               # out too small
    assert call(wsb=100) == -6                             # workspace too small
    assert call(fmt=4, k=256) == -2                        # FP4 needs k % 512 == 0
    assert call(n=70000, rows=1) == -2                     # more matrices than grid rows
    assert qm.qmoe_quantize_workspace_bytes(1, 4, 33) == 0
    assert qm.qmoe_quantize_workspace_bytes(2, 2048, 4096) >= 2 * 2048 * 4096 * 2


def test_matvec_group_host_checks():
    """Workspace sizing and argument checks of qmoe_matvec_group (host only:
    every refused call returns before any launch)."""
    c = gen.matvec_case(3, 64, 512, 2, seed=2, rot=1)
    w = formats.pack(3, c.codes, c.scales)
    cb = np.ascontiguousarray(c.cb)
    x = np.ascontiguousarray(c.x)
    y = np.zeros((2, 64), dtype=np.float32)
    items = [(3, 64, 512, w, cb, 1, x, y)]
    per = -(-2 * 512 // 256) * 256 + -(-2 * 16 * 4 // 256) * 256
    assert qm.qmoe_matvec_group_workspace_bytes(items, 2) == per
    assert qm.qmoe_matvec_group_workspace_bytes(items * 2, 2) == 2 * per
    assert qm.qmoe_matvec_group_workspace_bytes(items * 5, 2) == 0
    assert qm.qmoe_matvec_group_workspace_bytes(items, 5) == 0
    ws = np.zeros(per, dtype=np.uint8)
    for bad, n, ncols, code in ((items, 5, 2, -2), (items, 1, 0, -2), ([(7,) + items[0][1:]], 1, 2, -3),
                                ([(3, 64, 500) + items[0][3:]], 1, 2, -2)):
        arr = B.matvec_items(bad[:1] if n == 5 else bad)
        st = B.LIB.qmoe_matvec_group(arr, n, ncols, ws.ctypes.data, ws.nbytes, None)
        assert st == code, (n, ncols, st)
    arr = B.matvec_items(items)
    assert B.LIB.qmoe_matvec_group(arr, 1, 2, ws.ctypes.data, ws.nbytes - 1, None) == -6
