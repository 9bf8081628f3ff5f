"""GPU parity of the prefill layer (grouped int8 MFMA expert GEMMs) against the
CPU oracle, through the C ABI.

Bars: routing ids bit-exact; fp32 layer output within 1e-3 relative L2 of the
fp64 oracle (the int8 requantization of the SwiGLU output can flip by one code
at a rounding boundary, so outputs are compared by relative L2); repeated calls
bit-identical.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import bit_block_quantized_rocmfp2_amd as qm  # noqa: E402
from oracle import moe, router  # noqa: E402
from synth import gen  # noqa: E402

TOL = 1e-3


def oracle_layer(spec, seed, w_router, bias=None):
    cache = {}

    def get(name, e):
        if (name, e) not in cache:
            t = gen.expert_tensor(spec, name, e, seed)
            cache[(name, e)] = (t.fmt, t.codes, t.scales, t.cb)
        return cache[(name, e)]

    return moe.Layer(spec.hidden, spec.inter, spec.n_experts, spec.topk, w_router, get, bias,
                     spec.rot_gateup, spec.rot_down)


def run_prefill(dl, x, ws=None):
    xd = qm.device.to_device(x)
    out = torch.full_like(xd, float("nan"))
    ws = dl.workspace(max(1, x.shape[0])) if ws is None else ws
    qm.qmoe_prefill_layer(dl.desc, xd, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ws


@pytest.mark.parametrize("ntok", [1, 63, 64, 65, 200])
def test_prefill_tiny_ragged(ntok):
    """Tiles of 64 pairs: fewer, exactly one and one more than a tile."""
    spec = gen.LayerSpec.tiny()
    dl = qm.device.DeviceLayer(spec, seed=40)
    x = gen.tokens(ntok, spec.hidden, seed=40)
    out, ws = run_prefill(dl, x)
    ref, idx_ref, _ = moe.moe_grouped(oracle_layer(spec, 40, dl.w_router_host), x)
    assert moe.rel_l2(out, ref) < TOL
    lay = qm.qmoe_workspace_layout(dl.desc, max(1, ntok))
    idx = ws[lay["idx"]: lay["idx"] + 4 * ntok * spec.topk].cpu().numpy().view(np.int32).reshape(ntok, spec.topk)
    assert np.array_equal(idx, idx_ref)


@pytest.mark.parametrize("ntok,topk", [(1, 2), (7, 3), (333, 6), (1030, 5)])
def test_prefill_grouping_exact(ntok, topk):
    """Expert grouping for pair counts that are and are not multiples of four
    (the grouping reads pair ids 16 bytes at a time and takes the last
    npairs % 4 one by one) and that span several 1024-pair passes: counts
    equal the histogram of the routing ids, offsets their exclusive scan, and
    each expert's pairs are exactly its pair indices in ascending order."""
    spec = gen.LayerSpec.tiny(n_experts=24, topk=topk)
    dl = qm.device.DeviceLayer(spec, seed=44)
    x = gen.tokens(ntok, spec.hidden, seed=44)
    xd = qm.device.to_device(x)
    out = torch.empty_like(xd)
    ws = dl.workspace(ntok)
    qm.qmoe_prefill_layer(dl.desc, xd, out, ws)
    torch.cuda.synchronize()
    lay = qm.qmoe_workspace_layout(dl.desc, ntok)
    E, K = spec.n_experts, spec.topk
    idx = ws[lay["idx"]: lay["idx"] + 4 * ntok * K].cpu().numpy().view(np.int32).reshape(ntok, K)
    grp = ws[lay["group"]: lay["group"] + 4 * (3 * E + 1 + ntok * K)].cpu().numpy().view(np.int32)
    counts, offsets, pairs = grp[:E], grp[E:2 * E + 1], grp[3 * E + 1:]
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[E] == ntok * K and np.array_equal(np.diff(offsets), counts)
    for e in range(E):
        assert np.array_equal(pairs[offsets[e]: offsets[e + 1]], np.flatnonzero(flat == e))


@pytest.mark.parametrize("rots", [(0, 1), (1, 0), (1, 1)])
def test_prefill_rotations(rots):
    spec = gen.LayerSpec.tiny(rot_gateup=rots[0], rot_down=rots[1])
    dl = qm.device.DeviceLayer(spec, seed=41)
    x = gen.tokens(90, spec.hidden, seed=41)
    out, _ = run_prefill(dl, x)
    ref, _, _ = moe.moe_grouped(oracle_layer(spec, 41, dl.w_router_host), x)
    assert moe.rel_l2(out, ref) < TOL


@pytest.mark.parametrize("fmts", [(4, 4), (3, 2), (2, 4), (4, 3)])
def test_prefill_formats(fmts):
    """Every gate/up and down format pairing (FP4 needs K a multiple of 512)."""
    spec = gen.LayerSpec.tiny(hidden=512, inter=512, fmt_gate=fmts[0], fmt_up=fmts[0], fmt_down=fmts[1])
    dl = qm.device.DeviceLayer(spec, seed=42)
    x = gen.tokens(70, spec.hidden, seed=42)
    out, _ = run_prefill(dl, x)
    ref, _, _ = moe.moe_grouped(oracle_layer(spec, 42, dl.w_router_host), x)
    assert moe.rel_l2(out, ref) < TOL


def test_prefill_hidden_8192():
    """The largest hidden size: 32 K-stages in the gate/up GEMM, 64 row tiles of
    128 in the down GEMM, and the tiled router's deepest tree."""
    spec = gen.LayerSpec.tiny(hidden=8192, inter=512, n_experts=8, topk=2)
    dl = qm.device.DeviceLayer(spec, seed=48)
    x = gen.tokens(70, spec.hidden, seed=48)
    out, ws = run_prefill(dl, x)
    ref, idx_ref, _ = moe.moe_grouped(oracle_layer(spec, 48, dl.w_router_host), x)
    assert moe.rel_l2(out, ref) < TOL
    lay = qm.qmoe_workspace_layout(dl.desc, 70)
    idx = ws[lay["idx"]: lay["idx"] + 4 * 70 * spec.topk].cpu().numpy().view(np.int32).reshape(70, spec.topk)
    assert np.array_equal(idx, idx_ref)


def test_prefill_skewed_many_experts():
    """Zipf-biased routing over 40 experts, top-6: several tiles for the hot
    experts, idle experts, a ragged tail in each."""
    spec = gen.LayerSpec.tiny(n_experts=40, topk=6)
    bias = gen.zipf_bias(spec.n_experts)
    dl = qm.device.DeviceLayer(spec, seed=43, bias=bias)
    x = gen.tokens(300, spec.hidden, seed=43)
    out, ws = run_prefill(dl, x)
    L = oracle_layer(spec, 43, dl.w_router_host, bias)
    ref, idx_ref, _ = moe.moe_grouped(L, x)
    counts = np.bincount(idx_ref.ravel(), minlength=spec.n_experts)
    assert counts.max() > 128 and (counts == 0).any()      # the fixture is really skewed
    assert moe.rel_l2(out, ref) < TOL


def test_prefill_matches_decode_definition():
    """Prefill of q tokens equals the per-token definition (moe_tokens), the
    same reference the decode path is held to."""
    spec = gen.LayerSpec.tiny(n_experts=16, topk=4)
    dl = qm.device.DeviceLayer(spec, seed=44)
    x = gen.tokens(4, spec.hidden, seed=44)
    out, _ = run_prefill(dl, x)
    ref, _, _ = moe.moe_tokens(oracle_layer(spec, 44, dl.w_router_host), x)
    assert moe.rel_l2(out, ref) < TOL


def test_prefill_determinism_and_stale_workspace():
    spec = gen.LayerSpec.tiny(n_experts=12, topk=3)
    dl = qm.device.DeviceLayer(spec, seed=45)
    a = gen.tokens(150, spec.hidden, seed=450)
    b = gen.tokens(37, spec.hidden, seed=451)
    ws = dl.workspace(150)
    o1, _ = run_prefill(dl, a, ws)
    o2, _ = run_prefill(dl, b, ws)
    o3, _ = run_prefill(dl, a, ws)
    assert np.array_equal(o1, o3)
    ref_b, _, _ = moe.moe_grouped(oracle_layer(spec, 45, dl.w_router_host), b)
    assert moe.rel_l2(o2, ref_b) < TOL


def test_prefill_empty():
    spec = gen.LayerSpec.tiny()
    dl = qm.device.DeviceLayer(spec, seed=46)
    x = np.zeros((0, spec.hidden), dtype=np.float32)
    xd = torch.zeros((0, spec.hidden), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, spec.hidden), dtype=torch.float32, device="cuda")
    qm.qmoe_prefill_layer(dl.desc, xd, out, dl.workspace(1))
    torch.cuda.synchronize()
    assert x.shape == out.shape


def test_prefill_columns_independent():
    """A token's output does not depend on the other tokens in the batch (its
    position inside an expert tile changes, its result does not)."""
    spec = gen.LayerSpec.tiny(n_experts=8, topk=2)
    dl = qm.device.DeviceLayer(spec, seed=47)
    x = gen.tokens(130, spec.hidden, seed=47)
    full, _ = run_prefill(dl, x)
    part, _ = run_prefill(dl, x[100:103])
    assert np.array_equal(full[100:103], part)
