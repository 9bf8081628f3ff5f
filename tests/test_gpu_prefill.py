"""GPU parity of the prefill layer (grouped int8 MFMA expert GEMMs, and the
matvec path for experts with at most four pairs) against the CPU oracle,
through the C ABI.

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


SMALL = 4   # with qmoe_prefill_layer_ex(..., SMALL) experts with 1..SMALL pairs take the matvec path


def group_lists(ws, lay, E, npairs):
    """(counts, offsets, pairs, tiles [(expert, first)], small expert ids) from
    the workspace's group region."""
    n = 3 * E + 1 + npairs + 2 * (npairs + E) + 1 + E
    grp = ws[lay["group"]: lay["group"] + 4 * n].cpu().numpy().view(np.int32)
    counts, offsets, pairs = grp[:E], grp[E:2 * E + 1], grp[3 * E + 1: 3 * E + 1 + npairs]
    ntiles = int(grp[2 * E + 1])
    t0 = 3 * E + 1 + npairs
    tiles = grp[t0: t0 + 2 * ntiles].reshape(ntiles, 2)
    s0 = t0 + 2 * (npairs + E)
    small = grp[s0 + 1: s0 + 1 + int(grp[s0])]
    return counts, offsets, pairs, tiles, small


def run_prefill(dl, x, ws=None, small=None):
    xd = qm.device.to_device(x)
    out = torch.full_like(xd, float("nan"))
    ws = dl.workspace(max(1, x.shape[0])) if ws is None else ws
    if small is None:
        qm.qmoe_prefill_layer(dl.desc, xd, out, ws)
    else:
        qm.qmoe_prefill_layer_ex(dl.desc, xd, out, ws, small)
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


@pytest.mark.parametrize("small", [0, 2, SMALL])
@pytest.mark.parametrize("ntok,topk", [(1, 2), (7, 3), (333, 6), (1030, 5)])
def test_prefill_grouping_exact(ntok, topk, small):
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
    qm.qmoe_prefill_layer_ex(dl.desc, xd, out, ws, small)
    torch.cuda.synchronize()
    lay = qm.qmoe_workspace_layout(dl.desc, ntok)
    E, K = spec.n_experts, spec.topk
    idx = ws[lay["idx"]: lay["idx"] + 4 * ntok * K].cpu().numpy().view(np.int32).reshape(ntok, K)
    counts, offsets, pairs, tiles, small_ids = group_lists(ws, lay, E, ntok * K)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[E] == ntok * K and np.array_equal(np.diff(offsets), counts)
    for e in range(E):
        assert np.array_equal(pairs[offsets[e]: offsets[e + 1]], np.flatnonzero(flat == e))
    # experts with 1..small pairs are listed for the matvec path, the others cut into 64-pair tiles
    assert np.array_equal(small_ids, np.flatnonzero((counts >= 1) & (counts <= small)))
    want = [(e, f) for e in range(E) if counts[e] > small for f in range(0, counts[e], 64)]
    assert [tuple(t) for t in tiles] == want


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
    """Within a path a token's output does not depend on the other tokens of the
    batch: on the MFMA path its position inside an expert tile changes, its
    result does not; on the matvec path (experts with at most four pairs) each
    pair is its own column. Across paths the results differ only by rounding
    (both within the bar of the oracle)."""
    spec = gen.LayerSpec.tiny(n_experts=8, topk=2)
    dl = qm.device.DeviceLayer(spec, seed=47)
    x = gen.tokens(130, spec.hidden, seed=47)
    full, _ = run_prefill(dl, x)
    most, ws = run_prefill(dl, x[40:130])                 # every expert keeps more than 4 pairs
    lay = qm.qmoe_workspace_layout(dl.desc, 90)
    counts, _, _, _, small = group_lists(ws, lay, spec.n_experts, 90 * spec.topk)
    assert len(small) == 0 and counts.min() > SMALL
    assert np.array_equal(full[40:130], most)
    three, _ = run_prefill(dl, x[100:103], small=SMALL)   # every expert has at most 3 pairs
    one, _ = run_prefill(dl, x[101:102], small=SMALL)
    assert np.array_equal(three[1], one[0])
    tiles3, _ = run_prefill(dl, x[100:103], small=0)      # the same three tokens on the MFMA tiles
    ref, _, _ = moe.moe_tokens(oracle_layer(spec, 47, dl.w_router_host), x[100:103])
    assert np.array_equal(tiles3, full[100:103])
    assert moe.rel_l2(three, ref) < TOL and moe.rel_l2(full[100:103], ref) < TOL


@pytest.mark.parametrize("fmts", [(2, 3), (4, 4), (3, 2), (2, 4), (4, 3)])
def test_prefill_small_and_tile_paths(fmts):
    """A skewed batch that sends some experts down the MFMA tiles and others
    (one to four pairs) down the matvec path, for every format pairing, against
    the per-token oracle; and a batch where every expert is small."""
    spec = gen.LayerSpec.tiny(hidden=512, inter=512, n_experts=24, topk=6, fmt_gate=fmts[0], fmt_up=fmts[0],
                              fmt_down=fmts[1])
    bias = gen.zipf_bias(spec.n_experts)
    dl = qm.device.DeviceLayer(spec, seed=49, bias=bias)
    L = oracle_layer(spec, 49, dl.w_router_host, bias)
    x = gen.tokens(48, spec.hidden, seed=49)
    out, ws = run_prefill(dl, x, small=SMALL)
    lay = qm.qmoe_workspace_layout(dl.desc, 48)
    counts, _, _, tiles, small = group_lists(ws, lay, spec.n_experts, 48 * spec.topk)
    assert len(tiles) > 0 and len(small) > 0
    ref, idx_ref, _ = moe.moe_tokens(L, x)
    assert np.array_equal(np.bincount(idx_ref.ravel(), minlength=spec.n_experts), counts)
    errs = [moe.rel_l2(out[t], ref[t]) for t in range(48)]
    assert max(errs) < TOL, max(errs)
    out2, ws2 = run_prefill(dl, x[:2], small=SMALL)       # at most 2 pairs per expert
    counts2, _, _, tiles2, small2 = group_lists(ws2, qm.qmoe_workspace_layout(dl.desc, 2), spec.n_experts,
                                                2 * spec.topk)
    assert len(tiles2) == 0 and len(small2) == np.count_nonzero(counts2)
    assert moe.rel_l2(out2, ref[:2]) < TOL
    with pytest.raises(qm.QmoeError):
        run_prefill(dl, x[:2], small=SMALL + 1)
