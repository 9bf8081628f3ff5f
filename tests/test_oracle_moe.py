"""Pins for the oracle's MoE layer (no GPU).

The layer structure (routed experts, gate/up in the 2.5-bit format, down in the
3.5-bit format, per-expert codebooks) is from lucebox.com "DeepSeek V4 Flash:
284B model, up to 32 tok/s on AMD Ryzen AI MAX+ 395", section "ROCmFPX:
fitting 284B weights into 128 GB". Checks: a dense fp64 recomputation of the
whole layer from dequantized matrices, the top-k = E = 1 reduction to a dense
quantized FFN, the grouped (prefill) form against the per-token form, expert
permutation invariance and identical q columns.
"""
import numpy as np
import pytest

from oracle import formats, moe, quant, router
from synth import gen


def make_layer(spec, seed=0, bias=None):
    cache = {}

    def get(name, e):
        key = (name, e)
        if key not in cache:
            t = gen.expert_tensor(spec, name, e, seed)
            cache[key] = (t.fmt, t.codes, t.scales, t.cb)
        return cache[key]

    return moe.Layer(spec.hidden, spec.inter, spec.n_experts, spec.topk,
                     gen.router_weights(spec, seed), get, bias,
                     spec.rot_gateup, spec.rot_down)


def dense_reference(L, x):
    """Whole layer from dense dequantized fp64 matrices, one token at a time."""
    x = np.atleast_2d(x)
    idx, g, _ = router.route(L.w_router, x, L.bias, L.topk)
    out = np.zeros((x.shape[0], L.hidden))
    for t in range(x.shape[0]):
        xq, dx = quant.quantize_act(x[t], L.rot_gateup)
        xd = quant.dequant_act(xq, dx)
        for s, e in enumerate(idx[t]):
            Wg = formats.dequant(*L.get("gate", int(e)))
            Wu = formats.dequant(*L.get("up", int(e)))
            Wd = formats.dequant(*L.get("down", int(e)))
            gt, ut = Wg @ xd, Wu @ xd
            a = (gt / (1.0 + np.exp(-gt)) * ut).astype(np.float32)
            hq, dh = quant.quantize_act(a, L.rot_down)
            out[t] += g[t, s] * (Wd @ quant.dequant_act(hq, dh))
    return out


@pytest.mark.parametrize("rot", [(0, 0), (1, 1), (0, 1)])
def test_layer_matches_dense_recomputation(rot):
    spec = gen.LayerSpec.tiny(rot_gateup=rot[0], rot_down=rot[1])
    L = make_layer(spec, seed=1)
    x = gen.tokens(3, spec.hidden, seed=1)
    out, idx, g = moe.moe_tokens(L, x)
    ref = dense_reference(L, x)
    assert moe.rel_l2(out, ref) < 1e-12


def test_single_expert_reduces_to_dense_ffn():
    spec = gen.LayerSpec.tiny(n_experts=1, topk=1)
    L = make_layer(spec, seed=2)
    x = gen.tokens(2, spec.hidden, seed=2)
    out, idx, g = moe.moe_tokens(L, x)
    assert np.all(idx == 0) and np.all(g == 1.0)
    Wg = formats.dequant(*L.get("gate", 0))
    Wu = formats.dequant(*L.get("up", 0))
    Wd = formats.dequant(*L.get("down", 0))
    for t in range(2):
        xd = quant.dequant_act(*quant.quantize_act(x[t]))
        gt, ut = Wg @ xd, Wu @ xd
        a = (gt / (1.0 + np.exp(-gt)) * ut).astype(np.float32)
        y = Wd @ quant.dequant_act(*quant.quantize_act(a))
        assert moe.rel_l2(out[t], y) < 1e-13


def test_grouped_equals_per_token():
    spec = gen.LayerSpec.tiny(rot_down=1)
    L = make_layer(spec, seed=3, bias=gen.zipf_bias(spec.n_experts))
    x = gen.tokens(40, spec.hidden, seed=3)
    a, ia, ga = moe.moe_tokens(L, x)
    b, ib, gb = moe.moe_grouped(L, x)
    assert np.array_equal(ia, ib)
    assert moe.rel_l2(b, a) < 1e-9


def test_expert_permutation_invariance():
    spec = gen.LayerSpec.tiny()
    L = make_layer(spec, seed=4)
    perm = np.random.default_rng(0).permutation(spec.n_experts)   # new id -> old id
    P = moe.Layer(L.hidden, L.inter, L.n_experts, L.topk, L.w_router[perm],
                  lambda n, e: L.get(n, int(perm[e])), None)
    x = gen.tokens(4, spec.hidden, seed=4)
    a, ia, _ = moe.moe_tokens(L, x)
    b, ib, _ = moe.moe_tokens(P, x)
    for t in range(4):
        assert sorted(perm[ib[t]].tolist()) == ia[t].tolist()
    assert moe.rel_l2(b, a) < 1e-13


def test_identical_columns_identical_outputs():
    spec = gen.LayerSpec.tiny()
    L = make_layer(spec, seed=5)
    x = np.repeat(gen.tokens(1, spec.hidden, seed=5), 4, axis=0)
    out, idx, g = moe.moe_tokens(L, x)
    for t in range(1, 4):
        assert np.array_equal(out[t], out[0]) and np.array_equal(idx[t], idx[0])


def test_swiglu_definition():
    gt = np.array([0.0, 1.0, -30.0, 5.0])
    ut = np.array([2.0, 3.0, 1.0, -1.0])
    a = moe.swiglu(gt, ut)
    assert a.dtype == np.float32
    assert a[0] == 0.0
    assert a[1] == np.float32(1.0 / (1.0 + np.exp(-1.0)) * 3.0)
    assert abs(a[2]) < 1e-11
