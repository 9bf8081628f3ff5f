"""Pins for the oracle's block dots, rows and router (no GPU).

Block dots: brute-force integer loops on tiny inputs and a closed form. Rows:
the dequantized fp64 matrix-vector product. Router: exact rational logits
(fractions.Fraction) on tiny sizes, and hand-worked inputs whose fp64 result
depends on the summation order (the order is this repository's reading; the
pages — lucebox.com "Lucebox × Geometric: DeepSeek V4 Flash 0731 reaches 32.7
tok/s on AMD Strix Halo", section "Run with Lucebox Engine" — fix only 256
experts with 6 routed).
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import dots, formats, quant, router
from synth import gen


def test_block_dots_brute_force():
    g = np.random.default_rng(0)
    for fmt in (2, 3, 4):
        codes = g.integers(0, 1 << fmt, size=(3, 96), dtype=np.uint8)
        cb = g.integers(-128, 128, size=1 << fmt, dtype=np.int8)
        xq = g.integers(-127, 128, size=96, dtype=np.int8)
        P = dots.block_dots(codes, cb, xq)
        for r in range(3):
            for b in range(3):
                acc = 0
                for j in range(32):
                    acc += int(cb[int(codes[r, 32 * b + j])]) * int(xq[32 * b + j])
                assert P[r, b] == acc


def test_block_dots_closed_form_and_bound():
    codes = np.full((2, 64), 3, dtype=np.uint8)
    cb = np.array([0, 0, 0, -128], dtype=np.int8)
    xq = np.full(64, -127, dtype=np.int8)
    P = dots.block_dots(codes, cb, xq)
    assert np.all(P == 32 * 128 * 127) and 32 * 128 * 127 < 2 ** 31


def test_matvec_equals_dequantized_product():
    for fmt, rot in ((2, 0), (3, 1), (4, 0), (4, 1)):
        c = gen.matvec_case(fmt, 16, 256, ncols=3, seed=5, rot=rot)
        y, xq, d = dots.matvec(fmt, c.codes, c.scales, c.cb, c.x, rot)
        W = formats.dequant(fmt, c.codes, c.scales, c.cb)
        X = quant.dequant_act(xq, d)
        ref = X @ W.T
        assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_matvec_closed_form():
    rows, k = 4, 128
    codes = np.full((rows, k), 1, dtype=np.uint8)
    cb = np.array([0, 5, 0, 0], dtype=np.int8)
    scales = np.full((rows, k // 32), 0x3C00, dtype=np.uint16)   # 1.0
    x = np.full((1, k), 2.0, dtype=np.float32)                    # d = 2/127, q = 127
    y, xq, d = dots.matvec(2, codes, scales, cb, x)
    assert np.all(xq == 127)
    want = (k // 32) * float(np.float32(2.0) / np.float32(127.0)) * 5 * 127 * 32
    assert np.allclose(y, want, rtol=1e-15)


# ---------------------------------------------------------------- router

def _f16(v):
    return np.float16(v).view(np.uint16)


def _exact_logits(w_bits, x):
    w = np.asarray(w_bits, np.uint16).view(np.float16).astype(np.float64)
    out = []
    for e in range(w.shape[0]):
        out.append(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(w[e], x)))
    return out


def test_router_matches_exact_rationals_on_tiny_sizes():
    g = np.random.default_rng(6)
    checked = 0
    for trial in range(20):
        E, H, k = 12, 96, 3
        w = (g.normal(0, 0.02, (E, H))).astype(np.float16).view(np.uint16)
        x = g.standard_normal(H).astype(np.float32)
        lg = router.logits(w, x[None])[0]
        ex = _exact_logits(w, x)
        for e in range(E):
            assert abs(Fraction(lg[e]) - ex[e]) <= Fraction(1, 10 ** 12)
        order = sorted(range(E), key=lambda e: (-ex[e], e))
        if ex[order[k - 1]] - ex[order[k]] > Fraction(1, 10 ** 9):
            idx, gw, _ = router.route(w, x[None], None, k)
            assert list(idx[0]) == sorted(order[:k])
            checked += 1
    assert checked >= 15


def _block_input(block_values, hidden):
    """Router input whose block b sums to block_values[b]: w = 1 at the block's
    first position and x = value there (all values exact in fp16 x fp32)."""
    w = np.zeros((1, hidden), np.float16)
    x = np.zeros(hidden, np.float32)
    for b, v in enumerate(block_values):
        w[0, 32 * b] = 1.0
        x[32 * b] = v
    return w.view(np.uint16), x


def test_router_tree_order_hand_worked():
    """Block sums [1, 2^53, 1, -2^53]. Stride-halving tree (pairs (j, j+n)):
    (1+1) + (2^53-2^53) = 2. (An adjacent-pair tree would give 1 and a
    sequential sum 0: both would fail.)"""
    w, x = _block_input([1.0, 2.0 ** 53, 1.0, -(2.0 ** 53)], 128)
    assert router.logits(w, x[None])[0, 0] == 2.0


def test_router_tree_pads_to_power_of_two():
    """3 blocks pad to 4 with +0.0: (s0 + s2) + (s1 + 0)."""
    w, x = _block_input([2.0 ** 53, 1.0, 1.0], 96)
    # s0 + s2 = 2^53 + 1 -> 2^53 (tie to even); + s1 -> 2^53 + 1 -> 2^53
    assert router.logits(w, x[None])[0, 0] == 2.0 ** 53
    w, x = _block_input([1.0, 2.0 ** 53, -(2.0 ** 53)], 96)
    # (1 + -2^53) + (2^53 + 0) = 1
    assert router.logits(w, x[None])[0, 0] == 1.0


def test_router_in_block_order_is_sequential():
    """Inside one block: 0 + 1 + 2^53 + 1 - 2^53 sequentially = 0."""
    w = np.zeros((1, 32), np.float16)
    w[0, :4] = 1.0
    x = np.zeros(32, np.float32)
    x[:4] = [1.0, 2.0 ** 53, 1.0, -(2.0 ** 53)]
    assert router.logits(w.view(np.uint16), x[None])[0, 0] == 0.0


def test_router_ties_go_to_lower_id_and_ascending_output():
    H = 64
    g = np.random.default_rng(7)
    base = g.normal(0, 0.02, H).astype(np.float16)
    w = np.stack([base * 0.5, base, base * 0.25, base, base * 0.1]).astype(np.float16)
    x = (np.sign(base.astype(np.float32)) * 3).astype(np.float32)
    idx, gw, lg = router.route(w.view(np.uint16), x[None], None, 2)
    assert lg[0, 1] == lg[0, 3]
    assert list(idx[0]) == [1, 3]
    idx, gw, lg = router.route(w.view(np.uint16), x[None], None, 1)
    assert list(idx[0]) == [1]                      # tie 1 vs 3 -> lower id
    assert np.isclose(gw[0, 0], 1.0)


def test_router_softmax_and_bias():
    spec = gen.LayerSpec.tiny()
    w = gen.router_weights(spec, seed=3)
    x = gen.tokens(5, spec.hidden, seed=3)
    bias = gen.zipf_bias(spec.n_experts)
    idx, gw, lg = router.route(w, x, bias, spec.topk)
    lg0 = router.logits(w, x)
    assert np.array_equal(lg, lg0 + bias[None, :])
    for t in range(5):
        assert np.all(np.diff(idx[t]) > 0)
        assert abs(gw[t].sum() - 1.0) < 1e-15
        sel = lg[t, idx[t]]
        assert np.allclose(gw[t] / gw[t].max(), np.exp(sel - sel.max()), rtol=1e-14)
        rest = np.setdiff1d(np.arange(spec.n_experts), idx[t])
        assert lg[t, idx[t]].min() >= lg[t, rest].max()
    big = np.zeros(spec.n_experts)
    big[[5, 2]] = 1e6
    idx, gw, _ = router.route(w, x, big, 2)
    assert np.all(idx == [2, 5])
