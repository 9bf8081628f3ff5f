"""Pins of the weight quantizer oracle (float -> ROCmFPX with per-matrix
codebooks), each independent of the function it checks:

* exact recovery: weights built as d * L[code] with a known codebook L (every
  level present, each level nearest a distinct starting centroid, every block
  holding a +-127 level) come back with the same codes, codebook and scales,
  and dequantize to the same values bit for bit;
* Lloyd-Max closed form: for a uniform source the uniform quantizer is a fixed
  point, so the centroids of all integers of [-32512, 32511] stay at the
  starting midpoints (within the rounding of the means and the tie rule);
* scale rules: the stored fp16 is the nearest fp16 to fl32(amax / 127) (checked
  against its neighbours); the E8M0 power of two is the least one >= that value;
* a zero block stores a zero scale and zero values;
* a pure-Python per-weight implementation (loops over weights and entries, no
  numpy vectorization) gives the same codes, codebooks and packed bytes on
  small ragged inputs, for all three formats.
"""
import numpy as np
import pytest

from oracle import formats, quantize

LEVELS = {
    2: [-127, -40, 30, 127],
    3: [-127, -80, -45, -10, 12, 50, 85, 127],
    4: [-127] + [int(round(-119.0625 + 15.875 * i)) for i in range(1, 15)] + [127],
}


def build_exact(fmt, n, rows, k, seed):
    rng = np.random.default_rng(seed)
    L = np.array(LEVELS[fmt], dtype=np.int64)
    nl = len(L)
    codes = rng.integers(0, nl, size=(n, rows, k)).astype(np.uint8)
    # every block holds a +-127 level at a random position; every level appears
    blocks = codes.reshape(n, rows, k // 32, 32)
    pos = rng.integers(0, 32, size=blocks.shape[:-1])
    top = np.where(rng.integers(0, 2, size=blocks.shape[:-1]) == 1, nl - 1, 0)
    np.put_along_axis(blocks, pos[..., None], top[..., None].astype(np.uint8), axis=-1)
    for m in range(n):
        codes[m, 0, :nl] = np.arange(nl)
        codes[m, 0, nl - 1] = nl - 1
    codes = blocks.reshape(n, rows, k)
    if fmt == 4:
        e = rng.integers(118, 124, size=(n, rows, k // 32)).astype(np.int64)
        d = np.ldexp(1.0, e - 127)
        stored = e.astype(np.uint8)
    else:
        h = rng.uniform(0.01, 0.1, size=(n, rows, k // 32)).astype(np.float16)
        d = h.astype(np.float64)
        stored = h.view(np.uint16)
    w = (L[codes.astype(np.int64)].reshape(n, rows, k // 32, 32) * d[..., None]).reshape(n, rows, k)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)   # exact in fp32
    return w.astype(np.float32), codes, stored, L.astype(np.int8)


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_exact_recovery(fmt):
    w, codes, stored, L = build_exact(fmt, 2, 8, 256, seed=fmt)
    packed, cbs, got_codes, got_scales = quantize.quantize(fmt, w, iters=1)
    for m in range(2):
        assert np.array_equal(cbs[m], L)
        assert np.array_equal(got_codes[m], codes[m])
        assert np.array_equal(got_scales[m], stored[m])
        assert np.array_equal(packed[m], formats.pack(fmt, codes[m], stored[m]))
        assert np.array_equal(quantize.dequantize(fmt, packed[m], cbs[m], 256), w[m].astype(np.float64))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_uniform_source_fixed_point(bits):
    v = np.arange(-32512, 32512, dtype=np.int64)
    c0 = quantize.initial_centroids(bits)
    assert np.array_equal(np.diff(c0), np.full(len(c0) - 1, 65024 // len(c0)))   # equal cells
    assert c0[0] + c0[-1] == 0
    c = quantize.lloyd(v, bits, iters=6)
    # ties to the lower entry and means rounded half up drift each centroid by
    # at most about one unit per iteration; a cell is >= 4064 units wide
    assert np.max(np.abs(c - c0)) <= 8, (c, c0)


def test_lloyd_moves_to_cluster_means():
    """Three well separated clumps and four centroids: the clumps' exact means are
    reached after one iteration (the idle centroid keeps its start)."""
    v = np.concatenate([np.full(10, -30000), np.full(7, -10000) + np.arange(7), np.full(5, 25000)])
    c = quantize.lloyd(v, 2, iters=3)
    assert c[0] == -30000                       # nearest start -24384
    assert c[1] == -9997                        # mean of -10000..-9994 (start -8128)
    assert c[3] == 25000                        # start 24384
    assert c[2] == quantize.initial_centroids(2)[2]   # no members: unchanged


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_scale_rules(fmt):
    rng = np.random.default_rng(10 + fmt)
    w = (rng.standard_normal((16, 512)) * np.exp(rng.uniform(-8, 3, size=(16, 1)))).astype(np.float32)
    sc, d = quantize.block_scales(fmt, w)
    t = (np.max(np.abs(w.reshape(16, 16, 32)), axis=-1) / np.float32(127)).astype(np.float32).astype(np.float64)
    if fmt == 4:
        e = sc.astype(np.int64)
        assert np.all(np.ldexp(1.0, e - 127) >= t)
        assert np.all(np.ldexp(1.0, e - 128) < t)
    else:
        h = sc.astype(np.int64)
        val = sc.view(np.float16).astype(np.float64)
        for nb in (h - 1, h + 1):                 # no neighbouring fp16 is nearer
            other = nb.astype(np.uint16).view(np.float16).astype(np.float64)
            assert np.all(np.abs(val - t) <= np.abs(other - t))
    v = quantize.normalized(w, d)
    vmax = np.max(np.abs(v.reshape(16, 16, 32)), axis=-1)
    if fmt == 4:   # a power of two at or above amax / 127: the largest value lands in (63.5, 127]
        assert np.all((vmax > 16256) & (vmax <= 32512))
    else:          # fp16 normal range: relative rounding <= 2^-11
        normal = t >= 2.0 ** -14
        assert normal.sum() > 100
        assert np.all(np.abs(vmax - 32512)[normal] <= 32512 * 2.0 ** -11 + 1)


@pytest.mark.parametrize("fmt", [2, 4])
def test_zero_block(fmt):
    w = np.zeros((1, 2, 64), dtype=np.float32)
    w[0, 1, 40] = 1.5
    packed, cbs, codes, sc = quantize.quantize(fmt, w, iters=2)
    _, d = quantize.block_scales(fmt, w[0])
    assert d[0, 0] == 0 or fmt == 4
    assert np.all(sc[0, 0] == 0)
    deq = quantize.dequantize(fmt, packed[0], cbs[0], 64)
    assert np.all(np.abs(deq[0]) <= np.abs(deq).max())
    assert abs(deq[1, 40] - 1.5) <= 1.5 / 127


# ---------------------------------------------------------------- pure-Python reference
def py_quantize(fmt, w, iters):
    bits = formats.BITS[fmt]
    n, rows, k = w.shape
    f32 = np.float32
    out_codes = np.zeros((n, rows, k), np.uint8)
    out_cb = np.zeros((n, 1 << bits), np.int8)
    out_sc = []
    for m in range(n):
        vs = []
        scs = np.zeros((rows, k // 32), np.uint16 if fmt != 4 else np.uint8)
        for r in range(rows):
            for b in range(k // 32):
                blk = [f32(w[m, r, 32 * b + j]) for j in range(32)]
                a = f32(0.0)
                for x in blk:
                    a = max(a, f32(abs(x)))
                t = f32(a / f32(127.0))
                if fmt == 4:
                    if t == 0:
                        e = 0
                    else:
                        kk = -200
                        while 2.0 ** kk < float(t):
                            kk += 1
                        e = min(max(127 + kk, 1), 254)
                    d = f32(2.0 ** (e - 127))
                    scs[r, b] = e
                else:
                    h = np.float16(t) if float(t) < 65520.0 else np.float16(65504.0)
                    d = f32(h)
                    scs[r, b] = np.array([h]).view(np.uint16)[0]
                for x in blk:
                    if d == 0:
                        vs.append(0)
                    else:
                        y = f32(f32(x / d) * f32(256.0))
                        vs.append(int(min(max(int(np.rint(y)), -32767), 32767)))
        nc = 1 << bits
        c = [32512 * (2 * i + 1) // nc - 32512 for i in range(nc)]

        def near(x, cents):
            bi = 0
            for i in range(1, len(cents)):
                if abs(x - cents[i]) < abs(x - cents[bi]):
                    bi = i
            return bi
        for _ in range(iters):
            S = [0] * nc
            N = [0] * nc
            for x in vs:
                i = near(x, c)
                S[i] += x
                N[i] += 1
            c = [(2 * S[i] + N[i]) // (2 * N[i]) if N[i] else c[i] for i in range(nc)]
        C = [min(max((ci + 128) // 256, -127), 127) for ci in c]
        out_cb[m] = C
        for idx, x in enumerate(vs):
            out_codes[m].flat[idx] = near(x, [256 * ci for ci in C])
        out_sc.append(scs)
    return out_codes, out_cb, np.stack(out_sc)


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_matches_pure_python(fmt):
    rng = np.random.default_rng(20 + fmt)
    w = (rng.standard_normal((2, 3, 64)) * 0.02).astype(np.float32)
    w[1, 2, :32] = 0.0                                   # a zero block
    w[0, 1, 5] = 0.3                                     # an outlier
    packed, cbs, codes, sc = quantize.quantize(fmt, w, iters=3)
    pc, pcb, psc = py_quantize(fmt, w, iters=3)
    assert np.array_equal(cbs, pcb)
    assert np.array_equal(codes, pc)
    assert np.array_equal(sc, psc)
    for m in range(2):
        assert np.array_equal(packed[m], formats.pack(fmt, pc[m], psc[m]))
