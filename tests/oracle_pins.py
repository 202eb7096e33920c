"""Pins that tie the oracle to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a hand-worked example, a closed form, a
library routine, an invariant, or a brute force over values the test
chose itself (blocks are built from known scales and nibbles, so no decoder
is shared with the oracle).  ``tests/test_oracle_mutants.py`` plants
plausible mistakes in copies of the oracle and checks that some pin fails
for each of them.
"""
from __future__ import annotations

import math
import os

import numpy as np

from qhelpers import (RandomQ4_0, RandomQ4K, RandomQ8, f16_value, make_q4_0, make_q8, make_sb, pack_scales,
                      q4_0_values, sb_values)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _ulp32(v):
    return float(np.spacing(np.float32(abs(v)))) if v != 0 else float(np.finfo(np.float32).tiny)


# ----------------------------------------------------------------- f16 ----

def pin_f16_decode_exhaustive(o):
    """Every one of the 65,536 f16 patterns decodes as numpy decodes it."""
    h = np.arange(65536, dtype=np.uint16)
    got = o.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "f16 decode: NaN patterns differ"
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32)), "f16 decode differs from numpy"


def pin_f16_encode(o):
    """f32 -> f16 round-to-nearest-even agrees with numpy on every f16 value,
    every midpoint between neighbours (the ties), and random f32 values across
    the normal, subnormal and overflow ranges."""
    h = np.arange(65536, dtype=np.uint16)
    v = h.view(np.float16)
    fin = np.isfinite(v)
    vals = v[fin].astype(np.float32)
    assert np.array_equal(o.f32_to_f16(vals), h[fin]), "f16 encode: round trip of f16 values"
    pos = np.sort(v[fin & (v >= 0)].astype(np.float64))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)          # exact in f32
    mids = np.concatenate([mids, -mids, np.float32([65504 + 16, 65520, 65519.99, 1e9, -1e9])])
    with np.errstate(over="ignore"):
        want = mids.astype(np.float16).view(np.uint16)
    assert np.array_equal(o.f32_to_f16(mids), want), "f16 encode: ties"
    g = np.random.default_rng(7)
    r = (g.standard_normal(200_000) * np.exp2(g.integers(-30, 20, 200_000))).astype(np.float32)
    with np.errstate(over="ignore"):
        want = r.astype(np.float16).view(np.uint16)
    assert np.array_equal(o.f32_to_f16(r), want), "f16 encode: random"
    nan = o.f32_to_f16(np.float32([np.nan]))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0, "f16 encode: NaN"


# ---------------------------------------------------------------- q8_0 ----

def pin_q8_golden(o):
    """Hand-worked quantization examples: exact ties, zero block, subnormal d."""
    lines = _golden_lines("q8_0_rounding.txt")
    for i in range(0, len(lines), 3):
        x = np.array([float(t) for t in lines[i].split(":")[1].split()], np.float32)
        dbits = int(lines[i + 1].split(":")[1], 16)
        q = [int(t) for t in lines[i + 2].split(":")[1].split()]
        got = o.quantize_q8_0(x)
        want = np.frombuffer(np.uint16(dbits).tobytes() + np.array(q, np.int8).tobytes(), np.uint8)
        assert np.array_equal(got, want), f"q8_0 golden block {i // 3}: {got} != {want}"


def _q8_split(blocks):
    b = blocks.reshape(-1, 34)
    return b[:, 0:2].copy().view(np.uint16).ravel(), b[:, 2:].view(np.int8).astype(np.int64)


def pin_q8_properties(o):
    """Round-trip bound |x - d*q| <= d/2 (normal-range d), |q| <= 127, the
    largest magnitude maps to +-127, d == f16(amax/127) by numpy, sign
    symmetry, and exact power-of-two scale equivariance."""
    g = np.random.default_rng(11)
    for scale in (1.0, 2.0 ** 5, 2.0 ** -4, 3.7):
        x = (g.standard_normal(32 * 256) * scale).astype(np.float32)
        blk = o.quantize_q8_0(x)
        dbits, q = _q8_split(blk)
        d = dbits.view(np.float16).astype(np.float64)
        xb = x.reshape(-1, 32).astype(np.float64)
        amax = np.abs(x.reshape(-1, 32)).max(axis=1)
        want_d = (amax / np.float32(127)).astype(np.float32).astype(np.float16)
        assert np.array_equal(dbits, want_d.view(np.uint16)), "q8_0: d != f16(amax/127)"
        assert np.all(np.abs(q) <= 127), "q8_0: |q| > 127"
        err = np.abs(xb - d[:, None] * q)
        assert np.all(err <= d[:, None] * (0.5 + 1e-5)), f"q8_0: bound violated, max {np.max(err / d[:, None])}"
        arg = np.abs(xb).argmax(axis=1)
        assert np.all(np.abs(q[np.arange(q.shape[0]), arg]) == 127), "q8_0: amax element is not +-127"
        dn, qn = _q8_split(o.quantize_q8_0(-x))
        assert np.array_equal(dn, dbits) and np.array_equal(qn, -q), "q8_0: not sign symmetric"
        d2, q2 = _q8_split(o.quantize_q8_0((x * np.float32(4.0)).astype(np.float32)))
        assert np.array_equal(q2, q), "q8_0: codes change under x*4"
        assert np.array_equal(d2.view(np.float16).astype(np.float64), 4 * d), "q8_0: d does not scale by 4"
    z = o.quantize_q8_0(np.zeros(64, np.float32))
    assert not z.any(), "q8_0: zero block must be all-zero bytes"


# ---------------------------------------------------------------- q4_K ----

def pin_q4k_scale_golden(o):
    lines = _golden_lines("q4k_scale_decode.txt")
    for i in range(0, len(lines), 3):
        s = np.array([int(t, 16) for t in lines[i].split(":")[1].split()], np.uint8)
        sc = [int(t) for t in lines[i + 1].split(":")[1].split()]
        m = [int(t) for t in lines[i + 2].split(":")[1].split()]
        for j in range(8):
            assert o.scale_min(s, j) == (sc[j], m[j]), f"scale decode case {i // 3} j={j}"


def pin_q4k_pack_roundtrip(o):
    """Decoding the test's own packing of random 6-bit fields gives them back,
    and packing is onto all 96 bits (random bytes re-pack to themselves)."""
    g = np.random.default_rng(3)
    for _ in range(300):
        sc, m = g.integers(0, 64, 8), g.integers(0, 64, 8)
        s = np.frombuffer(pack_scales(sc, m), np.uint8)
        got = [o.scale_min(s, j) for j in range(8)]
        assert got == list(zip(sc.tolist(), m.tolist())), "scale decode != inverse of packing"
        raw = g.integers(0, 256, 12).astype(np.uint8)
        dec = [o.scale_min(raw, j) for j in range(8)]
        assert pack_scales([a for a, _ in dec], [b for _, b in dec]) == raw.tobytes(), "packing not a bijection"


def pin_q4k_isolation(o):
    """One nonzero nibble at each of the 256 positions, dmin = 0 and distinct
    scales: the decoded block is zero except d*sc_j*q at that position."""
    sc = [1, 9, 17, 25, 33, 41, 49, 63]
    m = [5, 6, 7, 8, 50, 60, 62, 63]
    for i in range(256):
        q = np.zeros(256, np.int64)
        q[i] = 1 + i % 15
        w = o.dequant_q4k(np.frombuffer(make_sb(0.5, 0.0, sc, m, q), np.uint8))
        want = np.zeros(256)
        want[i] = 0.5 * sc[i // 32] * q[i]
        assert np.array_equal(w, want), f"isolation at weight {i}"


def pin_q4k_min_closed_form(o):
    """All-zero nibbles: y_r = -sum_s dmin_s sum_j m_j * sum_{i in (s,j)} x_i."""
    g = np.random.default_rng(5)
    W = RandomQ4K(g, 7, 768, zero_q=True)
    X = RandomQ8(g, 768)
    y, sa = o.gemv_q4k(W.bytes, 7, 768, X.bytes)
    xs = X.values.reshape(3, 8, 32).sum(axis=2)                  # [sb, j]
    dmin = np.vectorize(f16_value)(W.dmin)
    want = -(dmin[:, :, None] * W.mn * xs[None]).sum(axis=(1, 2))
    assert np.all(np.abs(y - want) <= 1e-9 * sa + np.abs(want) * 2.0 ** -23), "min closed form"


def pin_q4k_values(o):
    """Dequantized weights equal the values the test built the blocks from."""
    g = np.random.default_rng(9)
    W = RandomQ4K(g, 3, 512)
    assert np.array_equal(o.dequant_q4k(W.bytes), W.values.ravel()), "dequant != built values"


def _fsum_gemv(Wv, xv, k):
    y, sa = [], []
    for r in range(Wv.shape[0]):
        p = Wv[r, :k] * xv[:k]
        y.append(math.fsum(p))
        sa.append(math.fsum(np.abs(p)))
    return np.array(y), np.array(sa)


def pin_gemv_bruteforce(o):
    """Exact-rounded (fsum) brute force on tiny shapes, including a K that is
    not a multiple of 256 (rows padded to whole super-blocks)."""
    g = np.random.default_rng(13)
    for m, k in [(1, 256), (2, 512), (3, 768), (17, 256), (5, 1408), (4, 1024)]:
        W, X = RandomQ4K(g, m, k), RandomQ8(g, k)
        y, sa = o.gemv_q4k(W.bytes, m, k, X.bytes)
        yr, sar = _fsum_gemv(W.values, X.values, k)
        for r in range(m):
            assert abs(float(y[r]) - yr[r]) <= _ulp32(yr[r]), f"gemv {m}x{k} row {r}: {y[r]} vs {yr[r]}"
        assert np.allclose(sa, sar, rtol=1e-12), "s_abs"
        rows = np.array([m - 1, 0], np.int64)
        y2, _ = o.gemv_q4k(W.bytes, m, k, X.bytes, rows=rows)
        assert np.array_equal(y2, y[rows]), "row-sampled gemv differs"


def pin_gemv_onehot(o):
    """A one-hot activation extracts one weight column: y = W[:, i] * x_i."""
    g = np.random.default_rng(17)
    W = RandomQ4K(g, 9, 512)
    for i in (0, 31, 32, 63, 64, 255, 256, 300, 511):
        x = np.zeros(512, np.float32)
        x[i] = 1.0
        xq = o.quantize_q8_0(x)
        xi = f16_value(1.0 / 127.0) * 127
        y, _ = o.gemv_q4k(W.bytes, 9, 512, xq)
        assert np.array_equal(y, (W.values[:, i] * xi).astype(np.float32)), f"one-hot column {i}"


def pin_gemv_golden(o):
    """The hand-worked super-block example."""
    lines = dict(ln.split(":", 1) for ln in _golden_lines("q4k_gemv_worked.txt"))
    sb = np.array([int(t, 16) for t in lines["sb"].split()], np.uint8)
    dbits = [int(t, 16) for t in lines["act_d_bits"].split()]
    q = np.zeros((8, 32), np.int64)
    for b in (0, 1, 7):
        q[b] = [int(t) for t in lines[f"act_q_block{b}"].split()]
    xq = np.frombuffer(b"".join(np.uint16(dbits[b]).tobytes() + q[b].astype(np.int8).tobytes()
                                for b in range(8)), np.uint8)
    y, sa = o.gemv_q4k(sb, 1, 256, xq)
    assert float(y[0]) == float(lines["y"]) and float(sa[0]) == float(lines["s_abs"]), f"worked example: {y} {sa}"
    isum, ysum = o.isums_q4k(sb, 1, 256, xq)
    assert isum[0].tolist() == [int(t) for t in lines["isum"].split()], "worked example isum"
    assert ysum.tolist() == [int(t) for t in lines["ysum"].split()], "worked example ysum"


def pin_isums(o):
    """Integer block sums against an integer brute force over the test's own
    nibbles and codes, and special cases (all nibbles 1 -> isum = ysum)."""
    g = np.random.default_rng(19)
    W, X = RandomQ4K(g, 3, 768), RandomQ8(g, 768)
    isum, ysum = o.isums_q4k(W.bytes, 3, 768, X.bytes)
    q4 = W.q.reshape(3, 24, 32)
    q8 = X.q.reshape(24, 32)
    assert np.array_equal(isum, (q4 * q8[None]).sum(axis=2)), "isum brute force"
    assert np.array_equal(ysum, q8.sum(axis=1)), "ysum brute force"
    ones = RandomQ4K(g, 1, 512)
    ones.q[:] = 1
    blob = b"".join(make_sb(ones.d[0, s], ones.dmin[0, s], ones.sc[0, s], ones.mn[0, s], ones.q[0, s])
                    for s in range(2))
    X2 = RandomQ8(g, 512)
    i2, y2 = o.isums_q4k(np.frombuffer(blob, np.uint8), 1, 512, X2.bytes)
    assert np.array_equal(i2[0], y2), "all-ones nibbles: isum != ysum"


# ------------------------------------------------------------- q4_0 ----

def pin_q4_0_golden(o):
    """The hand-worked q4_0 block."""
    lines = dict(ln.split(":", 1) for ln in _golden_lines("q4_0_gemv_worked.txt"))
    blk = np.array([int(t, 16) for t in lines["block"].split()], np.uint8)
    q = np.array([int(t) for t in lines["act_q"].split()], np.int64)
    xq = np.frombuffer(np.uint16(int(lines["act_d_bits"], 16)).tobytes() + q.astype(np.int8).tobytes(), np.uint8)
    y, sa = o.gemv_q4_0(blk, 1, 32, xq)
    assert float(y[0]) == float(lines["y"]) and float(sa[0]) == float(lines["s_abs"]), f"worked example: {y} {sa}"
    assert int(o.isums_q4_0(blk, 1, 32, xq)[0, 0]) == int(lines["isum"]), "worked example isum"


def pin_q4_0_isolation(o):
    """One quant away from 8 (weight 0) at each of the 32 positions: the
    decoded block is zero except d*(q - 8) there (pins which nibble of which
    byte holds each weight, and the offset)."""
    for i in range(32):
        q = np.full(32, 8, np.int64)
        q[i] = (i * 5) % 16 if (i * 5) % 16 != 8 else 3
        w = o.dequant_q4_0(np.frombuffer(make_q4_0(0.5, q), np.uint8))
        want = np.zeros(32)
        want[i] = 0.5 * (q[i] - 8)
        assert np.array_equal(w, want), f"q4_0 isolation at weight {i}"


def pin_q4_0_values(o):
    """Dequantized weights equal the values the test built the blocks from."""
    g = np.random.default_rng(47)
    W = RandomQ4_0(g, 3, 256)
    assert np.array_equal(o.dequant_q4_0(W.bytes), W.values.ravel()), "q4_0 dequant != built values"


def pin_q4_0_closed_forms(o):
    """All quants 8: every weight is 0, so y = 0 and S_abs = 0 exactly.  All
    quants 0: w = -8d, so y_r = -8 * sum_b d_b * sum_{i in b} x_i."""
    g = np.random.default_rng(53)
    X = RandomQ8(g, 320)
    W8 = RandomQ4_0(g, 4, 320, q_fill=8)
    y, sa = o.gemv_q4_0(W8.bytes, 4, 320, X.bytes)
    assert np.all(y == 0) and np.all(sa == 0), "all-8 quants"
    W0 = RandomQ4_0(g, 5, 320, q_fill=0)
    y, sa = o.gemv_q4_0(W0.bytes, 5, 320, X.bytes)
    d = np.vectorize(f16_value)(W0.d)
    want = -8.0 * (d * X.values.reshape(10, 32).sum(axis=1)[None]).sum(axis=1)
    assert np.all(np.abs(y - want) <= 1e-9 * sa + np.abs(want) * 2.0 ** -23), "all-0 quants closed form"


def pin_q4_0_gemv_bruteforce(o):
    """Exact-rounded (fsum) brute force on tiny shapes; row sampling."""
    g = np.random.default_rng(59)
    for m, k in [(1, 32), (2, 64), (3, 256), (17, 96), (4, 512)]:
        W, X = RandomQ4_0(g, m, k), RandomQ8(g, k)
        y, sa = o.gemv_q4_0(W.bytes, m, k, X.bytes)
        yr, sar = _fsum_gemv(W.values, X.values, k)
        for r in range(m):
            assert abs(float(y[r]) - yr[r]) <= _ulp32(yr[r]), f"q4_0 gemv {m}x{k} row {r}: {y[r]} vs {yr[r]}"
        assert np.allclose(sa, sar, rtol=1e-12), "q4_0 s_abs"
        rows = np.array([m - 1, 0], np.int64)
        y2, _ = o.gemv_q4_0(W.bytes, m, k, X.bytes, rows=rows)
        assert np.array_equal(y2, y[rows]), "row-sampled q4_0 gemv differs"


def pin_q4_0_isums(o):
    """Integer block sums against an integer brute force over the test's own
    nibbles and codes; all quants 8 give 8 times the activation sums."""
    g = np.random.default_rng(61)
    W, X = RandomQ4_0(g, 3, 256), RandomQ8(g, 256)
    isum = o.isums_q4_0(W.bytes, 3, 256, X.bytes)
    q8 = X.q.reshape(8, 32)
    assert np.array_equal(isum, (W.q * q8[None]).sum(axis=2)), "q4_0 isum brute force"
    W8 = RandomQ4_0(g, 1, 256, q_fill=8)
    assert np.array_equal(o.isums_q4_0(W8.bytes, 1, 256, X.bytes)[0], 8 * q8.sum(axis=1)), "all-8 isum"


# ----------------------------------------------------- q8_0 weights (lm) ----

def pin_q8_gemv(o):
    g = np.random.default_rng(23)
    m, k = 6, 320
    Wq = [RandomQ8(g, k) for _ in range(m)]
    w = np.stack([a.bytes for a in Wq])
    X = RandomQ8(g, k)
    y, sa = o.gemv_q8_0(w, m, k, X.bytes)
    Wv = np.stack([a.values for a in Wq])
    yr, sar = _fsum_gemv(Wv, X.values, k)
    for r in range(m):
        assert abs(float(y[r]) - yr[r]) <= _ulp32(yr[r]), "q8_0 gemv brute force"
    assert np.allclose(sa, sar, rtol=1e-12)
    isum = o.isums_q8_0(w, m, k, X.bytes)
    want = (np.stack([a.q for a in Wq]) * X.q[None]).sum(axis=2)
    assert np.array_equal(isum, want), "q8_0 isum brute force"
    ones = np.frombuffer(b"".join(make_q8(1.0, np.ones(32)) for _ in range(k // 32)), np.uint8)
    y1, _ = o.gemv_q8_0(ones, 1, k, X.bytes)
    assert abs(float(y1[0]) - math.fsum(X.values)) <= _ulp32(math.fsum(X.values)), "ones row = sum x"


# ---------------------------------------------------------------- glue ----

def pin_rmsnorm(o):
    # constant vector: mean(x^2) = c^2, scale = f32(1/sqrt(c^2 + eps)), y = c * scale in f32
    # (n chosen so that the f64 sum of the n equal squares is exact)
    for c, n in ((3.0, 64), (-0.5, 7), (1e-3, 16)):
        y = o.rmsnorm(np.full(n, c, np.float32), 1e-6)
        cf = np.float32(c)
        scale = np.float32(1.0 / math.sqrt(float(cf) * float(cf) + float(np.float32(1e-6))))
        assert np.all(y == cf * scale), "constant vector"
    n = 256
    e = np.zeros(n, np.float32)
    e[17] = 1.0
    y = o.rmsnorm(e, 0.0)
    assert y[17] == np.float32(16.0) and np.count_nonzero(y) == 1, "one-hot: sqrt(n)"
    x = np.random.default_rng(29).standard_normal(1000).astype(np.float32)
    y1, y2 = o.rmsnorm(x, 0.0), o.rmsnorm(x * np.float32(8), 0.0)
    assert np.array_equal(y1, y2), "scale invariance"
    assert abs(float(np.mean(y1.astype(np.float64) ** 2)) - 1.0) < 1e-6, "unit mean square"


def pin_swiglu(o):
    s1 = math.e / (1 + math.e)                                  # sigmoid(1)
    y = o.swiglu(np.float32([1.0, 0.0, 50.0, -3.0, 2.0, 5.0, 1.0, 0.0]))
    assert y[0] == np.float32(1.0 * s1 * 2.0), "silu(1)*2: gate first, up second"
    assert y[1] == 0.0, "silu(0) = 0"
    assert y[2] == np.float32(50.0), "silu(50) = 50 to f32 precision"
    assert y[3] == 0.0, "up = 0 gives 0"
    g = np.random.default_rng(31).standard_normal(500).astype(np.float32)
    a = o.swiglu(np.concatenate([g, np.ones(500, np.float32)])).astype(np.float64)
    b = o.swiglu(np.concatenate([-g, np.ones(500, np.float32)])).astype(np.float64)
    assert np.allclose(a - b, g, rtol=0, atol=4e-7 * (1 + np.abs(g))), "silu(x) - silu(-x) = x"


def pin_softmax(o):
    assert np.all(o.softmax(np.zeros(8, np.float32)) == np.float32(0.125)), "uniform"
    p = o.softmax(np.float32([0.0, math.log(3.0)]))
    assert np.allclose(p, [0.25, 0.75], rtol=1e-7), "[0, ln 3]"
    lg = np.random.default_rng(37).standard_normal(8).astype(np.float32)
    p = o.softmax(lg)
    assert abs(float(p.astype(np.float64).sum()) - 1) < 1e-6 and np.all(np.diff(p[np.argsort(lg)]) >= 0), "sum/order"


# ---------------------------------------------------------- decode step ----

class _TinyModel:
    hidden, qkv_rows, inter, vocab, eps = 256, 384, 512, 96, 1e-6

    def __init__(self, n_layers):
        self.n_layers = n_layers


def _tiny_weights(g, model):
    L = model.n_layers
    return {
        "qkv": [RandomQ4K(g, model.qkv_rows, model.hidden).bytes for _ in range(L)],
        "o": [RandomQ4K(g, model.hidden, getattr(model, "o_k", 0) or model.hidden).bytes for _ in range(L)],
        "gu": [RandomQ4K(g, 2 * model.inter, model.hidden).bytes for _ in range(L)],
        "down": [RandomQ4K(g, model.hidden, model.inter).bytes for _ in range(L)],
        "lm": np.stack([RandomQ8(g, model.hidden).bytes for _ in range(model.vocab)]),
    }


def pin_chain_structure(o):
    """The decode step is the stated composition of the pinned stages: a
    two-layer step recomposed here from those stages, step by step."""
    g = np.random.default_rng(41)
    model = _TinyModel(2)
    W = _tiny_weights(g, model)
    h = g.standard_normal(model.hidden).astype(np.float32)
    out = o.chain(model, W, h, traces=True)
    H, I = model.hidden, model.inter
    q8s = []
    for l in range(2):
        a = o.quantize_q8_0(o.rmsnorm(h, model.eps)); q8s.append(a)
        t, _ = o.gemv_q4k(W["qkv"][l], model.qkv_rows, H, a)
        b = o.quantize_q8_0(o.rmsnorm(t[:H], model.eps)); q8s.append(b)
        ov, _ = o.gemv_q4k(W["o"][l], H, H, b)
        c = o.quantize_q8_0(o.rmsnorm(ov, model.eps)); q8s.append(c)
        gu, _ = o.gemv_q4k(W["gu"][l], 2 * I, H, c)
        gg = o.quantize_q8_0(o.swiglu(gu)); q8s.append(gg)
        h, _ = o.gemv_q4k(W["down"][l], H, I, gg)
    z = o.quantize_q8_0(o.rmsnorm(h, model.eps)); q8s.append(z)
    logits, sa = o.gemv_q8_0(W["lm"], model.vocab, H, z)
    assert np.array_equal(out["logits"], logits), "chain logits != composition"
    assert np.array_equal(out["s_abs"], sa), "chain s_abs"
    assert np.array_equal(out["q8_trace"], np.concatenate(q8s)), "chain q8 trace"


class _TinyModelQ4_0(_TinyModel):
    weight_format = "q4_0"


class _TinyRank(_TinyModel):
    """One rank's share of a tensor-parallel split: fewer QKV rows than the
    hidden width, and O taking only the first o_k of them."""
    hidden, qkv_rows, inter, vocab, o_k = 512, 320, 512, 64, 256


def pin_chain_structure_o_k(o):
    """With O's K set below the hidden width, O normalizes and consumes only
    the first o_k QKV outputs (its (hidden x o_k) matrix), and the trace keeps
    that q8_0 vector in a hidden-wide slot, zero past its o_k/32 blocks; the
    rest of the step is unchanged."""
    g = np.random.default_rng(71)
    model = _TinyRank(2)
    W = _tiny_weights(g, model)
    h = g.standard_normal(model.hidden).astype(np.float32)
    out = o.chain(model, W, h, traces=True)
    H, I, K = model.hidden, model.inter, model.o_k
    q8s = []
    for l in range(2):
        a = o.quantize_q8_0(o.rmsnorm(h, model.eps)).ravel(); q8s.append(a)
        t, _ = o.gemv_q4k(W["qkv"][l], model.qkv_rows, H, a)
        assert t.size == model.qkv_rows
        b = o.quantize_q8_0(o.rmsnorm(t[:K], model.eps)).ravel()
        q8s.append(np.concatenate([b, np.zeros((H - K) // 32 * 34, np.uint8)]))
        ov, _ = o.gemv_q4k(W["o"][l], H, K, b)
        c = o.quantize_q8_0(o.rmsnorm(ov, model.eps)).ravel(); q8s.append(c)
        gu, _ = o.gemv_q4k(W["gu"][l], 2 * I, H, c)
        gg = o.quantize_q8_0(o.swiglu(gu)).ravel(); q8s.append(gg)
        h, _ = o.gemv_q4k(W["down"][l], H, I, gg)
    z = o.quantize_q8_0(o.rmsnorm(h, model.eps)).ravel(); q8s.append(z)
    logits, _ = o.gemv_q8_0(W["lm"], model.vocab, H, z)
    assert np.array_equal(out["logits"], logits), "rank chain logits != composition"
    assert np.array_equal(out["q8_trace"], np.concatenate(q8s)), "rank chain q8 trace"


def pin_chain_structure_q4_0(o):
    """With q4_0 layer weights the step is the same composition, every layer
    GEMV taken with the q4_0 product."""
    g = np.random.default_rng(67)
    model = _TinyModelQ4_0(2)
    H, I, L = model.hidden, model.inter, 2
    W = {"qkv": [RandomQ4_0(g, model.qkv_rows, H).bytes for _ in range(L)],
         "o": [RandomQ4_0(g, H, H).bytes for _ in range(L)],
         "gu": [RandomQ4_0(g, 2 * I, H).bytes for _ in range(L)],
         "down": [RandomQ4_0(g, H, I).bytes for _ in range(L)],
         "lm": np.stack([RandomQ8(g, H).bytes for _ in range(model.vocab)])}
    h = g.standard_normal(H).astype(np.float32)
    out = o.chain(model, W, h, traces=True)
    for l in range(L):
        t, _ = o.gemv_q4_0(W["qkv"][l], model.qkv_rows, H, o.quantize_q8_0(o.rmsnorm(h, model.eps)))
        ov, _ = o.gemv_q4_0(W["o"][l], H, H, o.quantize_q8_0(o.rmsnorm(t[:H], model.eps)))
        gu, _ = o.gemv_q4_0(W["gu"][l], 2 * I, H, o.quantize_q8_0(o.rmsnorm(ov, model.eps)))
        h, _ = o.gemv_q4_0(W["down"][l], H, I, o.quantize_q8_0(o.swiglu(gu)))
    logits, _ = o.gemv_q8_0(W["lm"], model.vocab, H, o.quantize_q8_0(o.rmsnorm(h, model.eps)))
    assert np.array_equal(out["logits"], logits), "q4_0 chain logits != composition"


# ------------------------------------------------------- routed experts ----

def pin_moe(o):
    """Softmax-weighted combine of per-expert FFNs: a dominant logit selects
    one expert's FFN; identical ids collapse to one FFN (weights sum to 1);
    permuting the slots permutes nothing in the result; each slot equals the
    FFN recomposed from the pinned stages."""
    g = np.random.default_rng(43)
    E, H, I = 5, 256, 320
    gu = [RandomQ4K(g, 2 * I, H).bytes for _ in range(E)]
    dn = [RandomQ4K(g, H, I).bytes for _ in range(E)]
    gu_all, dn_all = np.concatenate([a.ravel() for a in gu]), np.concatenate([a.ravel() for a in dn])
    gb, db = gu[0].size, dn[0].size
    x = g.standard_normal(H).astype(np.float32)
    ids = np.array([3, 0, 4, 1], np.int32)
    lg = g.standard_normal(4).astype(np.float32)
    y, ys, c = o.moe_token(gu_all, gb, dn_all, db, ids, lg, x, H, I)
    xq = o.quantize_q8_0(x)
    for s, e in enumerate(ids):
        t, _ = o.gemv_q4k(gu[e], 2 * I, H, xq)
        want, _ = o.gemv_q4k(dn[e], H, I, o.quantize_q8_0(o.swiglu(t)))
        assert np.array_equal(ys[s], want), f"slot {s} FFN"
    assert np.array_equal(c, o.softmax(lg)), "combine weights are the softmax"
    p = np.array([2, 0, 3, 1])
    y2, _, _ = o.moe_token(gu_all, gb, dn_all, db, ids[p], lg[p], x, H, I)
    scale = np.abs(ys).max(axis=0)
    assert np.all(np.abs(y2 - y) <= 1e-6 * scale + 1e-30), "slot permutation"
    y3, ys3, _ = o.moe_token(gu_all, gb, dn_all, db, ids, np.float32([60, -60, -60, -60]), x, H, I)
    assert np.array_equal(y3, ys3[0]), "dominant logit selects slot 0"
    y4, ys4, _ = o.moe_token(gu_all, gb, dn_all, db, np.full(4, 2, np.int32), lg, x, H, I)
    assert np.all(np.abs(y4 - ys4[0]) <= 1e-6 * np.abs(ys4[0]) + 1e-30), "identical ids collapse"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
