"""GPU parity of the single kernels against the oracle, through the C ABI.

Integer and byte results must be bit-exact (q8_0 bytes, int32 block sums);
float outputs must satisfy |y - y_ref| <= 1e-3 * sum_i |w_i x_i| + 1e-6 per
row, with sum_i |w_i x_i| computed by the oracle in f64.  Small shapes span
several tiles and a ragged tail and are compared in full; full-size shapes
run exactly as the benchmark launches them and are compared in full too,
every row against the oracle (its row function spread over host threads).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_helpers import check_tolerance, log, oracle_gemv_parallel, q8_code_diff, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_quantized_gemv_amd import binding
    binding.lib()
    return binding


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.fixture(scope="module")
def pool():
    with ThreadPoolExecutor(16) as p:
        yield p


def _synth():
    from block_quantized_gemv_amd import synth
    return synth


# ------------------------------------------------------------------ q8_0 ----

def test_quantize_bytes_exact(mq, o):
    synth = _synth()
    cases = {
        "normal 3x3584": synth.normal_f32(10, (1,), (3, 3584)),
        "large scale": synth.normal_f32(10, (2,), (2, 1024)) * np.float32(1e3),
        "subnormal scales": synth.normal_f32(10, (3,), (1, 2048)) * np.float32(1e-4),
        "mixed zero blocks": np.where(np.arange(4096) % 96 < 32, 0.0,
                                      synth.normal_f32(10, (4,), (4096,))).astype(np.float32)[None],
    }
    lines = [ln for ln in open(__file__.replace("test_gpu_kernels.py", "golden/q8_0_rounding.txt"))
             if ln.startswith("x:")]
    cases["hand-worked ties"] = np.array([[float(t) for ln in lines for t in ln.split(":")[1].split()]],
                                         np.float32)
    for name, x in cases.items():
        log(f"quantize case: {name} {x.shape}")
        got = to_host(mq.mq_quantize_q8_0(to_dev(x)))
        want = o.quantize_q8_0(x).ravel()
        assert np.array_equal(got, want), f"{name}: {q8_code_diff(got, want)}"


def _random_quantize_cases(count=12, seed=20261205):
    """Seeded random activation rows: length 32..131072 in blocks of 32
    (log-uniform), magnitude 10^-6..10^6, and a random share of all-zero
    blocks."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        nb = int(np.exp(g.uniform(0.0, np.log(4096.0))))
        cases.append((32 * max(nb, 1), float(10.0 ** g.uniform(-6.0, 6.0)), float(g.uniform(0.0, 0.5)), 500 + i))
    return cases


RANDOM_QUANT = _random_quantize_cases()


@pytest.mark.parametrize("k,scale,zero_share,seed", RANDOM_QUANT,
                         ids=[f"k{k}-s{sc:.0e}-z{z:.2f}" for k, sc, z, _ in RANDOM_QUANT])
def test_quantize_random_rows(mq, o, k, scale, zero_share, seed):
    """q8_0 bytes of seeded random rows equal the oracle's, byte for byte."""
    synth = _synth()
    x = synth.normal_f32(seed, (k,), (k,)) * np.float32(scale)
    zero = np.random.default_rng(seed).random(k // 32) < zero_share
    x = np.where(np.repeat(zero, 32), np.float32(0.0), x).astype(np.float32)
    got = to_host(mq.mq_quantize_q8_0(to_dev(x[None])))
    want = o.quantize_q8_0(x[None]).ravel()
    assert np.array_equal(got, want), f"k={k} scale={scale:.1e}: {q8_code_diff(got, want)}"


# ------------------------------------------------------------- q4_K GEMV ----

SMALL_SHAPES = [(1, 256), (3, 512), (17, 768), (1024, 1024), (1023, 1024), (1025, 3584), (4097, 1536),
                (333, 4864), (64, 18944), (5, 2048), (7, 6400), (130, 4096)]


@pytest.mark.parametrize("m,k", SMALL_SHAPES)
def test_gemv_q4k_small(mq, o, m, k):
    synth = _synth()
    log(f"q4_K GEMV {m}x{k}")
    w = synth.q4k_matrix(100 + k, (synth.KEY_MATRIX, m), m, k)
    x = synth.normal_f32(100 + k, (synth.KEY_COLUMNS, m), (k,))
    xq = o.quantize_q8_0(x).ravel()
    wd, xd = to_dev(w), to_dev(xq)
    y = to_host(mq.mq_gemv_q4k_q8(wd, xd, m, k))
    yd, isum, ysum = mq.mq_debug_gemv_q4k_q8_isums(wd, xd, m, k)
    yd, isum, ysum = to_host(yd), to_host(isum), to_host(ysum)
    ri, ry = o.isums_q4k(w, m, k, xq)
    assert np.array_equal(isum, ri), f"int32 block sums differ at {np.argwhere(isum != ri)[:4]}"
    assert np.array_equal(ysum, ry), "activation sums differ"
    assert np.array_equal(yd.view(np.uint32), y.view(np.uint32)), "dump build changed the float result"
    y_ref, s_abs = o.gemv_q4k(w, m, k, xq)
    check_tolerance(y, y_ref, s_abs, f"{m}x{k}")


def test_gemv_worked_example(mq, o):
    """The hand-worked super-block: y = -61.5 exactly."""
    from oracle_pins import _golden_lines
    lines = dict(ln.split(":", 1) for ln in _golden_lines("q4k_gemv_worked.txt"))
    sb = np.array([int(t, 16) for t in lines["sb"].split()], np.uint8)
    dbits = [int(t, 16) for t in lines["act_d_bits"].split()]
    q = np.zeros((8, 32), np.int64)
    for b in (0, 1, 7):
        q[b] = [int(t) for t in lines[f"act_q_block{b}"].split()]
    xq = np.frombuffer(b"".join(np.uint16(dbits[b]).tobytes() + q[b].astype(np.int8).tobytes()
                                for b in range(8)), np.uint8)
    y, isum, ysum = mq.mq_debug_gemv_q4k_q8_isums(to_dev(sb), to_dev(xq), 1, 256)
    assert float(to_host(y)[0]) == -61.5
    assert to_host(isum)[0].tolist() == [int(t) for t in lines["isum"].split()]
    assert to_host(ysum).tolist() == [int(t) for t in lines["ysum"].split()]


FULL_SHAPES = [("7B qkv", 4608, 3584), ("7B o", 3584, 3584), ("7B gate/up", 37888, 3584),
               ("7B down", 3584, 18944), ("0.5B qkv", 1280, 1024), ("0.5B gate/up", 9728, 1024),
               ("0.5B down", 1024, 4864), ("expert gate/up", 2816, 2048), ("expert down", 2048, 1536)]


@pytest.mark.parametrize("name,m,k", FULL_SHAPES, ids=[s[0] for s in FULL_SHAPES])
def test_gemv_q4k_full_size(mq, o, pool, name, m, k):
    synth = _synth()
    log(f"q4_K GEMV full size {name} {m}x{k}")
    w = synth.q4k_matrix(2, (synth.KEY_MATRIX, m, k), m, k)
    x = synth.normal_f32(2, (synth.KEY_COLUMNS, m, k), (k,))
    xq_dev = mq.mq_quantize_q8_0(to_dev(x))
    xq = o.quantize_q8_0(x).ravel()
    assert np.array_equal(to_host(xq_dev), xq)
    y = to_host(mq.mq_gemv_q4k_q8(to_dev(w), xq_dev, m, k))
    y_ref, s_abs = oracle_gemv_parallel(o.gemv_q4k, w, m, k, xq, pool=pool)
    check_tolerance(y, y_ref, s_abs, name)


def test_matrix_of_4_gib_or_more(mq, o):
    """A 4.32 GB q4_K matrix (30M rows of K = 256, over the 4 GiB that one
    launch addresses with 32-bit offsets): the one-column GEMV splits it into
    row blocks under 4 GiB; the batched GEMV at n = 5 takes the vector kernels,
    because the matrix-core kernel's offsets cannot hold it, and the
    matrix-core hook refuses it.  The matrix is a seeded 1M-row block repeated
    on the device, so row r is block row r mod 1M: the rows at and around the
    row-block boundary, both ends and a random sample are compared with the
    oracle, and column 0 of the batched result with the one-column GEMV."""
    import torch
    synth = _synth()
    base_rows, reps, k, n = 1_000_000, 30, 256, 5
    m = base_rows * reps
    wb = synth.q4k_matrix(7, (synth.KEY_MATRIX, base_rows, k), base_rows, k)
    assert m * wb.shape[1] >= 1 << 32
    w = to_dev(wb).reshape(-1).repeat(reps)
    x = synth.normal_f32(7, (synth.KEY_COLUMNS, 8, k), (8, k))
    xq8 = mq.mq_quantize_q8_0(to_dev(x))
    xq_host = o.quantize_q8_0(x).reshape(8, -1)
    assert np.array_equal(to_host(xq8), xq_host.ravel())
    col = (k // 32) * 34
    log(f"q4_K GEMV over {m * 144 / 1e9:.2f} GB ({m} rows)")
    y1 = mq.mq_gemv_q4k_q8(w, xq8[:col], m, k)
    y5 = mq.mq_gemv_q4k_q8_batched(w, xq8[:n * col], m, k, n)
    torch.cuda.synchronize()
    assert torch.equal(y1, y5[:, 0]), "batched column 0 differs from the one-column GEMV"
    step = ((1 << 32) - 1) // 144          # rows per launch under 32-bit offsets
    g = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, step - 1, step, step + 1, m - 2, m - 1], g.integers(0, m, 200)]))
    yh = to_host(y5)[rows]
    for c in range(n):
        y_ref, s_abs = o.gemv_q4k(wb, base_rows, k, xq_host[c], rows=rows % base_rows)
        check_tolerance(yh[:, c], y_ref, s_abs, f"4.32 GB matrix, column {c}")
    with pytest.raises(mq.MQError) as e:
        mq.mq_debug_gemv_q4k_batched_path(w, xq8, m, k, 8, 1)
    assert e.value.code == mq.MQ_ERR_SHAPE
    del w, y1, y5
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- batched ----

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8])
def test_batched_small(mq, o, n):
    """301 x 2560, n columns: the batched entry point and the vector
    kernels (path 0), each column against the oracle; the vector kernels'
    columns equal the n = 1 GEMV bit for bit, and so do the entry point's
    wherever it takes the vector kernels (at this size, every n)."""
    synth = _synth()
    m, k = 301, 2560
    w = synth.q4k_matrix(3, (synth.KEY_MATRIX, n), m, k)
    x = synth.normal_f32(3, (synth.KEY_COLUMNS, n), (n, k))
    xq = o.quantize_q8_0(x).reshape(n, -1)
    wd, xd = to_dev(w), to_dev(xq.ravel())
    y = to_host(mq.mq_gemv_q4k_q8_batched(wd, xd, m, k, n))
    yv = to_host(mq.mq_debug_gemv_q4k_batched_path(wd, xd, m, k, n, 0))
    for c in range(n):
        y_ref, s_abs = o.gemv_q4k(w, m, k, xq[c])
        check_tolerance(y[:, c], y_ref, s_abs, f"batched n={n} col {c}")
        check_tolerance(yv[:, c], y_ref, s_abs, f"batched n={n} col {c}, vector kernels")
        y1 = to_host(mq.mq_gemv_q4k_q8(wd, to_dev(xq[c]), m, k))
        assert np.array_equal(y1.view(np.uint32), yv[:, c].copy().view(np.uint32)), f"col {c} differs from n = 1"
        if mq.mq_gemv_batched_path(m, k, n) == 0:
            assert np.array_equal(y1.view(np.uint32), y[:, c].copy().view(np.uint32))


def _exact_friendly(rng, m, k, n):
    """q4_K weights with d = 1 and dmin = 1/2 (random six-bit scales and
    mins, random nibbles) and q8_0 columns with power-of-two scales 2^-2 ..
    2^-6 (random codes in [-127, 127]): every weight d*sc*q - dmin*m is a
    multiple of 1/2 below 2^10 and every activation d8*code a multiple of
    2^-6 below 2^5, so every product is a multiple of 2^-7 below 2^15 and,
    for k <= 65536, every partial sum stays below 2^38 units of 2^-7: any
    summation order in f64 gives the exact dot product."""
    nsb = k // 256
    wb = rng.integers(0, 256, size=(m * nsb, 144), dtype=np.uint8)
    wb[:, 0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    wb[:, 2:4] = np.frombuffer(np.float16(0.5).tobytes(), np.uint8)
    nb = k // 32
    xb = np.empty((n * nb, 34), np.uint8)
    d = np.float16(2.0) ** -rng.integers(2, 7, size=n * nb)
    xb[:, 0:2] = d.astype(np.float16).view(np.uint8).reshape(-1, 2)
    xb[:, 2:] = rng.integers(-127, 128, size=(n * nb, 32)).astype(np.int8).view(np.uint8)
    return wb.ravel(), xb.reshape(n, -1)


# (m, k, n): ragged and single 16-row tiles, one super-block, uneven k ranges; (24, 65536, 8) plans one
# super-block per k range (256 ranges), (1, 4096, 8) a single row at n = 8
MFMA_SMALL = [(1, 256, 2), (15, 512, 8), (17, 768, 3), (16, 256 * 40, 8), (301, 2560, 8), (64, 18944, 5),
              (1000, 4864, 8), (33, 256 * 33, 4), (2049, 1024, 6), (200, 4096, 7), (24, 65536, 8), (1, 4096, 8)]


@pytest.mark.parametrize("m,k,n", MFMA_SMALL)
def test_batched_matrix_cores_exact(mq, o, m, k, n):
    """The matrix-core path on inputs whose dot products f64 forms exactly
    in any order (_exact_friendly): every output equals the oracle's bit
    for bit, so any error in the integer sums, the scale and min decoding,
    the sub-block split or the k splits would show.  Shapes: ragged row
    tiles, one super-block, k split into several ranges (and not evenly)."""
    rng = np.random.default_rng(1000 + m + k + n)
    w, xq = _exact_friendly(rng, m, k, n)
    y = to_host(mq.mq_debug_gemv_q4k_batched_path(to_dev(w), to_dev(xq.ravel()), m, k, n, 1))
    for c in range(n):
        y_ref, _ = o.gemv_q4k(w, m, k, xq[c])
        bad = y[:, c].copy().view(np.uint32) != y_ref.view(np.uint32)
        assert not bad.any(), (f"{m}x{k} n={n} col {c}: {bad.sum()} rows differ, first {np.argmax(bad)}: "
                               f"{y[bad, c][:3]} vs {y_ref[bad][:3]}")


BATCH_SHAPES = [("qkv", 4608, 3584), ("o", 3584, 3584), ("gate/up", 37888, 3584), ("down", 3584, 18944)]


def _single_pass(m, k, n):
    """Whether the n-column GEMV stages all its columns in LDS (one pass over
    K per row, the n = 1 kernel's order) rather than taking split-k."""
    return n * ((k // 32 // 2 + 63) // 64) * 6144 <= 64 * 1024


@pytest.mark.parametrize("n", [2, 4, 8])
@pytest.mark.parametrize("name,m,k", BATCH_SHAPES, ids=[s[0] for s in BATCH_SHAPES])
def test_batched_full_size(mq, o, pool, name, m, k, n):
    """7B-class shapes, n columns, every row of every column against the
    oracle, through the batched entry point (the matrix cores at n = 8, and
    at n = 4 on the gate/up and down matrices) and through the vector
    kernels; the vector kernels' columns also against the n = 1 kernel, bit
    for bit where both take one pass over K (the same per-row order), within
    the gate where they split K."""
    synth = _synth()
    from block_quantized_gemv_amd import workloads
    seed = workloads.BATCHED.seed
    log(f"batched {name} {m}x{k} n={n}")
    w = synth.q4k_matrix(seed, (synth.KEY_MATRIX, m, k), m, k)
    x = synth.normal_f32(seed, (synth.KEY_COLUMNS, n, k), (n, k))
    xq_dev = mq.mq_quantize_q8_0(to_dev(x))
    xq = o.quantize_q8_0(x).reshape(n, -1)
    assert np.array_equal(to_host(xq_dev), xq.ravel())
    wd = to_dev(w)
    y = to_host(mq.mq_gemv_q4k_q8_batched(wd, xq_dev, m, k, n))
    yv = to_host(mq.mq_debug_gemv_q4k_batched_path(wd, xq_dev, m, k, n, 0))
    for c in range(n):
        y_ref, s_abs = oracle_gemv_parallel(o.gemv_q4k, w, m, k, xq[c], pool=pool)
        check_tolerance(y[:, c], y_ref, s_abs, f"{name} n={n} col {c}")
        check_tolerance(yv[:, c], y_ref, s_abs, f"{name} n={n} col {c}, vector kernels")
        y1 = to_host(mq.mq_gemv_q4k_q8(wd, xq_dev[c * xq.shape[1]:(c + 1) * xq.shape[1]], m, k))
        same = float(np.mean(y1.view(np.uint32) == yv[:, c].copy().view(np.uint32)))
        log(f"    col {c}: vector kernels bit-identical to the n=1 kernel on {same:.4f} of rows")
        if _single_pass(m, k, n):
            assert same == 1.0, f"{name} n={n} col {c}: batched column differs from the n = 1 kernel"


def _sweep_cases(count=36, large=8, seed=20261202):
    """Seeded random (format, m, k, n) beyond the hand-picked lists: m from 1
    to 6000 (log-uniform), k a multiple of 256 up to 12288, n from 1 to 8,
    every third case q4_0 (the long-k ones split k); then `large` q4_K cases
    of 2000 to 8000 rows, k from 4096 and n from 5, which the size rule
    sends to the matrix cores where it can."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        m = int(np.exp(g.uniform(0.0, np.log(6000.0))))
        k = 256 * int(g.integers(1, 49))
        n = int(g.integers(1, 9))
        cases.append(("q4_0" if i % 3 == 0 else "q4_K", max(m, 1), k, n))
    for _ in range(large):
        cases.append(("q4_K", int(g.integers(2000, 8001)), 256 * int(g.integers(16, 49)), int(g.integers(5, 9))))
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("fmt,m,k,n", SWEEP, ids=[f"{f}-{m}x{k}-n{n}" for f, m, k, n in SWEEP])
def test_random_shape_sweep(mq, o, pool, fmt, m, k, n):
    """Every column of every row against the oracle, through the batched
    entry point (whichever family the size rule picks) and, for q4_K, the
    vector kernels and the matrix cores forced; the vector kernels' columns
    equal the n = 1 kernel's bit for bit where they make one pass over k."""
    synth = _synth()
    log(f"sweep {fmt} {m}x{k} n={n} (batched path {mq.mq_gemv_batched_path(m, k, n, fmt)})")
    seed = 7000 + m + k + n
    q4k = fmt == "q4_K"
    w = (synth.q4k_matrix if q4k else synth.q4_0_matrix)(seed, (synth.KEY_MATRIX, m, k), m, k)
    x = synth.normal_f32(seed, (synth.KEY_COLUMNS, n, k), (n, k))
    xq = o.quantize_q8_0(x).reshape(n, -1)
    wd, xd = to_dev(w), to_dev(xq.ravel())
    ref = o.gemv_q4k if q4k else o.gemv_q4_0
    single = mq.mq_gemv_q4k_q8 if q4k else mq.mq_gemv_q4_0_q8
    y = to_host((mq.mq_gemv_q4k_q8_batched if q4k else mq.mq_gemv_q4_0_q8_batched)(wd, xd, m, k, n))
    forced = {}
    if q4k:
        forced["vector kernels"] = to_host(mq.mq_debug_gemv_q4k_batched_path(wd, xd, m, k, n, 0))
        if n >= 2:
            forced["matrix cores"] = to_host(mq.mq_debug_gemv_q4k_batched_path(wd, xd, m, k, n, 1))
    for c in range(n):
        y_ref, s_abs = oracle_gemv_parallel(ref, w, m, k, xq[c], pool=pool)
        check_tolerance(y[:, c], y_ref, s_abs, f"{fmt} {m}x{k} n={n} col {c}")
        for what, yf in forced.items():
            check_tolerance(yf[:, c], y_ref, s_abs, f"{fmt} {m}x{k} n={n} col {c}, {what}")
        y1 = to_host(single(wd, to_dev(xq[c]), m, k))
        check_tolerance(y1, y_ref, s_abs, f"{fmt} {m}x{k} col {c}, n = 1 kernel")
        yv = forced.get("vector kernels", y if mq.mq_gemv_batched_path(m, k, n, fmt) == 0 else None)
        if yv is not None and _single_pass(m, k, n):
            assert np.array_equal(y1.view(np.uint32), yv[:, c].copy().view(np.uint32)), \
                f"{fmt} {m}x{k} n={n} col {c}: vector kernels differ from the n = 1 kernel"


# ------------------------------------------------------------- q4_0 GEMV ----

Q4_0_SMALL = [(1, 256), (3, 512), (17, 768), (1023, 1024), (1025, 3584), (333, 4864), (64, 18944), (130, 4096)]


def _codes_sum(xq):
    return np.asarray(xq, np.uint8).reshape(-1, 34)[:, 2:].view(np.int8).astype(np.int32).sum(axis=1)


@pytest.mark.parametrize("m,k", Q4_0_SMALL)
def test_gemv_q4_0_small(mq, o, m, k):
    synth = _synth()
    log(f"q4_0 GEMV {m}x{k}")
    w = synth.q4_0_matrix(200 + k, (synth.KEY_MATRIX, m), m, k)
    x = synth.normal_f32(200 + k, (synth.KEY_COLUMNS, m), (k,))
    xq = o.quantize_q8_0(x).ravel()
    wd, xd = to_dev(w), to_dev(xq)
    y = to_host(mq.mq_gemv_q4_0_q8(wd, xd, m, k))
    yd, isum, ysum = (to_host(t) for t in mq.mq_debug_gemv_q4_0_q8_isums(wd, xd, m, k))
    ri = o.isums_q4_0(w, m, k, xq)
    assert np.array_equal(isum, ri), f"int32 block sums differ at {np.argwhere(isum != ri)[:4]}"
    assert np.array_equal(ysum, _codes_sum(xq)), "activation sums differ"
    assert np.array_equal(yd.view(np.uint32), y.view(np.uint32)), "dump build changed the float result"
    y_ref, s_abs = o.gemv_q4_0(w, m, k, xq)
    check_tolerance(y, y_ref, s_abs, f"q4_0 {m}x{k}")


def test_gemv_q4_0_worked_example(mq, o):
    """The hand-worked q4_0 block (y = 32.0, isum = 1600), first of eight in
    one 256-weight group; the other seven blocks have d = 0 and meet zero
    activation blocks."""
    from oracle_pins import _golden_lines
    lines = dict(ln.split(":", 1) for ln in _golden_lines("q4_0_gemv_worked.txt"))
    blk = bytes(int(t, 16) for t in lines["block"].split())
    w = np.frombuffer(blk + bytes([0, 0] + [0x5A] * 16) * 7, np.uint8)
    q = np.array([int(t) for t in lines["act_q"].split()], np.int8)
    xq = np.frombuffer(np.uint16(int(lines["act_d_bits"], 16)).tobytes() + q.tobytes() + bytes(34 * 7), np.uint8)
    y, isum, _ = mq.mq_debug_gemv_q4_0_q8_isums(to_dev(w), to_dev(xq), 1, 256)
    assert float(to_host(y)[0]) == float(lines["y"])
    assert int(to_host(isum)[0, 0]) == int(lines["isum"])


Q4_0_FULL = [("0.5B qkv", 1280, 1024), ("0.5B o", 1024, 1024), ("0.5B gate/up", 9728, 1024),
             ("0.5B down", 1024, 4864), ("7B gate/up", 37888, 3584), ("7B down", 3584, 18944)]


@pytest.mark.parametrize("name,m,k", Q4_0_FULL, ids=[s[0] for s in Q4_0_FULL])
def test_gemv_q4_0_full_size(mq, o, pool, name, m, k):
    synth = _synth()
    log(f"q4_0 GEMV full size {name} {m}x{k}")
    w = synth.q4_0_matrix(5, (synth.KEY_MATRIX, m, k), m, k)
    x = synth.normal_f32(5, (synth.KEY_COLUMNS, m, k), (k,))
    xq_dev = mq.mq_quantize_q8_0(to_dev(x))
    xq = o.quantize_q8_0(x).ravel()
    assert np.array_equal(to_host(xq_dev), xq)
    y = to_host(mq.mq_gemv_q4_0_q8(to_dev(w), xq_dev, m, k))
    y_ref, s_abs = oracle_gemv_parallel(o.gemv_q4_0, w, m, k, xq, pool=pool)
    check_tolerance(y, y_ref, s_abs, name)


@pytest.mark.parametrize("n,m,k", [(2, 301, 2560), (5, 130, 1024), (8, 301, 2560), (8, 515, 18944)])
def test_batched_q4_0(mq, o, n, m, k):
    """Every column against the oracle (k = 18944 at n = 8 takes split-k),
    and against the n = 1 kernel."""
    synth = _synth()
    log(f"q4_0 batched {m}x{k} n={n}")
    w = synth.q4_0_matrix(6, (synth.KEY_MATRIX, n, k), m, k)
    x = synth.normal_f32(6, (synth.KEY_COLUMNS, n, k), (n, k))
    xq = o.quantize_q8_0(x).reshape(n, -1)
    wd, xd = to_dev(w), to_dev(xq.ravel())
    y = to_host(mq.mq_gemv_q4_0_q8_batched(wd, xd, m, k, n))
    for c in range(n):
        y_ref, s_abs = o.gemv_q4_0(w, m, k, xq[c])
        check_tolerance(y[:, c], y_ref, s_abs, f"q4_0 batched n={n} col {c}")
        y1 = to_host(mq.mq_gemv_q4_0_q8(wd, to_dev(xq[c]), m, k))
        check_tolerance(y1, y_ref, s_abs, f"q4_0 n=1 col {c}")
        if _single_pass(m, k, n):
            assert np.array_equal(y1.view(np.uint32), y[:, c].copy().view(np.uint32)), f"col {c} differs from n = 1"


# ------------------------------------------------------------ edge cases ----

@pytest.mark.parametrize("fmt", ["q4_K", "q4_0"])
@pytest.mark.parametrize("n", [1, 2])
def test_gemv_split_k_large_k(mq, o, fmt, n):
    """k = 65536: one column no longer fits in LDS, so even n = 1 takes the
    split-k kernel and the ordered second pass."""
    synth = _synth()
    m, k = 37, 65536
    log(f"{fmt} split-k {m}x{k} n={n}")
    mat = synth.q4_0_matrix if fmt == "q4_0" else synth.q4k_matrix
    gemv = o.gemv_q4_0 if fmt == "q4_0" else o.gemv_q4k
    w = mat(7, (synth.KEY_MATRIX, n, k), m, k)
    x = synth.normal_f32(7, (synth.KEY_COLUMNS, n, k), (n, k))
    xq = o.quantize_q8_0(x).reshape(n, -1)
    wd, xd = to_dev(w), to_dev(xq.ravel())
    if n == 1:
        f = mq.mq_gemv_q4_0_q8 if fmt == "q4_0" else mq.mq_gemv_q4k_q8
        y = to_host(f(wd, xd, m, k))[:, None]
    else:
        f = mq.mq_gemv_q4_0_q8_batched if fmt == "q4_0" else mq.mq_gemv_q4k_q8_batched
        y = to_host(f(wd, xd, m, k, n))
    for c in range(n):
        y_ref, s_abs = gemv(w, m, k, xq[c])
        check_tolerance(y[:, c], y_ref, s_abs, f"{fmt} split-k col {c}")


def test_gemv_zero_activation(mq, o):
    """An all-zero activation quantizes to zero blocks (d = 0, q = 0); every
    product is then exactly zero, so every output is +0 or -0."""
    synth = _synth()
    m, k = 515, 3584
    xq = o.quantize_q8_0(np.zeros(k, np.float32)).ravel()
    assert not xq.any()
    xd = to_dev(xq)
    for name, w, f in (("q4_K", synth.q4k_matrix(8, (synth.KEY_MATRIX, 1), m, k), mq.mq_gemv_q4k_q8),
                       ("q4_0", synth.q4_0_matrix(8, (synth.KEY_MATRIX, 2), m, k), mq.mq_gemv_q4_0_q8),
                       ("q8_0", synth.q8_0_matrix(8, (synth.KEY_MATRIX, 3), m, k), mq.mq_gemv_q8_0_q8)):
        y = to_host(f(to_dev(w), xd, m, k))
        assert np.all(y == 0.0), f"{name}: nonzero output for a zero activation"


# ------------------------------------------------------------ q8_0 lm_head ----

@pytest.mark.parametrize("m,k", [(1, 64), (5, 128), (130, 1024), (67, 3584), (1000, 2048)])
def test_gemv_q8_0_small(mq, o, m, k):
    synth = _synth()
    w = synth.q8_0_matrix(5, (synth.KEY_MATRIX, m, k), m, k)
    x = synth.normal_f32(5, (synth.KEY_COLUMNS, m, k), (k,))
    xq = o.quantize_q8_0(x).ravel()
    y, isum = mq.mq_debug_gemv_q8_0_q8_isums(to_dev(w), to_dev(xq), m, k)
    assert np.array_equal(to_host(isum), o.isums_q8_0(w, m, k, xq)), "int32 block sums differ"
    y2 = to_host(mq.mq_gemv_q8_0_q8(to_dev(w), to_dev(xq), m, k))
    assert np.array_equal(to_host(y).view(np.uint32), y2.view(np.uint32))
    y_ref, s_abs = o.gemv_q8_0(w, m, k, xq)
    check_tolerance(y2, y_ref, s_abs, f"q8_0 {m}x{k}")


def _random_q8_0_shapes(count=10, seed=20261206):
    """Seeded random q8_0 GEMV shapes: m 1..200000 (log-uniform), k a
    multiple of 64 up to 8192."""
    g = np.random.default_rng(seed)
    return [(max(int(np.exp(g.uniform(0.0, np.log(200000.0)))), 1), 64 * int(g.integers(1, 129)))
            for _ in range(count)]


RANDOM_Q8_0 = _random_q8_0_shapes()


@pytest.mark.parametrize("m,k", RANDOM_Q8_0)
def test_gemv_q8_0_random_shapes(mq, o, pool, m, k):
    """Every row of seeded random q8_0 GEMV shapes within the gate of the
    oracle; the debug build's y equals the production y bit for bit."""
    synth = _synth()
    log(f"q8_0 GEMV {m}x{k}")
    w = synth.q8_0_matrix(6, (synth.KEY_MATRIX, m, k), m, k)
    x = synth.normal_f32(6, (synth.KEY_COLUMNS, m, k), (k,))
    xq = o.quantize_q8_0(x).ravel()
    wd, xd = to_dev(w), to_dev(xq)
    y = to_host(mq.mq_gemv_q8_0_q8(wd, xd, m, k))
    yd, _ = mq.mq_debug_gemv_q8_0_q8_isums(wd, xd, m, k)
    assert np.array_equal(to_host(yd).view(np.uint32), y.view(np.uint32))
    y_ref, s_abs = oracle_gemv_parallel(o.gemv_q8_0, w, m, k, xq, pool=pool)
    check_tolerance(y, y_ref, s_abs, f"q8_0 {m}x{k}")


@pytest.mark.parametrize("name,m,k", [("0.5B lm_head", 151552, 1024), ("7B lm_head", 152064, 3584)])
def test_gemv_q8_0_full_size(mq, o, pool, name, m, k):
    synth = _synth()
    log(f"q8_0 GEMV full size {name}")
    w = synth.q8_0_matrix(1, (synth.KEY_LM_HEAD, k), m, k)
    x = synth.normal_f32(1, (synth.KEY_COLUMNS, k), (k,))
    xq = o.quantize_q8_0(x).ravel()
    y = to_host(mq.mq_gemv_q8_0_q8(to_dev(w), to_dev(xq), m, k))
    y_ref, s_abs = oracle_gemv_parallel(o.gemv_q8_0, w, m, k, xq, pool=pool)
    check_tolerance(y, y_ref, s_abs, name)


# ------------------------------------------------------------------- glue ----

def test_rmsnorm_quantize(mq, o):
    synth = _synth()
    for k, scale in ((1024, 1.0), (3584, 37.0), (3584, 1e-3), (18944, 2e4)):
        x = synth.normal_f32(6, (k,), (k,)) * np.float32(scale)
        got = to_host(mq.mq_rmsnorm_quantize_q8_0(to_dev(x), 1e-6))
        want = o.quantize_q8_0(o.rmsnorm(x, 1e-6)).ravel()
        ds, dq, mx = q8_code_diff(got, want)
        log(f"  rmsnorm k={k} scale={scale}: scale diffs {ds}, code diffs {dq}, max {mx}")
        assert ds == 0 and dq <= 2 and mx <= 1, (ds, dq, mx)


def test_swiglu_quantize_padded(mq, o):
    synth = _synth()
    for inter, n_cols, k_pad in ((1408, 8, 1536), (4864, 1, 4864), (18944, 1, 18944)):
        gu = synth.normal_f32(7, (inter, n_cols), (n_cols, 2 * inter)) * np.float32(4.0)
        got = to_host(mq.mq_swiglu_quantize_q8_0(to_dev(gu), inter, n_cols, k_pad)).reshape(n_cols, -1)
        nbi = inter // 32 * 34
        for c in range(n_cols):
            want = o.quantize_q8_0(o.swiglu(gu[c])).ravel()
            ds, dq, mx = q8_code_diff(got[c, :nbi], want)
            assert ds == 0 and dq <= 2 and mx <= 1, (inter, c, ds, dq, mx)
            assert not got[c, nbi:].any(), "pad blocks must be zero"
        log(f"  swiglu inter={inter} cols={n_cols} pad={k_pad}: ok")


# ---------------------------------------------------------------- grouped ----

@pytest.fixture(scope="module")
def experts():
    synth = _synth()
    from block_quantized_gemv_amd import workloads
    wl = workloads.MOE
    log("generating 64 experts")
    gu = np.stack([synth.q4k_matrix(wl.seed, (synth.KEY_EXPERT, e, 0), 2 * wl.inter, wl.hidden)
                   for e in range(wl.n_experts)])
    dn = np.stack([synth.q4k_matrix(wl.seed, (synth.KEY_EXPERT, e, 1), wl.hidden, wl.inter)
                   for e in range(wl.n_experts)])
    return wl, gu, dn


def test_grouped_gate_up_and_down(mq, o, experts):
    wl, gu, dn = experts
    synth = _synth()
    import torch
    H, I, KP = wl.hidden, wl.inter, wl.k_pad
    gub, dnb = gu[0].nbytes, dn[0].nbytes
    gu_d, dn_d = to_dev(gu.ravel()), to_dev(dn.ravel())
    ids_all, logits_all = synth.routing(wl.seed, 4, wl.n_experts, wl.n_sel)
    for t in range(4):
        ids = ids_all[t]
        x = synth.normal_f32(wl.seed, (synth.KEY_TOKEN_X, t), (H,))
        xq = o.quantize_q8_0(x).ravel()
        y_gu, _ = mq.mq_gemv_q4k_grouped(gu_d, gub, wl.n_experts, to_dev(ids), to_dev(xq), 0, 2 * I, H)
        y_gu = to_host(y_gu)
        gu_ref = []
        for s, e in enumerate(ids):
            y_ref, s_abs = o.gemv_q4k(gu[e], 2 * I, H, xq)
            check_tolerance(y_gu[s], y_ref, s_abs, f"token {t} slot {s} gate/up (expert {e})")
            gu_ref.append(y_ref)
        # down with per-slot activations (the oracle's own SwiGLU of its own
        # gate/up values) and the combine
        g = np.stack([o.quantize_q8_0(o.swiglu(gu_ref[s])).ravel() for s in range(wl.n_sel)])
        gpad = np.zeros((wl.n_sel, KP // 32 * 34), np.uint8)
        gpad[:, :g.shape[1]] = g
        comb = o.softmax(logits_all[t])
        y_dn, y_out = mq.mq_gemv_q4k_grouped(dn_d, dnb, wl.n_experts, to_dev(ids), to_dev(gpad.ravel()),
                                             gpad.shape[1], H, KP, combine=to_dev(comb))
        y_dn, y_out = to_host(y_dn), to_host(y_out)
        acc = np.zeros(H)
        sab = np.zeros(H)
        for s, e in enumerate(ids):
            y_ref, s_abs = o.gemv_q4k(dn[e], H, I, g[s])
            check_tolerance(y_dn[s], y_ref, s_abs, f"token {t} slot {s} down")
            assert np.array_equal(y_dn[s].view(np.uint32), y_ref.view(np.uint32)), f"token {t} slot {s} down bits"
            acc += np.float64(comb[s]) * y_ref.astype(np.float64)
            sab += abs(float(comb[s])) * s_abs
        # the combine: sum_s c_s * y_s in f64 in slot order over the oracle's
        # slot values (equal to the kernel's, asserted above), rounded once
        check_tolerance(y_out, acc, sab, f"token {t} combine")
        assert np.array_equal(y_out, acc.astype(np.float32)), "combine differs from the slot-order f64 sum"
        # one slot against the single-GEMV kernel: identical bits
        single = to_host(mq.mq_gemv_q4k_q8(to_dev(dn[ids[0]].ravel()), to_dev(gpad[0]), H, KP))
        assert np.array_equal(single.view(np.uint32), y_dn[0].copy().view(np.uint32))
    # an out-of-range id is not read: NaN for that slot and the combine
    bad = np.array([3, 64, 5, -1], np.int32)
    y_b, y_o = mq.mq_gemv_q4k_grouped(dn_d, dnb, wl.n_experts, to_dev(bad), to_dev(gpad[:4].ravel()),
                                      gpad.shape[1], H, KP, combine=to_dev(np.full(4, 0.25, np.float32)))
    y_b, y_o = to_host(y_b), to_host(y_o)
    assert np.all(np.isfinite(y_b[0])) and np.all(np.isnan(y_b[1])) and np.all(np.isnan(y_b[3]))
    assert np.all(np.isnan(y_o))
    del torch


def test_grouped_down_combine_kernel(mq, o, experts):
    """y = NULL with a combine runs the slot-parallel combine kernel.  Slot
    columns packed back to back are staged as one vector; a wider stride
    stages them column by column: both give the same bytes, within the
    tolerance of the oracle's per-slot products combined in slot order."""
    wl, gu, dn = experts
    synth = _synth()
    H, I, KP = wl.hidden, wl.inter, wl.k_pad
    dn_d = to_dev(dn.ravel())
    ids_all, logits_all = synth.routing(wl.seed, 2, wl.n_experts, wl.n_sel)
    for t in range(2):
        ids = ids_all[t]
        x = synth.normal_f32(wl.seed, (synth.KEY_TOKEN_X, 100 + t), (wl.n_sel, I))
        g = np.stack([o.quantize_q8_0(x[s]).ravel() for s in range(wl.n_sel)])
        comb = o.softmax(logits_all[t])
        outs = []
        for pad in (0, 34):
            stride = KP // 32 * 34 + pad
            gp = np.zeros((wl.n_sel, stride), np.uint8)
            gp[:, :g.shape[1]] = g
            _, y_out = mq.mq_gemv_q4k_grouped(dn_d, dn[0].nbytes, wl.n_experts, to_dev(ids), to_dev(gp.ravel()),
                                              stride, H, KP, combine=to_dev(comb), want_y=False)
            outs.append(to_host(y_out).copy())
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), "staging layouts disagree"
        acc, sab = np.zeros(H), np.zeros(H)
        for s, e in enumerate(ids):
            y_ref, s_abs = o.gemv_q4k(dn[e], H, I, g[s])
            acc += float(comb[s]) * y_ref.astype(np.float64)
            sab += abs(float(comb[s])) * s_abs
        check_tolerance(outs[0], acc, sab, f"token {t} combine kernel")


# ------------------------------------------------------ measurement probe ----

def test_sync_probes(mq):
    """The grid-barrier probe orders its exchange (every word read back after
    each barrier is the one written before it, flat and per-XCD barriers, with
    and without an exchange), its per-round time is positive and finite, and
    the graph-boundary probe gives a positive time per kernel."""
    for hier in (0, 1):
        for words in (0, 4, 64):
            us, bad = mq.mq_probe_grid_barrier(hier, words, rounds=300)
            log(f"grid barrier hier={hier} words={words}: {us:.3f} us/round")
            assert bad == 0, (hier, words, bad)
            assert 0.0 < us < 1000.0, (hier, words, us)
    us = mq.mq_probe_graph_boundary(n_kernels=50, reps=3)
    log(f"graph boundary: {us:.3f} us/kernel")
    assert 0.0 < us < 1000.0


def test_stream_probe_reads_every_word(mq):
    """The streaming-read probe's XOR over all 32-bit words equals numpy's, for
    sizes that end inside the four-load body and inside the tail loop, and for
    an empty buffer."""
    import torch
    rng = np.random.default_rng(11)
    for n16, wgs in ((0, 0), (1, 0), (4097, 3), (256 * 1024 * 4 * 2 + 12345, 0), (1000003, 700)):
        host = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).cuda() if n16 else torch.empty(0, dtype=torch.int32,
                                                                                   device="cuda")
        got = int(mq.mq_probe_stream_read(buf, workgroups=wgs).cpu().numpy().view(np.uint32)[0])
        want = int(np.bitwise_xor.reduce(host)) if n16 else 0
        assert got == want, (n16, wgs, hex(got), hex(want))
