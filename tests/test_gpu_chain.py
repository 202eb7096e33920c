"""GPU tests of the graph-captured decode step and routed-expert chains.

Replay of a captured graph runs the same kernels with the same arguments as
the eager path, so the two must be byte-identical, over capture plus seven
replays with a different input each step: a frozen host value is correct on
the first replay and wrong from the second ('Part 4 · Lecture 08 —
Graph-Resident Decode', §4).  A/A controls (graph vs graph, eager vs eager)
run first (§5).  Against the oracle the chain is compared end to end at
real widths; its per-stage intermediates are compared to the oracle's own.
"""
import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_helpers import (check_chain_trace, check_tolerance, log, model_weights, oracle_chain_parallel, to_dev,
                         to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available()
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


def _dev_weights(W):
    return {k: ([to_dev(a) for a in v] if isinstance(v, list) else to_dev(v)) for k, v in W.items()}


@pytest.fixture(scope="module")
def small_model():
    """0.5B-class widths, 4 layers (real widths; fewer layers)."""
    from block_quantized_gemv_amd import synth, workloads
    model = dataclasses.replace(workloads.DECODE_05B, n_layers=4)
    W = model_weights(model, 4)
    X = synth.normal_f32(model.seed, (synth.KEY_STEP_INPUTS,), (8, model.hidden))
    return model, W, _dev_weights(W), X


def _run_steps(mq, chain, n, mode, traces=False):
    outs = []
    for _ in range(n):
        logits = to_host(chain.step(mode)).copy()
        if traces:
            q8, f32 = chain.trace()
            outs.append((logits, to_host(q8).copy(), to_host(f32).copy()))
        else:
            outs.append(logits)
    return outs


def _same(u, v):
    return np.array_equal(np.asarray(u).view(np.uint8), np.asarray(v).view(np.uint8))


def test_graph_equals_eager_over_replays(mq, o, small_model):
    """Capture plus 7 replays against the eager path, every intermediate byte
    compared; layer 0's quantized input at each step must be the oracle's
    Q8(RMSNorm(x[step mod 8])), which proves the device counter moved the
    input row on every replay.  (The stand-in step has no residual path, so
    after a few layers its output barely depends on the input; the logits
    alone cannot show the counter advancing.)"""
    model, W, Wd, X = small_model
    xd = to_dev(X)
    keep = mq.MQ_KEEP_INTERMEDIATES
    g = mq.DecodeChain(model, Wd, xd, flags=keep)
    e = mq.DecodeChain(model, Wd, xd, flags=keep | mq.MQ_EAGER_ONLY)
    info = g.info()
    log(f"captured={info['captured']} nodes={info['n_nodes']}")
    assert info["captured"] and info["n_nodes"] == 4 * model.n_layers + 1
    assert not e.info()["captured"]
    # A/A first: two eager runs of one chain object agree with themselves
    e.reset(0)
    a1 = _run_steps(mq, e, 2, mq.MQ_EAGER, traces=True)
    e.reset(0)
    a2 = _run_steps(mq, e, 2, mq.MQ_EAGER, traces=True)
    for u, v in zip(a1, a2):
        assert all(_same(p, q) for p, q in zip(u, v)), "A/A eager mismatch: the test is broken"
    e.reset(0)
    go = _run_steps(mq, g, 8, mq.MQ_GRAPH, traces=True)
    eo = _run_steps(mq, e, 8, mq.MQ_EAGER, traces=True)
    qa_bytes = model.hidden // 32 * 34
    for i, (u, v) in enumerate(zip(go, eo)):
        for part, p, q in zip(("logits", "q8 trace", "f32 trace"), u, v):
            assert _same(p, q), f"graph != eager at step {i} ({part})"
        want_a0 = o.quantize_q8_0(o.rmsnorm(X[i % X.shape[0]], model.eps)).ravel()
        assert _same(u[1][:qa_bytes], want_a0), f"step {i} did not read input row {i % X.shape[0]}"
    assert g.info()["step"] == 8 and e.info()["step"] == 8
    # the graph object can also be stepped eagerly: still identical
    g.reset(3)
    u = to_host(g.step(mq.MQ_EAGER)).copy()
    assert _same(u, go[3][0])
    g.close()
    e.close()


def _fast_vs_exact_glue(mq, model, W_dev, xd, n_steps):
    keep = mq.MQ_KEEP_INTERMEDIATES
    f = mq.DecodeChain(model, W_dev, xd, flags=keep)
    e = mq.DecodeChain(model, W_dev, xd, flags=keep | mq.MQ_EXACT_GLUE)
    of, oe = _run_steps(mq, f, n_steps, mq.MQ_GRAPH, traces=True), _run_steps(mq, e, n_steps, mq.MQ_GRAPH, traces=True)
    for i, (u, v) in enumerate(zip(of, oe)):
        for part, p, q in zip(("logits", "q8 trace", "f32 trace"), u, v):
            assert _same(p, q), f"reciprocal-product glue != division glue at step {i} ({part})"
    f.close()
    e.close()


def test_glue_fast_path_equals_divisions(mq, small_model):
    """The prologues' RMSNorm->q8_0 forms x/denom and n/d as checked
    reciprocal products; forcing the division path everywhere must give the
    same bytes (0.5B widths: one 4-value chunk per thread or less)."""
    model, W, Wd, X = small_model
    _fast_vs_exact_glue(mq, model, Wd, to_dev(X), 4)


def test_glue_fast_path_equals_divisions_7b_width(mq):
    """Same at hidden 3584, where threads hold one or two chunks, plus x
    scaled by 1e-30 and 1e30 (denominators far from 1) and a row of zeros."""
    from block_quantized_gemv_amd import synth, workloads
    model = dataclasses.replace(workloads.DECODE_7B, n_layers=2)
    W = model_weights(model, 2)
    X = synth.normal_f32(model.seed, (synth.KEY_STEP_INPUTS,), (4, model.hidden))
    X[1] *= np.float32(1e-30)
    X[2] *= np.float32(1e30)
    X[3] = 0.0
    _fast_vs_exact_glue(mq, model, _dev_weights(W), to_dev(X), 4)


def test_graph_aa_control(mq, small_model):
    model, W, Wd, X = small_model
    xd = to_dev(X)
    g1, g2 = mq.DecodeChain(model, Wd, xd), mq.DecodeChain(model, Wd, xd)
    o1, o2 = _run_steps(mq, g1, 3, mq.MQ_GRAPH), _run_steps(mq, g2, 3, mq.MQ_GRAPH)
    for u, v in zip(o1, o2):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), "A/A graph mismatch"


def test_span_stamps(mq, small_model):
    """MQ_SPAN_STAMPS: the stamped step gives the same bytes as the plain one;
    every GEMV kernel's stamp pair is filled (start < end), the kernels follow
    one another (each starts after the previous one's last wave ended, within
    the counter's 10 ns tick), every step overwrites the pairs, a read
    changes nothing, a clear resets them, and the chain refuses a wrong pair
    count or a chain without the flag."""
    model, W, Wd, X = small_model
    xd = to_dev(X)
    plain, stamped = mq.DecodeChain(model, Wd, xd), mq.DecodeChain(model, Wd, xd, flags=mq.MQ_SPAN_STAMPS)
    n = 4 * model.n_layers + 1
    assert stamped.n_stamped == n
    prev = None
    for _ in range(3):
        assert _same(to_host(plain.step()), to_host(stamped.step()))
        st = stamped.read_stamps().astype(np.int64)
        assert st.shape == (n, 2)
        assert (st[:, 1] > st[:, 0]).all(), st
        assert (st[1:, 0] >= st[:-1, 1] - 1).all(), "kernels of one replay overlap"
        span_us = (st[-1, 1] - st[0, 0]) * 0.01
        assert 0 < span_us < 10000, span_us
        if prev is not None:
            assert st[0, 0] > prev[-1, 1], "a step did not overwrite the previous step's stamps"
        prev = st
    assert np.array_equal(stamped.read_stamps().astype(np.int64), prev)   # a read changes nothing
    stamped.clear_stamps()              # the device-side clear
    st = stamped.read_stamps()
    assert (st[:, 0] == np.iinfo(np.uint64).max).all() and (st[:, 1] == 0).all()
    buf = np.zeros((n, 2), dtype=np.uint64)
    L = mq.lib()
    assert L.mq_chain_read_stamps(stamped.handle, buf.ctypes.data, n - 1, None) == mq.MQ_ERR_SHAPE
    assert L.mq_chain_read_stamps(plain.handle, buf.ctypes.data, n, None) == mq.MQ_ERR_ARG
    plain.close()
    stamped.close()


def test_capture_failure_falls_back_to_eager(mq, small_model):
    model, W, Wd, X = small_model
    xd = to_dev(X)
    ref = mq.DecodeChain(model, Wd, xd)
    mq.mq_test_set_fault(mq.MQ_FAULT_CAPTURE)
    try:
        f = mq.DecodeChain(model, Wd, xd)
    finally:
        mq.mq_test_set_fault(mq.MQ_FAULT_NONE)
    assert not f.info()["captured"]
    for i in range(4):
        u, v = to_host(ref.step()).copy(), to_host(f.step()).copy()
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), f"fallback differs at step {i}"


def test_lazy_capture_on_third_graph_step(mq, small_model):
    """The capture policy of '07 · R3' §2: no graph at creation or after two
    MQ_GRAPH steps, capture at the third, replays after; every step is
    byte-identical to an eager-only chain on the same inputs, and an
    eager-only chain never captures however often it is stepped."""
    model, W, Wd, X = small_model
    xd = to_dev(X)
    lazy = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_LAZY_CAPTURE)
    eager = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_EAGER_ONLY)
    assert not lazy.info()["captured"]
    assert lazy.capture_stats() == {"graph_steps": 0, "capture_ms": 0.0}
    for i in range(8):
        u = to_host(lazy.step(mq.MQ_GRAPH)).copy()
        v = to_host(eager.step(mq.MQ_GRAPH)).copy()
        assert _same(u, v), f"lazy chain differs from the eager one at step {i}"
        assert lazy.info()["captured"] == (i >= 2), f"step {i}"
    st = lazy.capture_stats()
    assert st["graph_steps"] == 8 and st["capture_ms"] > 0
    info = lazy.info()
    assert info["n_nodes"] == 4 * model.n_layers + 1 and info["step"] == 8
    assert not eager.info()["captured"] and eager.capture_stats()["capture_ms"] == 0.0
    log(f"lazy capture took {st['capture_ms']:.2f} ms")
    # without the flag the chain pays for its capture at creation
    assert mq.DecodeChain(model, Wd, xd).capture_stats()["capture_ms"] > 0


def test_read_logits_pinned_and_pageable(mq, small_model):
    model, W, Wd, X = small_model
    g = mq.DecodeChain(model, Wd, to_dev(X))
    for i in range(3):
        ref = to_host(g.step()).copy()
        assert _same(g.read_logits(), ref), f"pinned readback, step {i}"
        assert _same(g.read_logits(pageable=True), ref), f"pageable readback, step {i}"
    out = np.empty(model.vocab, np.float32)
    assert g.read_logits(out=out) is out
    assert mq.lib().mq_chain_read_logits(g.handle, out.ctypes.data, model.vocab - 1, 0, None) == mq.MQ_ERR_SHAPE


def test_host_logits_copy_in_the_graph(mq, small_model):
    """MQ_HOST_LOGITS: the step's last node copies the logits into the chain's
    pinned buffer.  The buffer is poisoned before every step, so each check
    proves that step's copy ran; graph and eager steps alike, byte-identical
    to an eager-only chain."""
    import torch
    model, W, Wd, X = small_model
    xd = to_dev(X)
    h = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_HOST_LOGITS)
    e = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_EAGER_ONLY)
    info = h.info()
    assert info["captured"] and info["n_nodes"] == 4 * model.n_layers + 2
    view = h.host_logits()
    assert view is not None and view.shape == (model.vocab,)
    for i in range(8):
        view[:] = np.nan
        dev_logits = h.step(mq.MQ_EAGER if i == 5 else mq.MQ_GRAPH)
        torch.cuda.synchronize()
        ref = to_host(e.step(mq.MQ_EAGER)).copy()
        assert _same(view, ref), f"host copy differs at step {i}"
        assert _same(to_host(dev_logits), ref), f"device logits differ at step {i}"
    # pinning failure: no host copy and no copy node; the chain still steps
    mq.mq_test_set_fault(mq.MQ_FAULT_PINNED_ALLOC)
    try:
        f = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_HOST_LOGITS)
    finally:
        mq.mq_test_set_fault(mq.MQ_FAULT_NONE)
    assert f.host_logits() is None and f.info()["n_nodes"] == 4 * model.n_layers + 1
    e.reset(0)
    assert _same(to_host(f.step()).copy(), to_host(e.step(mq.MQ_EAGER)).copy())


def _chain_vs_oracle(mq, o, pool, model, n_layers, n_inputs=2, flags=0):
    """The chain's trace against the oracle's own step, stage by stage: every
    q8_0 vector byte-identical, every GEMV output within the per-row gate,
    the logits within the gate; and, as DESIGN claims for these seeded
    inputs, every f32 value bit-identical (the f64 fixup makes each product
    exact, so GPU and oracle round the same sums)."""
    from block_quantized_gemv_amd import synth
    m = dataclasses.replace(model, n_layers=n_layers)
    log(f"generating {m.name} x{n_layers} layers")
    W = model_weights(m, n_layers)
    X = synth.normal_f32(m.seed, (synth.KEY_STEP_INPUTS,), (n_inputs, m.hidden))
    Wd = _dev_weights(W)
    ch = mq.DecodeChain(m, Wd, to_dev(X), flags=mq.MQ_KEEP_INTERMEDIATES | flags)
    for step in range(n_inputs):
        logits = to_host(ch.step()).copy()
        q8t, f32t = ch.trace()
        q8t, f32t = to_host(q8t), to_host(f32t)
        log(f"oracle step {step}")
        ref_logits, s_abs, rq8, rf32, rsabs = oracle_chain_parallel(o, m, W, X[step], n_layers, pool)
        same = check_chain_trace(m, n_layers, q8t, f32t, rq8, rf32, rsabs, f"{m.name} step {step}")
        _, exact = check_tolerance(logits, ref_logits, s_abs, f"{m.name} logits step {step}")
        assert same == 1.0 and exact == 1.0, "an intermediate or a logit is not bit-identical to the oracle's"
    ch.close()


def test_chain_05b_full_depth_vs_oracle(mq, o, pool):
    from block_quantized_gemv_amd import workloads
    _chain_vs_oracle(mq, o, pool, workloads.DECODE_05B, workloads.DECODE_05B.n_layers)


def test_chain_7b_real_width_vs_oracle(mq, o, pool):
    from block_quantized_gemv_amd import workloads
    _chain_vs_oracle(mq, o, pool, workloads.DECODE_7B, 2, n_inputs=1)


def test_chain_7b_full_depth_vs_oracle(mq, o, pool):
    """The benchmark's configuration: all 28 layers and the lm_head."""
    from block_quantized_gemv_amd import workloads
    _chain_vs_oracle(mq, o, pool, workloads.DECODE_7B, workloads.DECODE_7B.n_layers, n_inputs=1)


def test_chain_tp8_rank_full_depth_vs_oracle(mq, o, pool):
    """One rank of the 7B-class step split eight ways (QKV 576 rows, O taking
    the first 512 of them, gate/up 5120 rows, down K = 2560, lm_head 19008
    rows), all 28 layers, collectives left out: the same stage-by-stage parity."""
    from block_quantized_gemv_amd import workloads
    _chain_vs_oracle(mq, o, pool, workloads.DECODE_7B_TP8, workloads.DECODE_7B_TP8.n_layers, n_inputs=1)


def test_chain_05b_q4_0_full_depth_vs_oracle(mq, o, pool):
    """The pages' measured 0.5B model format: q4_0 layer weights, all 24 layers."""
    from block_quantized_gemv_amd import workloads
    _chain_vs_oracle(mq, o, pool, workloads.DECODE_05B_Q4_0, 24)


def _random_chain_dims(count=16, seed=20261203):
    """Seeded random decode-step shapes: hidden 256..3072, inter 256..10240
    log-uniform (from a few gate/up output blocks to more than two per CU,
    so the split of surplus blocks varies), QKV rows from O's K up to 2048 more, O's K
    the whole hidden vector or a prefix of it, 1..3 layers, a vocabulary of
    1..20000 rows, both weight formats."""
    from block_quantized_gemv_amd import workloads
    g = np.random.default_rng(seed)
    dims = []
    for i in range(count):
        h = 256 * int(g.integers(1, 13))
        o_k = 0 if i % 2 == 0 else 256 * int(g.integers(1, h // 256 + 1))
        dims.append(workloads.DecodeModel(
            name=f"random step {i}", hidden=h, n_layers=int(g.integers(1, 4)),
            qkv_rows=(o_k or h) + 4 * int(g.integers(0, 513)), inter=256 * int(np.exp(g.uniform(0.0, np.log(40.0)))),
            vocab=int(g.integers(1, 20001)), seed=300 + i, weight_format="q4_0" if i % 4 == 3 else "q4_K",
            o_k=o_k))
    return dims


RANDOM_DIMS = _random_chain_dims()


@pytest.mark.parametrize("model", RANDOM_DIMS, ids=[f"{m.weight_format}-h{m.hidden}-i{m.inter}-q{m.qkv_rows}-"
                                                    f"ok{m.o_k}-L{m.n_layers}-v{m.vocab}" for m in RANDOM_DIMS])
def test_chain_random_dims_vs_oracle(mq, o, pool, model):
    """The stage-by-stage parity of the full-size steps on seeded random
    shapes: every q8_0 vector byte-identical, every f32 intermediate and
    logit bit-identical to the oracle's step, over two steps."""
    _chain_vs_oracle(mq, o, pool, model, model.n_layers)


def test_q4_0_chain_graph_equals_eager(mq):
    from block_quantized_gemv_amd import synth, workloads
    model = dataclasses.replace(workloads.DECODE_05B_Q4_0, n_layers=3)
    W = model_weights(model, 3)
    Wd = _dev_weights(W)
    xd = to_dev(synth.normal_f32(model.seed, (synth.KEY_STEP_INPUTS,), (8, model.hidden)))
    g = mq.DecodeChain(model, Wd, xd)
    e = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_EAGER_ONLY)
    assert g.info()["captured"] and g.info()["n_nodes"] == 4 * 3 + 1
    for i in range(8):
        u, v = to_host(g.step()).copy(), to_host(e.step(mq.MQ_EAGER)).copy()
        assert _same(u, v), f"q4_0 graph != eager at step {i}"


def test_unfused_glue_chain_vs_oracle(mq, o, pool):
    """The unfused measurement arm (glue kernels between q8_0-input GEMVs)
    computes the same step: 0.5B, all layers, against the oracle."""
    from block_quantized_gemv_amd import workloads
    _chain_vs_oracle(mq, o, pool, workloads.DECODE_05B, workloads.DECODE_05B.n_layers, flags=mq.MQ_UNFUSED_GLUE)


def test_unfused_glue_chain_graph_equals_eager(mq, small_model):
    model, W, Wd, X = small_model
    xd = to_dev(X)
    g = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_UNFUSED_GLUE)
    e = mq.DecodeChain(model, Wd, xd, flags=mq.MQ_UNFUSED_GLUE | mq.MQ_EAGER_ONLY)
    assert g.info()["captured"] and g.info()["n_nodes"] == 8 * model.n_layers + 2
    for i in range(5):
        u, v = to_host(g.step(mq.MQ_GRAPH)).copy(), to_host(e.step(mq.MQ_EAGER)).copy()
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), f"unfused graph != eager at step {i}"
    assert g.info()["step"] == 5
    g.close()
    e.close()


# ----------------------------------------------------------- routed experts ----

def test_moe_chain(mq, o):
    from block_quantized_gemv_amd import synth, workloads
    wl = workloads.MOE
    H, I = wl.hidden, wl.inter
    T = 12
    log("generating 64 experts")
    gu = np.stack([synth.q4k_matrix(wl.seed, (synth.KEY_EXPERT, e, 0), 2 * I, H) for e in range(wl.n_experts)])
    dn = np.stack([synth.q4k_matrix(wl.seed, (synth.KEY_EXPERT, e, 1), H, I) for e in range(wl.n_experts)])
    ids, logits = synth.routing(wl.seed, T, wl.n_experts, wl.n_sel)
    X = synth.normal_f32(wl.seed, (synth.KEY_TOKEN_X,), (T, H))
    args = (wl.n_experts, wl.n_sel, H, I, to_dev(gu.ravel()), gu[0].nbytes, to_dev(dn.ravel()), dn[0].nbytes,
            to_dev(ids), to_dev(logits), to_dev(X))
    g = mq.MoEChain(*args)
    e = mq.MoEChain(*args, flags=mq.MQ_EAGER_ONLY)
    assert g.info()["captured"] and g.info()["n_nodes"] == 2
    for t in range(T):
        g.step(mq.MQ_GRAPH)
        e.step(mq.MQ_EAGER)
    yg, ye = to_host(g.y_table), to_host(e.y_table)
    assert np.array_equal(yg.view(np.uint32), ye.view(np.uint32)), "graph != eager"
    for t in range(T):
        y_ref, ys_ref, c_ref = o.moe_token(gu.ravel(), gu[0].nbytes, dn.ravel(), dn[0].nbytes, ids[t], logits[t],
                                           X[t], H, I)
        # the combine's own bound: sum_s |c_s| * S_abs of each slot, computed from the oracle's slots
        s_abs = np.zeros(H)
        xq = o.quantize_q8_0(X[t]).ravel()
        for s, ex in enumerate(ids[t]):
            t_gu, _ = o.gemv_q4k(gu[ex], 2 * I, H, xq)
            _, sa = o.gemv_q4k(dn[ex], H, I, o.quantize_q8_0(o.swiglu(t_gu)).ravel())
            s_abs += abs(float(c_ref[s])) * sa
        check_tolerance(yg[t], y_ref, s_abs, f"token {t}")
    assert g.info()["step"] == T
    # a reset points the counter (and the routing the chain keeps for it) at
    # token 5: the row is recomputed with the same bytes
    import torch
    g.y_table[5].zero_()
    g.reset(5)
    g.step(mq.MQ_GRAPH)
    assert np.array_equal(to_host(g.y_table)[5].view(np.uint32), yg[5].view(np.uint32)), "reset to token 5"
    assert g.info()["step"] == 6
    # several tokens per launch: the same bytes, tokens_per_launch tokens per call
    m4 = mq.MoEChain(*args, tokens_per_launch=4)
    assert m4.info()["captured"] and m4.info()["n_nodes"] == 8
    for _ in range(T // 4):
        m4.step(mq.MQ_GRAPH)
    assert m4.info()["step"] == T
    assert np.array_equal(to_host(m4.y_table).view(np.uint32), yg.view(np.uint32)), "4 tokens per launch != 1"
    # lazy capture: the third step captures, the bytes do not change
    lz = mq.MoEChain(*args, flags=mq.MQ_LAZY_CAPTURE, tokens_per_launch=4)
    for i in range(T // 4):
        assert not lz.info()["captured"], f"captured before step {i + 1}"
        lz.step(mq.MQ_GRAPH)
    assert lz.info()["captured"] and lz.info()["step"] == T
    assert np.array_equal(to_host(lz.y_table).view(np.uint32), yg.view(np.uint32)), "lazy capture changed the bytes"


def _random_moe_dims(count=8, seed=20261204):
    """Seeded random routed-expert shapes: 1..64 experts, 1..8 selected
    (at most all of them), hidden 256..4096, expert inter 32..3072 in steps
    of 32 (down's K padded to whole super-blocks where it is not one)."""
    g = np.random.default_rng(seed)
    dims = []
    for i in range(count):
        ne = int(g.integers(1, 65))
        dims.append((ne, int(g.integers(1, min(8, ne) + 1)), 256 * int(g.integers(1, 17)),
                     32 * int(g.integers(1, 97)), 400 + i))
    return dims


RANDOM_MOE = _random_moe_dims()


@pytest.mark.parametrize("n_experts,n_sel,hidden,inter,seed", RANDOM_MOE,
                         ids=[f"e{a}-s{b}-h{c}-i{d}" for a, b, c, d, _ in RANDOM_MOE])
def test_moe_random_dims(mq, o, n_experts, n_sel, hidden, inter, seed):
    """Four tokens of a routed-expert chain on seeded random shapes: graph
    and eager byte-identical, each token within the combine's bound of the
    oracle's token (sum over slots of |c_s| times the slot's S_abs)."""
    from block_quantized_gemv_amd import synth
    H, I, T = hidden, inter, 4
    log(f"MoE {n_experts} experts, top-{n_sel}, hidden {H}, inter {I}")
    gu = np.stack([synth.q4k_matrix(seed, (synth.KEY_EXPERT, e, 0), 2 * I, H) for e in range(n_experts)])
    dn = np.stack([synth.q4k_matrix(seed, (synth.KEY_EXPERT, e, 1), H, I) for e in range(n_experts)])
    ids, logits = synth.routing(seed, T, n_experts, n_sel)
    X = synth.normal_f32(seed, (synth.KEY_TOKEN_X,), (T, H))
    args = (n_experts, n_sel, H, I, to_dev(gu.ravel()), gu[0].nbytes, to_dev(dn.ravel()), dn[0].nbytes,
            to_dev(ids), to_dev(logits), to_dev(X))
    g = mq.MoEChain(*args)
    e = mq.MoEChain(*args, flags=mq.MQ_EAGER_ONLY)
    for _ in range(T):
        g.step(mq.MQ_GRAPH)
        e.step(mq.MQ_EAGER)
    yg, ye = to_host(g.y_table), to_host(e.y_table)
    assert np.array_equal(yg.view(np.uint32), ye.view(np.uint32)), "graph != eager"
    for t in range(T):
        y_ref, _, c_ref = o.moe_token(gu.ravel(), gu[0].nbytes, dn.ravel(), dn[0].nbytes, ids[t], logits[t],
                                      X[t], H, I)
        s_abs = np.zeros(H)
        xq = o.quantize_q8_0(X[t]).ravel()
        for sl, ex in enumerate(ids[t]):
            t_gu, _ = o.gemv_q4k(gu[ex], 2 * I, H, xq)
            _, sa = o.gemv_q4k(dn[ex], H, I, o.quantize_q8_0(o.swiglu(t_gu)).ravel())
            s_abs += abs(float(c_ref[sl])) * sa
        check_tolerance(yg[t], y_ref, s_abs, f"token {t}")


def _split_case(mq, o, pool, m, what):
    """Graph == eager over six steps and a reset, for a one-layer chain whose
    gate/up has split blocks; then the step's trace against the oracle's own
    step, stage by stage (check_chain_trace: the SwiGLU q8_0 vector equal to
    the oracle's bytes, every gate/up row within the gate), and every
    gate/up row, the split ones included, bit-identical to the oracle's."""
    import torch
    from block_quantized_gemv_amd import synth
    H, I, QKV = m.hidden, m.inter, m.qkv_rows
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nblk = I // 32
    two_passes = (H // 256 + 3) // 4 >= 2
    ns = (nblk % cus if nblk > cus else nblk if 2 * nblk <= cus else 0) if two_passes else 0
    assert ns > 0, f"{nblk} gate/up blocks on {cus} CUs: no split blocks to test"
    W = model_weights(m, 1)
    Wd = _dev_weights(W)
    X = synth.normal_f32(m.seed, (synth.KEY_STEP_INPUTS,), (3, H))
    xd = to_dev(X)
    g = mq.DecodeChain(m, Wd, xd, flags=mq.MQ_KEEP_INTERMEDIATES)
    e = mq.DecodeChain(m, Wd, xd, flags=mq.MQ_KEEP_INTERMEDIATES | mq.MQ_EAGER_ONLY)
    assert g.info()["captured"]
    for i in range(6):
        lg = to_host(g.step()).copy()
        qg, fg = (to_host(t).copy() for t in g.trace())
        le = to_host(e.step(mq.MQ_EAGER)).copy()
        qe, fe = (to_host(t).copy() for t in e.trace())
        assert _same(lg, le) and _same(qg, qe) and _same(fg, fe), f"graph != eager at step {i}"
    g.reset(0)
    e.reset(0)
    lg = to_host(g.step()).copy()
    assert _same(lg, to_host(e.step(mq.MQ_EAGER)).copy()), "graph != eager after reset"
    qg, fg = (to_host(t).copy() for t in g.trace())
    ref_logits, s_abs, rq8, rf32, rsabs = oracle_chain_parallel(o, m, W, X[0], 1, pool)
    check_chain_trace(m, 1, qg, fg, rq8, rf32, rsabs, what)
    check_tolerance(lg, ref_logits, s_abs, f"{what} logits")
    gu, gu_ref = fg[QKV + H:QKV + H + 2 * I], rf32[QKV + H:QKV + H + 2 * I]
    first = 32 * (nblk - ns)
    split_rows = np.concatenate([np.arange(first, I), I + np.arange(first, I)])
    same_all = float(np.mean(gu.view(np.uint32) == gu_ref.view(np.uint32)))
    same_split = float(np.mean(gu[split_rows].view(np.uint32) == gu_ref[split_rows].view(np.uint32)))
    log(f"  {ns} split blocks; gate/up bit-identical to the oracle: all rows {same_all:.5f}, "
        f"split rows {same_split:.5f}")
    assert same_all == 1.0 and same_split == 1.0, "gate/up rows are not bit-identical to the oracle's"
    g.close()
    e.close()


@pytest.mark.parametrize("fmt", ["q4_K", "q4_0"])
def test_gate_up_split_blocks_7b_width(mq, o, pool, fmt):
    """At 7B widths the gate/up kernel has 592 output blocks; the blocks beyond
    a multiple of the CU count are each computed by two workgroups, one per
    half of K, that hand over through a counter (k_gemv_q4k_swiglu)."""
    from block_quantized_gemv_amd import workloads
    m = dataclasses.replace(workloads.DECODE_7B, n_layers=1)
    if fmt == "q4_0":
        m = dataclasses.replace(m, weight_format="q4_0")
    _split_case(mq, o, pool, m, f"7B {fmt}")


@pytest.mark.parametrize("fmt", ["q4_K", "q4_0"])
def test_span_stamps_7b_width(mq, fmt):
    """The stamped kernels at 7B widths (two layers, vocabulary 8192), where
    gate/up has split blocks, in both weight formats: over three graph
    steps and an eager one, the stamped chain's logits and every traced
    intermediate equal the plain chain's byte for byte, and every kernel's
    stamp pair is filled and ordered."""
    from block_quantized_gemv_amd import synth, workloads
    m = dataclasses.replace(workloads.DECODE_7B, n_layers=2, vocab=8192)
    if fmt == "q4_0":
        m = dataclasses.replace(m, weight_format="q4_0")
    W = model_weights(m, 2)
    Wd = _dev_weights(W)
    xd = to_dev(synth.normal_f32(m.seed, (synth.KEY_STEP_INPUTS,), (3, m.hidden)))
    plain = mq.DecodeChain(m, Wd, xd, flags=mq.MQ_KEEP_INTERMEDIATES)
    stamped = mq.DecodeChain(m, Wd, xd, flags=mq.MQ_KEEP_INTERMEDIATES | mq.MQ_SPAN_STAMPS)
    n = 4 * m.n_layers + 1
    for i, mode in enumerate((mq.MQ_GRAPH, mq.MQ_GRAPH, mq.MQ_EAGER, mq.MQ_GRAPH)):
        a = to_host(plain.step(mode)).copy()
        qa, fa = (to_host(t).copy() for t in plain.trace())
        b = to_host(stamped.step(mode)).copy()
        qb, fb = (to_host(t).copy() for t in stamped.trace())
        assert _same(a, b) and _same(qa, qb) and _same(fa, fb), f"{fmt}: stamped step {i} differs"
        st = stamped.read_stamps()
        assert st.shape == (n, 2) and (st[:, 0] < st[:, 1]).all(), f"{fmt}: unfilled stamp pair at step {i}"
        assert (st[1:, 0] >= st[:-1, 1] - 1).all(), f"{fmt}: kernels overlap at step {i}"
    plain.close()
    stamped.close()


@pytest.mark.parametrize("inter", [2560, 8448, 16128])
def test_gate_up_split_block_counts(mq, o, pool, inter):
    """Few, many and all blocks split: hidden 1280 (two passes over K), 264
    and 504 gate/up blocks, so 8 and 248 of them split on a 256-CU GPU, and
    80 blocks, which fill fewer than half the CUs, so every one splits."""
    from block_quantized_gemv_amd import workloads
    m = dataclasses.replace(workloads.DECODE_7B, n_layers=1, hidden=1280, qkv_rows=1280 + 256, inter=inter,
                            vocab=4096)
    _split_case(mq, o, pool, m, f"hidden 1280, inter {inter}")


@pytest.mark.parametrize("fmt", ["q4_K", "q4_0"])
def test_gate_up_split_counts_and_fallbacks(mq, o, fmt):
    """The fused gate/up kernel on its own (mq_debug_gate_up_swiglu) at
    hidden 1280 (two passes over K) with 64 output blocks, under split
    counts the chains never pass: none, one, all 64; and counts that do not
    fit the shape, which must run every block whole: 65 > 64 blocks, no
    hand-over space, and K = 256 (one pass, nothing to split).  Each case:
    every gate/up row within the gate and bit-identical to the oracle's,
    the SwiGLU q8_0 bytes equal to the oracle's, the counters left zero."""
    import torch
    from block_quantized_gemv_amd import synth
    mat = synth.q4_0_matrix if fmt == "q4_0" else synth.q4k_matrix
    gemv = o.gemv_q4_0 if fmt == "q4_0" else o.gemv_q4k
    I = 2048
    cases = [(1280, 0, True), (1280, 1, True), (1280, 64, True), (1280, 65, True), (1280, 3, False),
             (256, 2, True)]
    for k, ns, space in cases:
        log(f"gate/up {fmt} k={k} inter={I} n_split={ns} hand-over space={space}")
        w = mat(9, (synth.KEY_MATRIX, k, 1), 2 * I, k)
        x = synth.normal_f32(9, (synth.KEY_COLUMNS, k, 1), (k,))
        a = o.quantize_q8_0(o.rmsnorm(x, 1e-6)).ravel()
        gu_ref, s_abs = gemv(w, 2 * I, k, a)
        g_ref = np.asarray(o.quantize_q8_0(o.swiglu(gu_ref)), np.uint8).ravel()
        part = torch.full((max(ns, 1) * 128,), float("nan"), dtype=torch.float64, device="cuda") if space else None
        cnt = torch.zeros(max(ns, 1), dtype=torch.int32, device="cuda") if space else None
        gu, g = mq.mq_debug_gate_up_swiglu(to_dev(w), to_dev(x), I, k, ns, part, cnt, weight_format=fmt)
        gu, g = to_host(gu), to_host(g)
        _, exact = check_tolerance(gu, gu_ref, s_abs, f"gate/up k={k} n_split={ns}")
        assert exact == 1.0, "gate/up rows are not bit-identical to the oracle's"
        assert np.array_equal(g, g_ref), "SwiGLU q8_0 bytes differ from the oracle's"
        if space:
            assert not to_host(cnt).any(), "hand-over counters not left zero"
