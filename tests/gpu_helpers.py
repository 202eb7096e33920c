"""Shared pieces of the GPU parity tests (import only from gpu-marked tests)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TOL_REL = 1e-3      # |y - y_ref| <= 1e-3 * sum_i |w_i x_i| + 1e-6 per row
TOL_ABS = 1e-6
THREADS = min(16, os.cpu_count() or 1)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def check_tolerance(y, y_ref, s_abs, what):
    """Asserts the per-row float gate; returns (max |dy|/S_abs, fraction bit-identical)."""
    y = np.asarray(y, np.float32).ravel()
    y_ref = np.asarray(y_ref, np.float32).ravel()
    s_abs = np.asarray(s_abs, np.float64).ravel()
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    bad = ~(err <= TOL_REL * s_abs + TOL_ABS)
    assert not bad.any(), (f"{what}: {bad.sum()} rows outside tolerance, first at {np.argmax(bad)}: "
                           f"{y[bad][:3]} vs {y_ref[bad][:3]} (S_abs {s_abs[bad][:3]})")
    rel = float(np.max(err / np.maximum(s_abs, 1e-300)))
    exact = float(np.mean(y.view(np.uint32) == y_ref.view(np.uint32)))
    log(f"  {what}: rows={y.size} max|dy|/S_abs={rel:.2e} bit-identical={exact:.4f}")
    return rel, exact


def sample_rows(m, n, seed):
    g = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, m - 1], g.choice(m, size=min(n, m), replace=False)]))
    return rows.astype(np.int64)


def oracle_gemv_parallel(fn, w, m, k, xq, rows=None, pool=None):
    """Row-partitioned calls of the oracle's single-threaded row function."""
    rows = np.arange(m, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    chunks = np.array_split(rows, max(1, min(THREADS * 4, rows.size // 64 or 1)))
    own = pool is None
    pool = pool or ThreadPoolExecutor(THREADS)
    try:
        parts = list(pool.map(lambda r: fn(w, m, k, xq, rows=r), chunks))
    finally:
        if own:
            pool.shutdown()
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_chain_parallel(o, model, W, h0, n_layers, pool):
    """The decode step composed from the oracle's stages (the composition is
    the one oracle.chain implements, pinned by pin_chain_structure and
    pin_chain_structure_q4_0), with the GEMV rows spread over threads.
    Returns logits, s_abs, q8 trace, f32 trace, and the f64 sum_i |w_i x_i|
    of every f32 trace value (the per-row tolerance of its GEMV)."""
    H, I, eps = model.hidden, model.inter, model.eps
    K = getattr(model, "o_k", 0) or H          # O's K: the first K QKV outputs
    gemv = o.gemv_q4_0 if getattr(model, "weight_format", "q4_K") == "q4_0" else o.gemv_q4k
    h = np.asarray(h0, np.float32)
    q8s, f32s, sabs = [], [], []
    for l in range(n_layers):
        a = o.quantize_q8_0(o.rmsnorm(h, eps)).ravel(); q8s.append(a)
        t, st = oracle_gemv_parallel(gemv, W["qkv"][l], model.qkv_rows, H, a, pool=pool)
        b = o.quantize_q8_0(o.rmsnorm(t[:K], eps)).ravel()
        q8s.append(np.concatenate([b, np.zeros((H - K) // 32 * 34, np.uint8)]))   # a hidden-wide trace slot
        ov, so = oracle_gemv_parallel(gemv, W["o"][l], H, K, b, pool=pool)
        c = o.quantize_q8_0(o.rmsnorm(ov, eps)).ravel(); q8s.append(c)
        gu, sg = oracle_gemv_parallel(gemv, W["gu"][l], 2 * I, H, c, pool=pool)
        g = o.quantize_q8_0(o.swiglu(gu)).ravel(); q8s.append(g)
        h, sd = oracle_gemv_parallel(gemv, W["down"][l], H, I, g, pool=pool)
        f32s += [t, ov, gu, h]
        sabs += [st, so, sg, sd]
    z = o.quantize_q8_0(o.rmsnorm(h, eps)).ravel(); q8s.append(z)
    logits, s_abs = oracle_gemv_parallel(o.gemv_q8_0, W["lm"], model.vocab, H, z, pool=pool)
    return logits, s_abs, np.concatenate(q8s), np.concatenate(f32s), np.concatenate(sabs)


def trace_stages(model, n_layers):
    """Names and (q8 byte range | f32 value range) of every stage of a chain
    trace, in step order: per layer the q8_0 inputs of QKV, O, gate/up and
    down and the f32 outputs of the four GEMVs; then the lm_head input."""
    H, I, Q = model.hidden, model.inter, model.qkv_rows
    qH, qI = H // 32 * 34, I // 32 * 34
    q8, f32 = [], []
    qo = fo = 0
    for l in range(n_layers):
        for name, n in (("qkv in", qH), ("o in", qH), ("gate/up in", qH), ("down in", qI)):
            q8.append((f"layer {l} {name}", qo, qo + n))
            qo += n
        for name, n in (("qkv", Q), ("o", H), ("gate/up", 2 * I), ("down", H)):
            f32.append((f"layer {l} {name}", fo, fo + n))
            fo += n
    q8.append(("lm_head in", qo, qo + qH))
    return q8, f32


def check_chain_trace(model, n_layers, q8t, f32t, rq8, rf32, rsabs, what):
    """Stage-by-stage parity of a decode step's trace against the oracle's
    own step on the same seeded input.  Every q8_0 vector a glue stage formed
    must equal the oracle's bytes; every GEMV output must be within the
    per-row gate of the oracle's value (sum_i |w_i x_i| from the oracle).
    Because the q8_0 inputs are asserted equal first, each GEMV is checked
    against the oracle on the very input it consumed.  Returns the fraction
    of f32 values that are bit-identical."""
    q8s, f32s = trace_stages(model, n_layers)
    assert q8t.size == q8s[-1][2] and f32t.size == f32s[-1][2], "trace sizes"
    for name, a, b in q8s:
        ds, dq, mx = q8_code_diff(q8t[a:b], rq8[a:b])
        assert ds == 0 and dq == 0, (f"{what}: {name}: q8_0 bytes differ from the oracle's "
                                     f"(scales {ds}, codes {dq}, max |dq| {mx})")
    for name, a, b in f32s:
        y, yr, sa = f32t[a:b], rf32[a:b], rsabs[a:b]
        err = np.abs(y.astype(np.float64) - yr.astype(np.float64))
        bad = ~(err <= TOL_REL * sa + TOL_ABS)
        assert not bad.any(), f"{what}: {name}: {bad.sum()} rows outside tolerance, first {np.argmax(bad)}"
    same = float(np.mean(f32t.view(np.uint32) == rf32.view(np.uint32)))
    log(f"  {what}: {len(q8s)} q8_0 stages byte-identical, {len(f32s)} GEMV stages within tolerance, "
        f"f32 bit-identical {same:.6f}")
    return same


def model_weights(model, n_layers):
    """Seeded synthetic weights of a decode-step model (host numpy)."""
    from block_quantized_gemv_amd import synth
    s = model.seed
    mat = synth.q4_0_matrix if getattr(model, "weight_format", "q4_K") == "q4_0" else synth.q4k_matrix
    W = {"qkv": [], "o": [], "gu": [], "down": []}
    for l in range(n_layers):
        W["qkv"].append(mat(s, (synth.KEY_LAYER, l, 0), model.qkv_rows, model.hidden))
        W["o"].append(mat(s, (synth.KEY_LAYER, l, 1), model.hidden, getattr(model, "o_k", 0) or model.hidden))
        W["gu"].append(mat(s, (synth.KEY_LAYER, l, 2), 2 * model.inter, model.hidden))
        W["down"].append(mat(s, (synth.KEY_LAYER, l, 3), model.hidden, model.inter))
    W["lm"] = synth.q8_0_matrix(s, (synth.KEY_LM_HEAD,), model.vocab, model.hidden)
    return W


def q8_code_diff(a, b):
    """Compare two q8_0 byte streams: (#blocks whose scale differs, #codes that differ, max |code diff|)."""
    a = np.asarray(a, np.uint8).reshape(-1, 34)
    b = np.asarray(b, np.uint8).reshape(-1, 34)
    ds = int(np.sum(np.any(a[:, :2] != b[:, :2], axis=1)))
    qa = a[:, 2:].view(np.int8).astype(np.int32)
    qb = b[:, 2:].view(np.int8).astype(np.int32)
    d = np.abs(qa - qb)
    return ds, int(np.count_nonzero(d)), int(d.max()) if d.size else 0
