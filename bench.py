"""Benchmark: q4_K x q8_0 decode GEMV throughput on one MI355X.

Default workload: one 7B-class decode step (hidden 3584, 28 layers, q4_K
QKV/O/gate-up/down GEMVs at n=1 with RMSNorm/SwiGLU glue, q8_0 lm_head
152064x3584), replayed as one hipGraph per step.  A step streams
4.25 GB of weights once; the timed region starts with every input resident
in HBM.  Prints one JSON line (rank 0):

  value      = algorithmic bytes per step / step time, GB/s
  tok_per_s  = decode steps per second
  roofline   = the GEMV kernel with the largest share of step time: its
               average algorithmic bytes per launch / average launch
               duration, each launch timed by its own dispatch events on the
               launching stream (eager steps, the same kernels and arguments
               the graph replays), against 8 TB/s; `traffic` is the HBM bytes
               per launch the committed rocprofv3 counter record measured;
               also as a fraction of the streaming-read probe, and the
               byte-weighted aggregate of the four per-layer q4_K GEMVs
  stream_probe = the rate of a plain 16-byte-load read of 4 GiB
               (mq_probe_stream_read), measured first in the same run
  sync_probe = per GEMV boundary, what a resident (persistent) step would
               pay (a grid barrier carrying the hidden vector between the
               XCDs) against the graph's own cost per kernel boundary
  span_stamps = the step's replay span against the sum of its kernels' own
               spans (first wave start to last wave end), both from the
               kernels' real-time-counter stamps with no tracer present
               (MQ_SPAN_STAMPS); the roofline object adds the dominant
               kernel's in-graph span from the same stamps
  cpu_baseline = the reference oracle on the host, on a bounded sample

Other workloads (--workload 05b|05b_q4_0|7b_tp8|single|batched|moe) print their
own line; 7b_tp8 is the step of the largest of eight tensor-parallel ranks of
the 7B-class model (its shard shapes, the collectives not run).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "q4_K x q8_0 GEMV HBM GB/s (% of peak); decode-step tok/s, 1 GPU"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="7b", choices=["7b", "05b", "05b_q4_0", "7b_tp8", "single", "batched", "moe"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-ab", action="store_true", help="skip the interleaved A/B arms (for counter runs)")
    p.add_argument("--no-stamps", action="store_true", help="skip the span-stamp measurement of the step")
    p.add_argument("--no-extra", action="store_true",
                   help="the default 7B line only (skip the compact lines of the other four workloads)")
    p.add_argument("--kernel-reps", type=int, default=3, help="passes of the dominant-kernel timing region")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def sem(xs):
    xs = np.asarray(xs, np.float64)
    return float(xs.std(ddof=1) / math.sqrt(xs.size)) if xs.size > 1 else 0.0


# ------------------------------------------------------------------------------

def upload_model(model, dev, keep_host=False):
    """Weights generated per matrix on the host and moved to HBM; the host
    copies are kept only when the CPU baseline needs them."""
    import torch
    from block_quantized_gemv_amd import synth
    s = model.seed
    W = {"qkv": [], "o": [], "gu": [], "down": []}
    H = {"qkv": [], "o": [], "gu": [], "down": []} if keep_host else None
    shapes = model.layer_shapes()
    mat = synth.q4_0_matrix if model.weight_format == "q4_0" else synth.q4k_matrix
    for l in range(model.n_layers):
        for key, kind, (m, k) in zip(("qkv", "o", "gu", "down"), range(4), shapes):
            a = mat(s, (synth.KEY_LAYER, l, kind), m, k)
            W[key].append(torch.from_numpy(a).to(dev))
            if keep_host:
                H[key].append(a)
    lm = synth.q8_0_matrix(s, (synth.KEY_LM_HEAD,), model.vocab, model.hidden)
    W["lm"] = torch.from_numpy(lm).to(dev)
    if keep_host:
        H["lm"] = lm
    return W, H


class HipEvents:
    """hipEventCreate / hipEventElapsedTime on the HIP runtime torch loaded."""

    def __init__(self):
        import ctypes as C
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.C = C
        self.hip = C.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.events = []

    def create(self):
        ev = self.C.c_void_p()
        if self.hip.hipEventCreate(self.C.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(ev.value)
        return ev.value

    def elapsed_ms(self, a, b):
        ms = self.C.c_float()
        if self.hip.hipEventElapsedTime(self.C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.events:
            self.hip.hipEventDestroy(e)
        self.events = []


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_q4k_gemv_7b_decode_step.txt")


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter record (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when there is no record for that kernel and workload or the kernel
    sources changed since it was taken."""
    import hashlib
    try:
        rec = dict(ln.split(": ", 1) for ln in open(TRAFFIC_RECORD).read().splitlines() if ": " in ln)
    except OSError:
        return None
    if rec.get("dominant_kernel", "").strip() != kernel.split(" ")[0]:
        return None
    if rec.get("workload", "").strip() != workload:
        return None
    h = hashlib.sha256()
    for f in rec.get("kernel_sources", "").split():
        try:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        except OSError:
            return None
    if h.hexdigest()[:16] != rec.get("kernel_sources_sha256_16", "").strip():
        return None
    return int(float(rec["traffic_bytes_per_launch"]))


def gemv_kinds(model):
    """The step's kernels in order, with their names and algorithmic bytes:
    weights + activation in (f32 where the kernel forms Q8(RMSNorm(x)) in its
    prologue, q8_0 otherwise) + output written (f32, or q8_0 after SwiGLU)."""
    from block_quantized_gemv_amd import workloads as wl
    H, I, Q, KO = model.hidden, model.inter, model.qkv_rows, model.o_in
    wb = model.layer_matrix_bytes
    f = 1 if model.weight_format == "q4_0" else 0      # the kernels' format template argument
    norm = f"mq::k_gemv_q4k<{f},1,false,2,false>"
    kinds = []
    for _ in range(model.n_layers):
        kinds += [("qkv", norm, wb(Q, H) + 4 * H + 4 * Q),
                  ("o", norm, wb(H, KO) + 4 * KO + 4 * H),
                  ("gate/up", f"mq::k_gemv_q4k_swiglu<{f},true,false>", wb(2 * I, H) + 4 * H + wl.q8_bytes(1, I)),
                  ("down", f"mq::k_gemv_q4k<{f},1,false,1,false>", wb(H, I) + wl.q8_bytes(1, I) + 4 * H)]
    kinds.append(("lm_head", "mq::k_gemv_q8_0<false,true,false>", wl.q8_bytes(model.vocab, H) + 4 * H + 4 * model.vocab))
    return kinds


def time_kernels(mq, model, eager_chain, reps):
    """Every GEMV of `reps` eager steps (the kernels and arguments the graph
    replays), each timed by its own dispatch timestamps through
    mq_time_next_launches, on the launching stream."""
    import torch
    kinds = gemv_kinds(model)
    hip = HipEvents()
    n = len(kinds) * reps
    starts = [hip.create() for _ in range(n)]
    stops = [hip.create() for _ in range(n)]
    torch.cuda.synchronize()
    mq.mq_time_next_launches(starts, stops)
    for _ in range(reps):
        eager_chain.step(mq.MQ_EAGER)
    torch.cuda.synchronize()
    mq.mq_time_next_launches([], [])
    us = [hip.elapsed_ms(a, b) * 1e3 for a, b in zip(starts, stops)]
    hip.close()
    by_kind, by_kernel = {}, {}
    for i, u in enumerate(us):
        name, kernel, nbytes = kinds[i % len(kinds)]
        d = by_kind.setdefault(name, {"kernel": kernel, "bytes": nbytes, "us": []})
        d["us"].append(u)
        k = by_kernel.setdefault(kernel, {"bytes": 0, "us": 0.0, "n": 0})
        k["bytes"] += nbytes
        k["us"] += u
        k["n"] += 1
    dominant = max(by_kernel, key=lambda k: by_kernel[k]["us"])
    dk = by_kernel[dominant]
    avg_b, avg_us = dk["bytes"] / dk["n"], dk["us"] / dk["n"]
    achieved = avg_b / avg_us / 1e3
    per_shape = {name: {"kernel": d["kernel"], "us": round(float(np.mean(d["us"])), 3),
                        "sem_us": round(sem(d["us"]), 4),
                        "GB_s": round(d["bytes"] / float(np.mean(d["us"])) / 1e3, 1)}
                 for name, d in by_kind.items()}
    kernel_sum_ms = sum(us) / reps / 1e3
    layer = [by_kind[k] for k in ("qkv", "o", "gate/up", "down") if k in by_kind]
    agg_b = sum(d["bytes"] * len(d["us"]) for d in layer)
    agg_us = sum(sum(d["us"]) for d in layer)
    aggregate = {"what": f"byte-weighted aggregate of the per-layer {model.weight_format} GEMVs "
                         "(QKV, O, gate/up, down)",
                 "GB_s": round(agg_b / agg_us / 1e3, 1), "frac": round(agg_b / agg_us / 1e3 / HBM_PEAK_GBS, 4)}
    return {"bound": "hbm", "kernel": dominant, "launches": dk["n"], "bytes_per_launch": round(avg_b),
            "us_per_launch": round(avg_us, 3), "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dominant, model.name),
            "timing": "dispatch events of each launch (hipExtLaunchKernelGGL), launched from an idle stream "
                      "in eager steps; includes the dispatch latency a graph replay hides",
            "per_shape": per_shape, "q4k_layer_aggregate": aggregate}, kernel_sum_ms


def stream_probe(mq, gib=4, reps=5):
    """The plain streaming-read rate (mq_probe_stream_read over `gib` GiB, a
    few workgroup counts, best mean over `reps` timed passes each)."""
    import torch
    buf = torch.empty(gib << 28, dtype=torch.int32, device="cuda:0")
    nbytes = buf.numel() * 4
    best = None
    for wgs in (256, 512, 1024):
        for _ in range(2):
            mq.mq_probe_stream_read(buf, workgroups=wgs)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            mq.mq_probe_stream_read(buf, workgroups=wgs)
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"stream probe {gib} GiB, {wgs} x 1024 threads: {ms:.3f} ms, {gbs:.1f} GB/s")
        if best is None or gbs > best["GB_s"]:
            best = {"GB_s": round(gbs, 1), "bytes": nbytes, "workgroups": wgs, "ms": round(ms, 4)}
    del buf
    torch.cuda.empty_cache()
    best["frac_of_peak"] = round(best["GB_s"] / HBM_PEAK_GBS, 4)
    return best


def cpu_baseline_decode(model, host_w, n_layers_sample):
    """The oracle, single thread, on the first layers of the step (all four
    GEMVs with their glue) plus the same fraction of lm_head rows."""
    import oracle
    from block_quantized_gemv_amd import synth, workloads
    o = oracle.Oracle()
    s = model.seed
    H, I, eps = model.hidden, model.inter, model.eps
    lm_rows = int(round(model.vocab * n_layers_sample / model.n_layers))
    lm = host_w["lm"][:lm_rows]
    h = synth.normal_f32(s, (synth.KEY_STEP_INPUTS,), (1, H))[0]
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    gemv = o.gemv_q4_0 if model.weight_format == "q4_0" else o.gemv_q4k
    t0 = time.perf_counter()
    nbytes = 0
    for l in range(n_layers_sample):
        qkv, ow, gu, dn = (host_w[k][l] for k in ("qkv", "o", "gu", "down"))
        a = o.quantize_q8_0(o.rmsnorm(h, eps)).ravel()
        t, _ = gemv(qkv, model.qkv_rows, H, a)
        b = o.quantize_q8_0(o.rmsnorm(t[:H], eps)).ravel()
        ov, _ = gemv(ow, H, H, b)
        c = o.quantize_q8_0(o.rmsnorm(ov, eps)).ravel()
        g_u, _ = gemv(gu, 2 * I, H, c)
        g = o.quantize_q8_0(o.swiglu(g_u)).ravel()
        h, _ = gemv(dn, H, I, g)
        nbytes += sum(model.layer_matrix_bytes(m, k) + workloads.q8_bytes(1, k) + 4 * m
                      for m, k in model.layer_shapes())
    z = o.quantize_q8_0(o.rmsnorm(h, eps)).ravel()
    o.gemv_q8_0(lm, lm_rows, H, z)
    nbytes += workloads.q8_bytes(lm_rows, H) + workloads.q8_bytes(1, H) + 4 * lm_rows
    dt = time.perf_counter() - t0
    frac = n_layers_sample / model.n_layers
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tok_per_s": round(frac / dt, 6), "seconds": round(dt, 2),
            "sample": (f"{n_layers_sample} of {model.n_layers} layers (4 GEMVs + glue each) and "
                       f"{lm_rows} of {model.vocab} lm_head rows of one decode step, single thread pinned to one core"
                       + ("" if n_layers_sample == model.n_layers else
                          f"; tok/s scaled by {model.n_layers}/{n_layers_sample}")),
            "cpu": _cpu_model()}


def _pin_one_core():
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass


def _cpu_line(nbytes, seconds, sample, **extra):
    out = {"value": round(nbytes / seconds / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "seconds": round(seconds, 3), "sample": sample + ", single thread pinned to one core", "cpu": _cpu_model()}
    out.update(extra)
    return out


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def interleaved_arms(args, mq, model, W, X, chain, eager):
    import torch
    # Interleaved A/B arms on one binary, one step of each in turn: the
    # graph, the same kernels launched eagerly, and the unfused-glue graph
    # (standalone RMSNorm/SwiGLU->q8_0 kernels between q8_0-input GEMVs).
    unfused = mq.DecodeChain(model, W, X, flags=mq.MQ_UNFUSED_GLUE)
    for _ in range(args.warmup):
        unfused.step(mq.MQ_GRAPH)
    arms = {"graph": (chain, mq.MQ_GRAPH), "eager": (eager, mq.MQ_EAGER), "unfused_glue_graph": (unfused, mq.MQ_GRAPH)}
    evs = {k: [] for k in arms}
    for _ in range(args.steps):
        for k, (arm, mode) in arms.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            arm.step(mode)
            b.record()
            evs[k].append((a, b))
    torch.cuda.synchronize()
    ab = {"steps_per_arm": args.steps, "unfused_glue_nodes": unfused.info()["n_nodes"]}
    for k, v in evs.items():
        t = [a.elapsed_time(b) for a, b in v]
        ab[f"{k}_ms"] = round(float(np.mean(t)), 4)
        ab[f"{k}_sem_ms"] = round(sem(t), 5)
    unfused.close()
    log(f"interleaved A/B: {ab}")
    return ab


def span_stamps(args, mq, model, W, X, steps=100):
    """The replay span of one step against the sum of its kernels' own spans,
    from the kernels' real-time-counter stamps (MQ_SPAN_STAMPS: first wave
    start and last wave end of every GEMV kernel, 100 MHz), with no tracer in
    the process.  Each measured step directly follows a warm step and its
    stamps are read after it.  Also: the stamped chain's own back-to-back time per step
    (events over 20 replays, to set against the plain chain's), and a check
    of the counter's rate against the host clock over 0.2 s."""
    import torch
    tick_us = 0.01
    c = mq.DecodeChain(model, W, X, flags=mq.MQ_SPAN_STAMPS)
    for _ in range(max(args.warmup, 3)):
        c.step(mq.MQ_GRAPH)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(20):
        c.step(mq.MQ_GRAPH)
    b.record()
    torch.cuda.synchronize()
    b2b_us = a.elapsed_time(b) * 1e3 / 20
    h0 = time.perf_counter()
    c.step(mq.MQ_GRAPH)
    s0 = int(c.read_stamps()[0, 0])
    time.sleep(0.2)
    h1 = time.perf_counter()
    c.step(mq.MQ_GRAPH)
    s1 = int(c.read_stamps()[0, 0])
    clock = (h1 - h0) * 1e6 / ((s1 - s0) * tick_us)
    spans, sums, gaps = [], [], []
    per = None
    for _ in range(steps):
        # a warm step, then the measured step right behind it (the GPU does
        # not idle before it); its waves overwrite the warm step's stamps
        c.step(mq.MQ_GRAPH)
        c.step(mq.MQ_GRAPH)
        st = c.read_stamps().astype(np.int64)
        d = (st[:, 1] - st[:, 0]) * tick_us
        per = d if per is None else per + d
        spans.append((st[:, 1].max() - st[:, 0].min()) * tick_us)
        sums.append(d.sum())
        gaps.append(float(np.mean((st[1:, 0] - st[:-1, 1]) * tick_us)))
    c.close()
    per /= steps
    L = model.n_layers
    kinds = {"qkv": per[0:4 * L:4], "o": per[1:4 * L:4], "gate_up": per[2:4 * L:4], "down": per[3:4 * L:4]}
    res = {"steps": steps, "kernels_per_step": int(st.shape[0]),
           "replay_span_us": round(float(np.mean(spans)), 2), "replay_span_sem_us": round(sem(spans), 3),
           "kernel_sum_us": round(float(np.mean(sums)), 2),
           "span_over_sum": round(float(np.mean(spans)) / float(np.mean(sums)), 4),
           "mean_gap_between_kernels_us": round(float(np.mean(gaps)), 3),
           "per_kernel_us": {k: round(float(v.mean()), 3) for k, v in kinds.items()},
           "lm_head_us": round(float(per[-1]), 3),
           "stamped_chain_back_to_back_us_per_step": round(float(b2b_us), 2),
           "host_over_stamp_clock_0p2s": round(float(clock), 5)}
    log(f"span stamps: {res}")
    return res


def sync_probe(mq, model, stamps=None):
    """What a resident (persistent) step would pay per GEMV boundary against
    what the graph pays: grid-barrier rounds on one 512-thread workgroup per
    CU (flat and per-XCD counters), bare and carrying the model's hidden
    vector (each workgroup writes its slice with agent-scope stores, then all
    read all of it), and the graph's cost per empty kernel on the same grid."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    words = -(-model.hidden // cus)
    res = {"threads": 512, "workgroups": cus, "exchange_words_per_workgroup": words,
           "exchange": f"each workgroup writes {words} f32 of the {model.hidden}-wide vector, then reads all of it"}
    for hier, name in ((0, "flat"), (1, "xcd_hierarchical")):
        bare, bad0 = mq.mq_probe_grid_barrier(hier, 0, rounds=2000)
        ex, bad1 = mq.mq_probe_grid_barrier(hier, words, rounds=2000)
        assert bad0 == 0 and bad1 == 0, "the barrier probe read a stale word"
        res[f"barrier_{name}_us"] = round(bare, 3)
        res[f"barrier_{name}_with_exchange_us"] = round(ex, 3)
    res["graph_empty_kernel_us"] = round(mq.mq_probe_graph_boundary(n_kernels=200, threads=512, reps=10), 3)
    best = min(res["barrier_flat_with_exchange_us"], res["barrier_xcd_hierarchical_with_exchange_us"])
    res["best_barrier_with_exchange_us"] = best
    if stamps:
        n = stamps["kernels_per_step"]
        res["graph_gaps_per_step_us"] = round((n - 1) * stamps["mean_gap_between_kernels_us"], 1)
        res["persistent_barriers_per_step_us"] = round((n - 1) * best, 1)
    log(f"sync probe: {res}")
    return res


def host_step_latency(args, mq, model, W, X, chain):
    import torch
    # End-to-end step latency as a caller sees it: launch the step, wait for
    # it, read the logits into host memory.  Arms interleaved step by step:
    # readback through the library's pinned buffer, straight into pageable
    # memory, and no readback.  Plus the one-time capture cost and the lazy
    # capture policy's own capture.
    # The in-graph arm's chain copies the logits into its own pinned buffer
    # as the step's last node; its logits are in host memory when the wait
    # returns.
    out_p = np.empty(model.vocab, np.float32)
    out_q = np.empty(model.vocab, np.float32)
    in_graph = mq.DecodeChain(model, W, X, flags=mq.MQ_HOST_LOGITS)
    assert in_graph.host_logits() is not None, "pinning the host logits failed"
    arms = {"pinned_readback": (chain, lambda: chain.read_logits(out=out_p)),
            "pageable_readback": (chain, lambda: chain.read_logits(out=out_q, pageable=True)),
            "in_graph_host_copy": (in_graph, lambda: None),
            "no_readback": (chain, lambda: None)}
    for _ in range(args.warmup):
        for c, f in arms.values():
            c.step(mq.MQ_GRAPH)
            torch.cuda.synchronize()
            f()
    t_sync = {k: [] for k in arms}
    t_read = {k: [] for k in arms}
    for _ in range(args.steps):
        for k, (c, f) in arms.items():
            t0 = time.perf_counter()
            c.step(mq.MQ_GRAPH)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            f()
            t2 = time.perf_counter()
            t_sync[k].append((t1 - t0) * 1e3)
            t_read[k].append((t2 - t1) * 1e3)
    res = {"steps_per_arm": args.steps, "logits_bytes": 4 * model.vocab}
    for k in arms:
        tot = [a + b for a, b in zip(t_sync[k], t_read[k])]
        res[f"{k}_step_ms"] = round(float(np.mean(tot)), 4)
        res[f"{k}_step_sem_ms"] = round(sem(tot), 5)
        if k in ("pinned_readback", "pageable_readback"):
            res[f"{k}_read_us"] = round(1e3 * float(np.mean(t_read[k])), 2)
            res[f"{k}_read_GB_s"] = round(4 * model.vocab / (float(np.mean(t_read[k])) * 1e-3) / 1e9, 2)
    res["in_graph_host_copy_nodes"] = in_graph.info()["n_nodes"]
    in_graph.close()
    res["capture_ms_at_create"] = round(chain.capture_stats()["capture_ms"], 3)
    lazy = mq.DecodeChain(model, W, X, flags=mq.MQ_LAZY_CAPTURE)
    for _ in range(3):
        lazy.step(mq.MQ_GRAPH)
    torch.cuda.synchronize()
    res["lazy_capture_ms_at_third_step"] = round(lazy.capture_stats()["capture_ms"], 3)
    res["lazy_captured"] = bool(lazy.info()["captured"])
    lazy.close()
    log(f"host step latency: {res}")
    return res


def run_decode(args, model, cpu_layers, probe=None):
    import torch
    from block_quantized_gemv_amd import binding as mq
    from block_quantized_gemv_amd import synth
    dev = torch.device("cuda:0")
    probe = probe or stream_probe(mq)
    log(f"generating and uploading {model.weight_bytes() / 1e9:.2f} GB of weights")
    W, host_w = upload_model(model, dev, keep_host=not args.no_cpu_baseline)
    X = torch.from_numpy(synth.normal_f32(model.seed, (synth.KEY_STEP_INPUTS,), (16, model.hidden))).to(dev)
    chain = mq.DecodeChain(model, W, X)
    eager = mq.DecodeChain(model, W, X, flags=mq.MQ_EAGER_ONLY)
    info = chain.info()
    log(f"chain captured={info['captured']} nodes={info['n_nodes']}")
    for _ in range(args.warmup):
        chain.step(mq.MQ_GRAPH)
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        chain.step(mq.MQ_GRAPH)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = wall * 1e3 / args.steps
    log(f"graph: {ms:.4f} ms/step wall, event mean {np.mean(per_step):.4f} sem {sem(per_step):.4f}")

    stamps = None if args.no_stamps else span_stamps(args, mq, model, W, X)
    sync = None if args.no_stamps else sync_probe(mq, model, stamps)
    ab = None if args.no_ab else interleaved_arms(args, mq, model, W, X, chain, eager)
    lat = None if args.no_ab else host_step_latency(args, mq, model, W, X, chain)

    roof, kernel_sum_ms = time_kernels(mq, model, eager, args.kernel_reps)
    roof["frac_of_stream_probe"] = round(roof["achieved"] / probe["GB_s"], 4)
    roof["q4k_layer_aggregate"]["frac_of_stream_probe"] = round(roof["q4k_layer_aggregate"]["GB_s"] / probe["GB_s"], 4)
    log(f"dominant kernel {roof['kernel']}: {roof['achieved']} GB/s per launch "
        f"({roof['frac'] * 100:.1f}% of 8 TB/s); GEMV kernel sum {kernel_sum_ms:.3f} ms/step")
    nbytes = model.algorithmic_bytes()
    value = nbytes / (ms * 1e-3) / 1e9
    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": model.name, "hidden": model.hidden, "layers": model.n_layers,
                      "qkv_rows": model.qkv_rows, "o_k": model.o_in, "inter": model.inter, "vocab": model.vocab,
                      "n": 1,
                      "seed": model.seed, "weights": f"{model.weight_format} (lm_head q8_0)", "graph": bool(info["captured"]),
                      "graph_nodes": info["n_nodes"], "bytes_per_step": nbytes},
           "tok_per_s": round(1e3 / ms, 2), "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
           "pct_of_stream_probe": round(100 * value / probe["GB_s"], 2), "stream_probe": probe,
           "step_event_ms": round(float(np.mean(per_step)), 4), "step_event_sem_ms": round(sem(per_step), 5),
           "gemv_kernel_sum_ms": round(kernel_sum_ms, 4),
           "roofline": roof}
    if stamps and roof["kernel"].startswith("mq::k_gemv_q4k_swiglu"):
        us = stamps["per_kernel_us"]["gate_up"]
        roof["in_graph_stamped_us_per_launch"] = us
        roof["frac_in_graph_stamped"] = round(roof["bytes_per_launch"] / us / 1e3 / HBM_PEAK_GBS, 4)
    if stamps:
        out["span_stamps"] = stamps
    if sync:
        out["sync_probe"] = sync
    if ab:
        out["ab_interleaved"] = ab
    if lat:
        out["host_step_latency"] = lat
    chain.close()
    eager.close()
    del W
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline_decode(model, host_w, cpu_layers)
    return out


# ------------------------------------------------------------ other workloads ----

def run_single(args):
    import torch
    from block_quantized_gemv_amd import binding as mq
    from block_quantized_gemv_amd import synth, workloads
    wl = workloads.SINGLE
    dev = torch.device("cuda:0")
    # cold: rotate enough copies that the working set (>= 1.2 GB) exceeds every cache
    copies = 2048
    base = synth.q4k_matrix(wl.seed, (synth.KEY_MATRIX,), wl.m, wl.k)
    W = torch.from_numpy(base).to(dev).repeat(copies, 1).view(copies, -1)
    xq = mq.mq_quantize_q8_0(torch.from_numpy(synth.normal_f32(wl.seed, (synth.KEY_COLUMNS,), (wl.k,))).to(dev))
    y = torch.empty(wl.m, dtype=torch.float32, device=dev)
    res = {}
    for mode in ("hot", "cold"):
        for i in range(args.warmup):
            mq.mq_gemv_q4k_q8(W[0 if mode == "hot" else i % copies], xq, wl.m, wl.k, y=y)
        torch.cuda.synchronize()
        evs = []
        for i in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            mq.mq_gemv_q4k_q8(W[0 if mode == "hot" else (i * 7) % copies], xq, wl.m, wl.k, y=y)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        res[mode] = {"us": round(float(np.median(us)), 3), "sem_us": round(sem(us), 4),
                     "GB_s": round(wl.algorithmic_bytes() / float(np.median(us)) / 1e3, 1)}
    out = {"metric": METRIC, "value": res["cold"]["GB_s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": res["cold"]["us"] / 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": wl.name, "m": wl.m, "k": wl.k, "seed": wl.seed}, "modes": res}
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.Oracle()
        xqh = o.quantize_q8_0(synth.normal_f32(wl.seed, (synth.KEY_COLUMNS,), (wl.k,))).ravel()
        _pin_one_core()
        ts = []
        for _ in range(20):
            t0 = time.perf_counter()
            o.gemv_q4k(base, wl.m, wl.k, xqh)
            ts.append(time.perf_counter() - t0)
        med = float(np.median(ts))
        out["cpu_baseline"] = _cpu_line(wl.algorithmic_bytes(), med, "median of 20 runs of the whole GEMV",
                                        us_per_gemv=round(med * 1e6, 1))
    return out


def run_batched(args):
    import torch
    from block_quantized_gemv_amd import binding as mq
    from block_quantized_gemv_amd import synth, workloads
    wl = workloads.BATCHED
    dev = torch.device("cuda:0")
    rows = {}
    host_gu = None
    for (m, k) in wl.shapes:
        reps = max(2, int(math.ceil(1.2e9 / workloads.q4k_bytes(m, k))))
        Wh = synth.q4k_matrix(wl.seed, (synth.KEY_MATRIX, m, k), m, k)
        if (m, k) == (37888, 3584):
            host_gu = Wh
        W = torch.from_numpy(Wh).to(dev)
        Ws = [W] + [W.clone() for _ in range(reps - 1)]
        for n in (1,) + tuple(wl.ns):
            xq = mq.mq_quantize_q8_0(torch.from_numpy(synth.normal_f32(wl.seed, (synth.KEY_COLUMNS, n, k), (n, k))).to(dev))
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            for i in range(args.warmup):
                mq.mq_gemv_q4k_q8_batched(Ws[i % reps], xq, m, k, n, y=y)
            evs = []
            for i in range(args.steps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                mq.mq_gemv_q4k_q8_batched(Ws[i % reps], xq, m, k, n, y=y)
                b.record()
                evs.append((a, b))
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))
            nbytes = workloads.q4k_bytes(m, k) + workloads.q8_bytes(n, k) + 4 * m * n
            rows[f"{m}x{k} n={n}"] = {"us": round(us, 2), "GB_s": round(nbytes / us / 1e3, 1)}
            log(f"{m}x{k} n={n}: {us:.2f} us, {nbytes / us / 1e3:.1f} GB/s")
        del Ws, W
        torch.cuda.empty_cache()
    best = rows[f"37888x3584 n=8"]["GB_s"]
    out = {"metric": METRIC, "value": best, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": rows["37888x3584 n=8"]["us"] / 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": wl.name, "seed": wl.seed, "value_is": "7B gate/up n=8, cold"}, "shapes": rows}
    if not args.no_cpu_baseline and host_gu is not None:
        import oracle
        o = oracle.Oracle()
        m, k, n = 37888, 3584, 8
        xq = o.quantize_q8_0(synth.normal_f32(wl.seed, (synth.KEY_COLUMNS, n, k), (n, k))).reshape(n, -1)
        _pin_one_core()
        t0 = time.perf_counter()
        for c in range(n):
            o.gemv_q4k(host_gu, m, k, xq[c])
        dt = time.perf_counter() - t0
        nbytes = workloads.q4k_bytes(m, k) + workloads.q8_bytes(n, k) + 4 * m * n
        out["cpu_baseline"] = _cpu_line(nbytes, dt, "the 37888x3584 gate/up shape with n = 8 columns, one oracle "
                                        "GEMV per column", ms_per_call=round(dt * 1e3, 1))
    return out


def run_moe(args):
    import torch
    from block_quantized_gemv_amd import binding as mq
    from block_quantized_gemv_amd import synth, workloads
    wl = workloads.MOE
    dev = torch.device("cuda:0")
    H, I = wl.hidden, wl.inter
    gu_h = np.stack([synth.q4k_matrix(wl.seed, (synth.KEY_EXPERT, e, 0), 2 * I, H) for e in range(wl.n_experts)])
    dn_h = np.stack([synth.q4k_matrix(wl.seed, (synth.KEY_EXPERT, e, 1), H, I) for e in range(wl.n_experts)])
    gu, dn = torch.from_numpy(gu_h).to(dev), torch.from_numpy(dn_h).to(dev)
    T = wl.n_tokens
    ids, logits = synth.routing(wl.seed, T, wl.n_experts, wl.n_sel)
    X = synth.normal_f32(wl.seed, (synth.KEY_TOKEN_X,), (T, H))
    tables = (torch.from_numpy(ids).to(dev), torch.from_numpy(logits).to(dev), torch.from_numpy(X).to(dev))
    per = 8    # tokens per graph launch (one launch per token is host-bound)

    def make(flags=0, tpl=per):
        return mq.MoEChain(wl.n_experts, wl.n_sel, H, I, gu.view(-1), gu[0].numel(), dn.view(-1), dn[0].numel(),
                           *tables, flags=flags, tokens_per_launch=tpl)

    chain = make()
    for _ in range(args.warmup):
        chain.step()
    chain.reset(0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(T // per):
        chain.step()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = wall * 1e6 / (T // per * per)
    # interleaved arms in blocks of 104 tokens (a token takes ~20 us, less
    # than the host needs to submit it with events around it): graphs of 8
    # and of 1 token per launch, and the same kernels launched eagerly (each
    # chain with its own token counter)
    arms = {"graph_8_per_launch": (chain, mq.MQ_GRAPH, per), "graph_1_per_launch": (make(tpl=1), mq.MQ_GRAPH, 1),
            "eager": (make(flags=mq.MQ_EAGER_ONLY, tpl=1), mq.MQ_EAGER, 1)}
    chain.reset(0)
    rounds, block = 10, 104
    evs = {k: [] for k in arms}
    for _ in range(rounds):
        for k, (arm, mode, tpl) in arms.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(block // tpl):
                arm.step(mode)
            e1.record()
            evs[k].append((e0, e1))
    torch.cuda.synchronize()
    ab = {"rounds": rounds, "tokens_per_block": block}
    for k, v in evs.items():
        t = [e0.elapsed_time(e1) * 1e3 / block for e0, e1 in v]
        ab[f"{k}_us_per_token"] = round(float(np.mean(t)), 3)
        ab[f"{k}_sem_us"] = round(sem(t), 4)
    for k, (arm, _, _) in arms.items():
        if arm is not chain:
            arm.close()
    log(f"interleaved A/B: {ab}")
    nbytes = wl.token_weight_bytes()
    out = {"metric": METRIC, "value": round(nbytes / us / 1e3, 1), "unit": "GB/s", "n_gpus": 1, "steps": T,
           "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "int8", "data": "synthetic",
           "config": {"workload": wl.name, "seed": wl.seed, "tokens": T, "tokens_per_graph_launch": per,
                      "bytes_per_token_padded": nbytes},
           "us_per_token": round(us, 3), "event_us_per_token": round(a.elapsed_time(b) * 1e3 / (T // per * per), 3),
           "tokens_per_s": round(1e6 / us, 1), "ab_interleaved": ab}
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.Oracle()
        gu_all, dn_all = gu_h.reshape(-1), dn_h.reshape(-1)
        n_cpu = 16
        _pin_one_core()
        t0 = time.perf_counter()
        for t in range(n_cpu):
            o.moe_token(gu_all, gu_h[0].nbytes, dn_all, dn_h[0].nbytes, ids[t], logits[t], X[t], H, I)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = _cpu_line(nbytes * n_cpu, dt, f"the first {n_cpu} of the {T} tokens",
                                        ms_per_token=round(dt * 1e3 / n_cpu, 2))
    return out


TP8_COLLECTIVES = ("not run: a tensor-parallel step adds two all-reduces of the 14,336-byte f32 hidden "
                   "vector per layer (after O and after down) and gathers the lm_head's vocabulary slices")


def other_configs(args, probe, full_step_ms=None):
    """Compact results of the other workloads (0.5B step, single GEMV,
    batched 7B shapes, routed-expert token, one tensor-parallel rank of the
    7B step), GPU side only, for the default line: each with its time, its
    algorithmic-byte rate and that rate as a fraction of 8 TB/s."""
    import copy
    from block_quantized_gemv_amd import workloads
    a = copy.copy(args)
    a.steps, a.warmup, a.no_cpu_baseline, a.no_ab, a.kernel_reps = min(args.steps, 100), 10, True, True, 1

    def frac(gbs):
        return round(gbs / HBM_PEAK_GBS, 4)

    out = {}
    t0 = time.perf_counter()
    d = run_decode(a, workloads.DECODE_05B, cpu_layers=0, probe=probe)
    out["c1_05b_decode_step"] = {"workload": d["config"]["workload"], "ms_per_step": d["ms_per_step"],
                                 "tok_per_s": d["tok_per_s"], "GB_s": d["value"], "frac_of_8TBs": frac(d["value"]),
                                 "graph_nodes": d["config"]["graph_nodes"],
                                 "dominant_kernel_us": d["roofline"]["us_per_launch"]}
    if "span_stamps" in d:
        ss = d["span_stamps"]
        out["c1_05b_decode_step"].update({"replay_span_us": ss["replay_span_us"], "kernel_sum_us": ss["kernel_sum_us"],
                                          "span_over_kernel_sum": ss["span_over_sum"],
                                          "mean_gap_between_kernels_us": ss["mean_gap_between_kernels_us"]})
    if "sync_probe" in d:
        sp = d["sync_probe"]
        out["c1_05b_decode_step"].update({"best_grid_barrier_with_exchange_us": sp["best_barrier_with_exchange_us"],
                                          "graph_empty_kernel_us": sp["graph_empty_kernel_us"]})
    log(f"extra: 0.5B step {d['ms_per_step']} ms ({time.perf_counter() - t0:.1f} s)")
    s1 = run_single(a)
    out["c0_single_gemv"] = {"workload": s1["config"]["workload"],
                             "us_cold": s1["modes"]["cold"]["us"], "GB_s_cold": s1["modes"]["cold"]["GB_s"],
                             "frac_of_8TBs_cold": frac(s1["modes"]["cold"]["GB_s"]),
                             "us_hot": s1["modes"]["hot"]["us"], "GB_s_hot": s1["modes"]["hot"]["GB_s"],
                             "note": "launch-latency bound (0.6 MB per GEMV)"}
    log(f"extra: single GEMV {s1['modes']['cold']['us']} us ({time.perf_counter() - t0:.1f} s)")
    b = run_batched(a)
    out["c3_batched_7b_shapes"] = {"workload": b["config"]["workload"],
                                   "cold_median_us": {k: {"us": v["us"], "GB_s": v["GB_s"], "frac_of_8TBs": frac(v["GB_s"])}
                                                      for k, v in b["shapes"].items()}}
    log(f"extra: batched ({time.perf_counter() - t0:.1f} s)")
    m = run_moe(a)
    out["c4_moe_token"] = {"workload": m["config"]["workload"], "us_per_token": m["us_per_token"],
                           "tokens_per_s": m["tokens_per_s"], "GB_s": m["value"], "frac_of_8TBs": frac(m["value"]),
                           "tokens_per_graph_launch": m["config"]["tokens_per_graph_launch"]}
    log(f"extra: routed-expert token {m['us_per_token']} us ({time.perf_counter() - t0:.1f} s)")
    a.no_stamps = True
    r = run_decode(a, workloads.DECODE_7B_TP8, cpu_layers=0, probe=probe)
    out["tp8_rank_7b_decode_step"] = {"workload": r["config"]["workload"], "ms_per_step": r["ms_per_step"],
                                      "GB_s": r["value"], "frac_of_8TBs": frac(r["value"]),
                                      "bytes_per_step": r["config"]["bytes_per_step"],
                                      "graph_nodes": r["config"]["graph_nodes"],
                                      "per_kernel_us": {k: v["us"] for k, v in r["roofline"]["per_shape"].items()},
                                      "collectives": TP8_COLLECTIVES}
    if full_step_ms:
        out["tp8_rank_7b_decode_step"]["full_step_over_rank_step"] = round(full_step_ms / r["ms_per_step"], 3)
    log(f"extra: tensor-parallel rank step {r['ms_per_step']} ms ({time.perf_counter() - t0:.1f} s)")
    return out


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the row-sharded multi-GPU design is described, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    from block_quantized_gemv_amd import workloads
    if args.workload == "7b":
        from block_quantized_gemv_amd import binding as mq
        probe = stream_probe(mq)
        out = run_decode(args, workloads.DECODE_7B, cpu_layers=workloads.DECODE_7B.n_layers, probe=probe)
        if not args.no_extra:
            out["other_configs"] = other_configs(args, probe, out["ms_per_step"])
    elif args.workload == "05b":
        out = run_decode(args, workloads.DECODE_05B, cpu_layers=workloads.DECODE_05B.n_layers)
    elif args.workload == "05b_q4_0":
        out = run_decode(args, workloads.DECODE_05B_Q4_0, cpu_layers=workloads.DECODE_05B_Q4_0.n_layers)
    elif args.workload == "7b_tp8":
        out = run_decode(args, workloads.DECODE_7B_TP8, cpu_layers=workloads.DECODE_7B_TP8.n_layers)
        out["config"]["collectives"] = TP8_COLLECTIVES
    elif args.workload == "single":
        out = run_single(args)
    elif args.workload == "batched":
        out = run_batched(args)
    else:
        out = run_moe(args)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
