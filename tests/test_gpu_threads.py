"""The threading contract of the C ABI: several host threads, each on its
own stream, call the stateless entry points at once; the split-k
workspace is kept per (device, stream), created by each stream's first
split-k call, and only grows."""
import threading

import numpy as np
import pytest

from gpu_helpers import log, to_dev, to_host

pytestmark = pytest.mark.gpu

N_THREADS = 8


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available()
    from block_quantized_gemv_amd import binding
    binding.lib()
    return binding


def _inputs():
    from block_quantized_gemv_amd import synth
    import oracle
    o = oracle.Oracle()
    w1 = synth.q4k_matrix(12, (synth.KEY_MATRIX, 1), 3584, 3584)
    x1 = o.quantize_q8_0(synth.normal_f32(12, (synth.KEY_COLUMNS, 1), (3584,))).ravel()
    w8 = synth.q4k_matrix(12, (synth.KEY_MATRIX, 8), 3584, 18944)
    x8 = o.quantize_q8_0(synth.normal_f32(12, (synth.KEY_COLUMNS, 8), (8, 18944))).ravel()
    w4 = synth.q4_0_matrix(12, (synth.KEY_MATRIX, 4), 3584, 18944)
    wq = synth.q8_0_matrix(12, (synth.KEY_MATRIX, 3), 4096, 1024)
    xq = o.quantize_q8_0(synth.normal_f32(12, (synth.KEY_COLUMNS, 3), (1024,))).ravel()
    return [to_dev(a) for a in (w1, x1, w8, x8, w4, wq, xq)]


def _calls(mq, d, stream):
    w1, x1, w8, x8, w4, wq, xq = d
    return [mq.mq_gemv_q4k_q8(w1, x1, 3584, 3584, stream=stream),
            mq.mq_gemv_q4k_q8_batched(w8, x8, 3584, 18944, 8, stream=stream),     # split-k: 5 splits
            mq.mq_gemv_q4_0_q8_batched(w4, x8, 3584, 18944, 4, stream=stream),
            mq.mq_gemv_q8_0_q8(wq, xq, 4096, 1024, stream=stream)]


def _same(a, b):
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_threads_on_their_own_streams(mq):
    """8 threads released together by a barrier, 4 rounds of the same calls
    each (n = 1, batched n = 8 and q4_0 n = 4 through split-k, the q8_0
    GEMV); every result byte-identical to the single-threaded one, and one
    workspace per thread's stream."""
    import torch
    d = _inputs()
    ref = [to_host(t).copy() for t in _calls(mq, d, None)]
    torch.cuda.synchronize()
    mq.mq_workspace_release()
    assert mq.mq_workspace_stats() == {"bytes": 0, "streams": 0, "retired": 0}
    barrier = threading.Barrier(N_THREADS, timeout=120)
    results, errors = {}, {}

    def worker(i):
        try:
            s = torch.cuda.Stream()
            barrier.wait()
            outs = []
            for _ in range(4):
                outs.append(_calls(mq, d, s))
            s.synchronize()
            results[i] = [[to_host(t).copy() for t in r] for r in outs]
        except Exception as e:          # reported by the main thread
            errors[i] = repr(e)
            barrier.abort()

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(N_THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=300)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i in range(N_THREADS):
        for r, outs in enumerate(results[i]):
            for j, (u, v) in enumerate(zip(outs, ref)):
                assert _same(u, v), f"thread {i} round {r} call {j} differs from the single-threaded result"
    st = mq.mq_workspace_stats()
    log(f"workspaces after the threads: {st}")
    assert st["streams"] == N_THREADS and st["retired"] == 0


def test_workspace_grows_and_keeps_the_outgrown_buffer(mq):
    """On a fresh stream: a small split-k call, then a larger one that must
    grow the stream's workspace; the outgrown buffer is kept, both results
    equal the default stream's, and release frees everything."""
    import torch
    w1, x1, w8, x8, w4, wq, xq = _inputs()
    small_ref = to_host(mq.mq_gemv_q4k_q8_batched(w8[:64 * 74 * 144], x8, 64, 18944, 8)).copy()
    big_ref = to_host(mq.mq_gemv_q4k_q8_batched(w8, x8, 3584, 18944, 8)).copy()
    mq.mq_workspace_release()
    s = torch.cuda.Stream()
    small = mq.mq_gemv_q4k_q8_batched(w8[:64 * 74 * 144], x8, 64, 18944, 8, stream=s)
    st1 = mq.mq_workspace_stats()
    big = mq.mq_gemv_q4k_q8_batched(w8, x8, 3584, 18944, 8, stream=s)
    st2 = mq.mq_workspace_stats()
    s.synchronize()
    log(f"workspace after the small call {st1}, after the large one {st2}")
    assert st1["streams"] == 1 and st1["retired"] == 0 and st1["bytes"] == 1 << 20
    grown = st2["bytes"] - (1 << 20)            # the outgrown 1 MiB buffer is kept beside the new one
    assert st2["streams"] == 1 and st2["retired"] == 1
    assert grown >= 1 << 21 and grown & (grown - 1) == 0, st2
    assert _same(to_host(small), small_ref) and _same(to_host(big), big_ref)
    mq.mq_workspace_release()
    assert mq.mq_workspace_stats() == {"bytes": 0, "streams": 0, "retired": 0}
