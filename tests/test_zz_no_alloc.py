"""The no-allocation batched GEMV (mq_gemv_q4k_q8_batched_noalloc) against
the allocating entry point, through the C ABI: two split-k calls in a row,
the second with a smaller input, then a one-pass shape; the results must
be byte-identical, and no split-k workspace may appear."""
import numpy as np
import pytest

from gpu_helpers import log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available()
    from block_quantized_gemv_amd import binding
    binding.lib()
    return binding


def test_no_alloc_matches_the_allocating_entry_point(mq):
    import torch
    import oracle
    from block_quantized_gemv_amd import synth
    o = oracle.Oracle()
    mq.mq_workspace_release()
    # (m, k, n): the 7B down projection at n = 8 (the matrix cores, ten k
    # ranges, 2.2 MiB of partials), a smaller split-k call of the vector
    # kernels after it, then a one-pass shape
    cases = [(3584, 18944, 8), (515, 18944, 4), (301, 2560, 3)]
    assert [mq.mq_gemv_batched_path(m, k, n) for m, k, n in cases] == [1, 0, 0]
    outs = []
    for m, k, n in cases:
        log(f"no-alloc batched {m}x{k} n={n}")
        w = to_dev(synth.q4k_matrix(13, (synth.KEY_MATRIX, m, k), m, k))
        xq = to_dev(o.quantize_q8_0(synth.normal_f32(13, (synth.KEY_COLUMNS, n, k), (n, k))).ravel())
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        mq.mq_gemv_q4k_q8_batched_noalloc(w, xq, m, k, n, y)
        outs.append((w, xq, to_host(y).copy()))
    assert mq.mq_workspace_stats()["bytes"] == 0, "the no-allocation entry point created a workspace"
    for (m, k, n), (w, xq, got) in zip(cases, outs):
        want = to_host(mq.mq_gemv_q4k_q8_batched(w, xq, m, k, n)).copy()
        assert np.isfinite(got).all(), f"{m}x{k} n={n}: outputs left unwritten"
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{m}x{k} n={n} differs"
    # a size beyond the fixed scratch is refused on the host
    big_m = 14000
    w = torch.empty(big_m * 74 * 144, dtype=torch.uint8, device="cuda")
    xq = torch.empty(8 * 592 * 34, dtype=torch.uint8, device="cuda")
    y = torch.empty((big_m, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(mq.MQError) as e:
        mq.mq_gemv_q4k_q8_batched_noalloc(w, xq, big_m, 18944, 8, y)
    assert e.value.code == mq.MQ_ERR_SHAPE and "scratch" in str(e.value)


def test_no_alloc_under_graph_capture(mq):
    """The entry point inside a captured graph (the callers it exists for):
    the graph is replayed four times, with eager GEMVs and synchronizations
    between the replays, and every replay's output must equal the eager
    output byte for byte.  Shapes: the matrix-core path with k split into
    ranges (partials in the fixed array), and the vector kernels' split-k."""
    import torch
    import oracle
    from block_quantized_gemv_amd import synth
    o = oracle.Oracle()
    for m, k, n in ((2049, 8192, 8), (515, 18944, 3)):
        assert mq.mq_gemv_batched_path(m, k, n) == (1 if n == 8 else 0)
        log(f"no-alloc batched under capture {m}x{k} n={n}")
        w = to_dev(synth.q4k_matrix(17, (synth.KEY_MATRIX, m, k), m, k))
        xq = to_dev(o.quantize_q8_0(synth.normal_f32(17, (synth.KEY_COLUMNS, n, k), (n, k))).ravel())
        y_eager = torch.empty((m, n), dtype=torch.float32, device="cuda")
        mq.mq_gemv_q4k_q8_batched_noalloc(w, xq, m, k, n, y_eager)
        want = to_host(y_eager).copy()
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                mq.mq_gemv_q4k_q8_batched_noalloc(w, xq, m, k, n, y)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        other = torch.empty((m, n), dtype=torch.float32, device="cuda")
        for r in range(4):
            y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            got = to_host(y).copy()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{m}x{k} n={n}: replay {r} differs"
            # eager work on the same fixed array between replays
            mq.mq_gemv_q4k_q8_batched_noalloc(w, xq, m, k, n, other)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(other).view(np.uint32), want.view(np.uint32))
        del g
