"""The C ABI on the CPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before any HIP call."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mq.h")


@pytest.fixture(scope="module")
def mq():
    from block_quantized_gemv_amd import binding, build
    if not os.path.exists(binding.LIBRARY):
        build.build()
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("mq_quantize_q8_0", "mq_gemv_q4k_q8", "mq_gemv_q4k_q8_batched", "mq_gemv_q4k_grouped",
                     "mq_decode_chain", "mq_chain_create", "mq_gemv_q8_0_q8"):
        assert required in names


def test_every_declared_symbol_is_exported(mq):
    lib = mq.lib()
    raw = C.CDLL(mq.LIBRARY)
    for name in declared_functions():
        assert hasattr(raw, name), f"{name} declared in mq.h but not exported"
        assert name in mq.SIGNATURES, f"{name} has no Python binding"
    assert lib.mq_version().decode().startswith("libmq")


FAKE = C.c_void_p(0x10000)     # aligned, never dereferenced: validation fails first


def test_gemv_argument_errors(mq):
    L = mq.lib()
    assert L.mq_gemv_q4k_q8(None, FAKE, FAKE, 16, 256, None) == mq.MQ_ERR_ARG
    assert "null" in L.mq_last_error().decode()
    assert L.mq_gemv_q4k_q8(C.c_void_p(0x10008), FAKE, FAKE, 16, 256, None) == mq.MQ_ERR_ARG   # not 16-aligned
    assert L.mq_gemv_q4k_q8(FAKE, FAKE, FAKE, 16, 300, None) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_q4k_q8(FAKE, FAKE, FAKE, 0, 256, None) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_q4k_q8(FAKE, FAKE, FAKE, (1 << 30) + 1, 256, None) == mq.MQ_ERR_SHAPE   # rows above 2^30
    assert L.mq_gemv_q4k_q8(FAKE, FAKE, FAKE, 16, (1 << 24) + 256, None) == mq.MQ_ERR_SHAPE  # k above 2^24
    assert L.mq_gemv_q4_0_q8(FAKE, FAKE, FAKE, (1 << 30) + 1, 256, None) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_q4k_q8_batched(FAKE, FAKE, FAKE, 16, 256, 9, None) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_q4k_q8_batched(FAKE, FAKE, FAKE, 16, 256, 0, None) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_q8_0_q8(FAKE, FAKE, FAKE, 16, 96, None) == mq.MQ_ERR_SHAPE
    assert L.mq_quantize_q8_0(FAKE, FAKE, 33, 1, None) == mq.MQ_ERR_SHAPE
    assert L.mq_quantize_q8_0(FAKE, C.c_void_p(0x10001), 32, 1, None) == mq.MQ_ERR_ARG
    assert L.mq_swiglu_quantize_q8_0(FAKE, FAKE, 64, 1, 32, None) == mq.MQ_ERR_SHAPE
    assert L.mq_rmsnorm_quantize_q8_0(FAKE, FAKE, 64, -1.0, None) == mq.MQ_ERR_ARG
    assert L.mq_gemv_q4_0_q8(FAKE, FAKE, FAKE, 16, 288, None) == mq.MQ_ERR_SHAPE             # k % 256
    assert L.mq_gemv_q4_0_q8(C.c_void_p(0x10004), FAKE, FAKE, 16, 256, None) == mq.MQ_ERR_ARG
    assert L.mq_gemv_q4_0_q8_batched(FAKE, FAKE, FAKE, 16, 256, 9, None) == mq.MQ_ERR_SHAPE
    assert L.mq_debug_gemv_q4_0_q8_isums(FAKE, FAKE, FAKE, None, None, 16, 256, None) == mq.MQ_ERR_ARG
    assert L.mq_debug_gemv_q4_0_q8_isums(FAKE, FAKE, FAKE, FAKE, None, 16, 256 * 300, None) == mq.MQ_ERR_SHAPE


def test_stream_probe_argument_errors(mq):
    L = mq.lib()
    assert L.mq_probe_stream_read(FAKE, 64, None, 0, None) == mq.MQ_ERR_ARG                  # null xor_out
    assert L.mq_probe_stream_read(None, 64, FAKE, 0, None) == mq.MQ_ERR_ARG                  # null buffer
    assert L.mq_probe_stream_read(C.c_void_p(0x10008), 64, FAKE, 0, None) == mq.MQ_ERR_ARG   # not 16-aligned
    assert L.mq_probe_stream_read(FAKE, 40, FAKE, 0, None) == mq.MQ_ERR_ARG                  # not a multiple of 16
    assert L.mq_probe_stream_read(FAKE, 64, FAKE, 70000, None) == mq.MQ_ERR_ARG              # workgroups
    us, bad = C.c_double(), C.c_uint32()
    assert L.mq_probe_grid_barrier(2, 4, 10, 512, C.byref(us), C.byref(bad), None) == mq.MQ_ERR_ARG   # hierarchical
    assert L.mq_probe_grid_barrier(0, 5000, 10, 512, C.byref(us), C.byref(bad), None) == mq.MQ_ERR_ARG
    assert L.mq_probe_grid_barrier(0, 4, 0, 512, C.byref(us), C.byref(bad), None) == mq.MQ_ERR_ARG    # rounds
    assert L.mq_probe_grid_barrier(0, 4, 10, 100, C.byref(us), C.byref(bad), None) == mq.MQ_ERR_ARG   # threads
    assert L.mq_probe_grid_barrier(0, 4, 10, 512, None, C.byref(bad), None) == mq.MQ_ERR_ARG
    assert L.mq_probe_graph_boundary(0, 512, 10, C.byref(us)) == mq.MQ_ERR_ARG
    assert L.mq_probe_graph_boundary(10, 512, 10, None) == mq.MQ_ERR_ARG


def test_readback_argument_errors(mq):
    L = mq.lib()
    buf = (C.c_uint8 * 64)()
    assert L.mq_read_to_host(FAKE, buf, 64, 4, None) == mq.MQ_ERR_ARG              # unknown flag
    assert "flags" in L.mq_last_error().decode()
    assert L.mq_read_to_host(FAKE, buf, -1, 0, None) == mq.MQ_ERR_ARG              # negative size
    assert L.mq_read_to_host(None, buf, 64, 0, None) == mq.MQ_ERR_ARG              # null source
    assert L.mq_read_to_host(FAKE, None, 64, mq.MQ_READ_PAGEABLE, None) == mq.MQ_ERR_ARG
    assert L.mq_chain_read_logits(None, C.cast(buf, C.c_void_p), 16, 0, None) == mq.MQ_ERR_ARG
    assert L.mq_chain_capture_stats(None, None, None) == mq.MQ_ERR_ARG
    assert L.mq_chain_host_logits(None, C.byref(C.c_void_p())) == mq.MQ_ERR_ARG
    # no pinned buffer exists before the first read; releasing none is fine
    assert L.mq_readback_release() == mq.MQ_OK
    assert mq.mq_readback_stats() == {"pinned_bytes": 0, "pinned_reads": 0, "pageable_reads": 0, "warned": False}


def test_grouped_argument_errors(mq):
    L = mq.lib()
    # combine without y_out
    assert L.mq_gemv_q4k_grouped(FAKE, 144 * 16, 4, FAKE, 2, FAKE, 0, FAKE, FAKE, None, 16, 256, None) == mq.MQ_ERR_ARG
    # expert_bytes smaller than one matrix
    assert L.mq_gemv_q4k_grouped(FAKE, 144, 4, FAKE, 2, FAKE, 0, FAKE, None, None, 16, 256, None) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_q4k_grouped(FAKE, 144 * 16, 4, FAKE, 17, FAKE, 0, FAKE, None, None, 16, 256, None) == mq.MQ_ERR_SHAPE


def test_chain_argument_errors(mq):
    L = mq.lib()
    out = C.c_void_p()
    arr = (C.c_void_p * 1)(FAKE.value)
    d = mq.ChainDesc(1, 1000, 1280, 4864, 100, arr, arr, arr, arr, FAKE, FAKE, 1, FAKE, 1e-6, 0)
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_SHAPE        # hidden % 256
    d.hidden, d.n_inputs = 1024, 0
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_ARG          # n_inputs
    d.n_inputs, d.qkv_rows = 1, 512
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_SHAPE        # qkv_rows < hidden
    d.qkv_rows, d.o_k = 1280, 100
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_SHAPE        # o_k % 256
    d.o_k = 2048
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_SHAPE        # o_k > hidden
    d.o_k, d.qkv_rows = 512, 256
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_SHAPE        # qkv_rows < o_k
    assert "o_k" in L.mq_last_error().decode()
    d.qkv_rows, d.o_k, d.weight_format = 1280, 0, 7
    assert L.mq_chain_create(C.byref(d), None, C.byref(out)) == mq.MQ_ERR_ARG          # weight_format
    assert "weight_format" in L.mq_last_error().decode()
    d.weight_format = mq.MQ_FMT_Q4_K
    assert L.mq_decode_chain(None, 0, None) == mq.MQ_ERR_ARG
    buf = (C.c_uint64 * 4)()
    assert L.mq_chain_read_stamps(None, buf, 2, None) == mq.MQ_ERR_ARG
    assert L.mq_chain_clear_stamps(None, None) == mq.MQ_ERR_ARG
    assert L.mq_chain_destroy(None) == mq.MQ_OK
    m = mq.MoEDesc(64, 8, 2048, 1408, FAKE, 16, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 10, 0)
    assert L.mq_moe_create(C.byref(m), None, C.byref(out)) == mq.MQ_ERR_SHAPE          # expert bytes too small
    m = mq.MoEDesc(64, 8, 2048, 1408, FAKE, 1 << 24, FAKE, 1 << 24, FAKE, FAKE, FAKE, FAKE, 10, 0, 257)
    assert L.mq_moe_create(C.byref(m), None, C.byref(out)) == mq.MQ_ERR_SHAPE          # tokens_per_launch
    assert L.mq_test_set_fault(0) == mq.MQ_OK


def test_workspace_and_gate_up_hook_on_the_host(mq):
    L = mq.lib()
    # no split-k call has run in this process: nothing held, releasing nothing is fine
    assert mq.mq_workspace_stats() == {"bytes": 0, "streams": 0, "retired": 0}
    assert L.mq_workspace_release() == mq.MQ_OK
    g = L.mq_debug_gate_up_swiglu
    assert g(None, FAKE, 1e-6, None, FAKE, 64, 256, 0, None, None, 0, None) == mq.MQ_ERR_ARG          # null w
    assert g(FAKE, FAKE, 1e-6, None, FAKE, 48, 256, 0, None, None, 0, None) == mq.MQ_ERR_SHAPE        # inter % 32
    assert g(FAKE, FAKE, 1e-6, None, FAKE, 64, 300, 0, None, None, 0, None) == mq.MQ_ERR_SHAPE        # k % 256
    assert g(FAKE, FAKE, 1e-6, None, FAKE, 64, 256, -1, None, None, 0, None) == mq.MQ_ERR_ARG         # n_split
    assert g(FAKE, FAKE, 1e-6, None, FAKE, 64, 256, 0, None, None, 5, None) == mq.MQ_ERR_ARG          # format
    assert g(FAKE, C.c_void_p(0x10004), 1e-6, None, FAKE, 64, 256, 0, None, None, 0, None) == mq.MQ_ERR_ARG


def test_batched_path_rule(mq):
    """The kernel family of the batched entry points by shape, on the host:
    the matrix cores from n = 4 on 76 MB (7B gate/up) and on the 38 MB 7B
    down projection (whose vector kernels would split k at n = 4), from
    n = 6 on 33-38 MB matrices of short rows and on a 19 MB one whose vector
    kernels would split k at n = 6, from n = 7 on 9.3-16.5 MB ones (7B QKV),
    from n = 8 on the 7.2 MB 7B O, never on the 0.5B ones; q4_0 and a matrix
    past 32-bit offsets never."""
    cases = [((37888, 3584), 4), ((3584, 18944), 4), ((18944, 3584), 6), ((16384, 3584), 6),
             ((1792, 18944), 6), ((8192, 3584), 7), ((6144, 3584), 7), ((4608, 3584), 7), ((3584, 3584), 8),
             ((9728, 1024), 9), ((1280, 1024), 9), ((1024, 4864), 9), ((30_000_000, 256), 9)]
    for (m, k), first in cases:
        got = [mq.mq_gemv_batched_path(m, k, n) for n in range(1, 9)]
        assert got == [int(n >= first) for n in range(1, 9)], (m, k, got)
        assert all(mq.mq_gemv_batched_path(m, k, n, "q4_0") == 0 for n in range(1, 9))
    L = mq.lib()
    p = C.c_int()
    assert L.mq_gemv_batched_path(100, 256, 9, 0, C.byref(p)) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_batched_path(100, 300, 2, 0, C.byref(p)) == mq.MQ_ERR_SHAPE
    assert L.mq_gemv_batched_path(100, 256, 2, 3, C.byref(p)) == mq.MQ_ERR_ARG
    assert L.mq_gemv_batched_path(100, 256, 2, 0, None) == mq.MQ_ERR_ARG


def test_random_sweeps_reach_every_kernel_family(mq):
    """The seeded random GEMV sweep of the GPU tests keeps covering both
    kernel families of the batched entry point, one-pass and split-k vector
    shapes, and both weight formats (checked on the host, so that a change
    of the size rule cannot quietly narrow it)."""
    import test_gpu_kernels as tk
    cases = tk._sweep_cases()
    assert len(cases) == len(set(cases))
    paths = [mq.mq_gemv_batched_path(m, k, n, f) for f, m, k, n in cases]
    assert 1 in paths and 0 in paths
    assert {f for f, *_ in cases} == {"q4_K", "q4_0"}
    vec = [(m, k, n) for (f, m, k, n), p in zip(cases, paths) if p == 0 and n > 1]
    assert any(tk._single_pass(m, k, n) for m, k, n in vec) and not all(tk._single_pass(m, k, n) for m, k, n in vec)


def test_no_alloc_entry_point_refuses_on_the_host(mq):
    L = mq.lib()
    f = L.mq_gemv_q4k_q8_batched_noalloc
    assert f(None, FAKE, FAKE, 16, 256, 2, None) == mq.MQ_ERR_ARG
    assert f(FAKE, FAKE, FAKE, 16, 256, 9, None) == mq.MQ_ERR_SHAPE
    # 14000 rows x 8 columns x 5 splits of f64 partials exceed the fixed 4 MiB scratch
    assert f(FAKE, FAKE, FAKE, 14000, 18944, 8, None) == mq.MQ_ERR_SHAPE
    assert "scratch" in L.mq_last_error().decode()
