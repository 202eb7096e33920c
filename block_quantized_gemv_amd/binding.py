"""Thin ctypes binding of libmq: the C entry points under the same names.

Argument marshalling only: every step runs in the HIP library.  torch is
used for device memory and streams; the wrappers check dtype, device,
contiguity and byte counts, pass raw pointers and the current HIP stream,
and raise MQError on a non-zero status.  There is no CPU fallback: if
libmq.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libmq.so")

MQ_OK, MQ_ERR_ARG, MQ_ERR_SHAPE, MQ_ERR_HIP, MQ_ERR_CAPTURE, MQ_ERR_NOMEM = 0, -1, -2, -3, -4, -5
MQ_EAGER_ONLY, MQ_KEEP_INTERMEDIATES, MQ_EXACT_GLUE, MQ_UNFUSED_GLUE, MQ_LAZY_CAPTURE, MQ_HOST_LOGITS = 1, 2, 4, 8, 16, 32
MQ_SPAN_STAMPS = 64
MQ_GRAPH, MQ_EAGER = 0, 1
MQ_READ_PINNED, MQ_READ_PAGEABLE = 0, 1
MQ_FMT_Q4_K, MQ_FMT_Q4_0 = 0, 1
MQ_FAULT_NONE, MQ_FAULT_CAPTURE, MQ_FAULT_PINNED_ALLOC = 0, 1, 2

Q4K_BLOCK_BYTES, Q8_BLOCK_BYTES, Q4_0_BLOCK_BYTES = 144, 34, 18


class MQError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"libmq error {code}: {message}")
        self.code = code


_vp, _i64, _int, _f32, _u32 = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_uint


class ChainDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("hidden", C.c_int64), ("qkv_rows", C.c_int64),
                ("inter", C.c_int64), ("vocab", C.c_int64),
                ("w_qkv", C.POINTER(_vp)), ("w_o", C.POINTER(_vp)), ("w_gu", C.POINTER(_vp)),
                ("w_down", C.POINTER(_vp)), ("w_lm", _vp), ("x_table", _vp), ("n_inputs", C.c_int),
                ("logits", _vp), ("eps", C.c_float), ("flags", C.c_uint), ("weight_format", C.c_int),
                ("o_k", _i64)]


class MoEDesc(C.Structure):
    _fields_ = [("n_experts", C.c_int), ("n_sel", C.c_int), ("hidden", C.c_int64), ("inter", C.c_int64),
                ("w_gu_all", _vp), ("gu_expert_bytes", C.c_int64), ("w_dn_all", _vp),
                ("dn_expert_bytes", C.c_int64), ("ids_table", _vp), ("logits_table", _vp),
                ("x_table", _vp), ("y_table", _vp), ("n_tokens", C.c_int), ("flags", C.c_uint),
                ("tokens_per_launch", C.c_int)]


SIGNATURES = {
    "mq_last_error": ([], C.c_char_p),
    "mq_version": ([], C.c_char_p),
    "mq_quantize_q8_0": ([_vp, _vp, _i64, _int, _vp], _int),
    "mq_gemv_q4k_q8": ([_vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_gemv_q4k_q8_batched": ([_vp, _vp, _vp, _i64, _i64, _int, _vp], _int),
    "mq_gemv_q4k_q8_batched_noalloc": ([_vp, _vp, _vp, _i64, _i64, _int, _vp], _int),
    "mq_gemv_q4k_grouped": ([_vp, _i64, _int, _vp, _int, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_gemv_q8_0_q8": ([_vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_gemv_q4_0_q8": ([_vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_gemv_q4_0_q8_batched": ([_vp, _vp, _vp, _i64, _i64, _int, _vp], _int),
    "mq_debug_gemv_q4_0_q8_isums": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_rmsnorm_quantize_q8_0": ([_vp, _vp, _i64, _f32, _vp], _int),
    "mq_swiglu_quantize_q8_0": ([_vp, _vp, _i64, _int, _i64, _vp], _int),
    "mq_debug_gemv_q4k_q8_isums": ([_vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_debug_gemv_q8_0_q8_isums": ([_vp, _vp, _vp, _vp, _i64, _i64, _vp], _int),
    "mq_debug_gate_up_swiglu": ([_vp, _vp, _f32, _vp, _vp, _i64, _i64, _int, _vp, _vp, _int, _vp], _int),
    "mq_chain_create": ([C.POINTER(ChainDesc), _vp, C.POINTER(_vp)], _int),
    "mq_decode_chain": ([_vp, _int, _vp], _int),
    "mq_chain_info": ([_vp, C.POINTER(_int), C.POINTER(_int), C.POINTER(_i64)], _int),
    "mq_chain_reset": ([_vp, _i64, _vp], _int),
    "mq_chain_capture_stats": ([_vp, C.POINTER(_i64), C.POINTER(C.c_double)], _int),
    "mq_chain_read_logits": ([_vp, _vp, _i64, _u32, _vp], _int),
    "mq_chain_host_logits": ([_vp, C.POINTER(_vp)], _int),
    "mq_read_to_host": ([_vp, _vp, _i64, _u32, _vp], _int),
    "mq_readback_stats": ([C.POINTER(_i64), C.POINTER(_i64), C.POINTER(_i64), C.POINTER(_int)], _int),
    "mq_readback_release": ([], _int),
    "mq_workspace_stats": ([C.POINTER(_i64), C.POINTER(_int), C.POINTER(_int)], _int),
    "mq_workspace_release": ([], _int),
    "mq_chain_trace_sizes": ([_vp, C.POINTER(_i64), C.POINTER(_i64)], _int),
    "mq_chain_read_trace": ([_vp, _vp, _vp, _vp], _int),
    "mq_chain_read_stamps": ([_vp, _vp, _i64, _vp], _int),
    "mq_chain_clear_stamps": ([_vp, _vp], _int),
    "mq_chain_destroy": ([_vp], _int),
    "mq_moe_create": ([C.POINTER(MoEDesc), _vp, C.POINTER(_vp)], _int),
    "mq_moe_step": ([_vp, _int, _vp], _int),
    "mq_test_set_fault": ([_u32], _int),
    "mq_time_next_launches": ([C.POINTER(_vp), C.POINTER(_vp), _int], _int),
    "mq_probe_stream_read": ([_vp, _i64, _vp, _int, _vp], _int),
    "mq_probe_grid_barrier": ([_int, _int, _int, _int, _vp, _vp, _vp], _int),
    "mq_debug_gemv_q4k_batched_path": ([_vp, _vp, _vp, _i64, _i64, _int, _int, _vp], _int),
    "mq_gemv_batched_path": ([_i64, _i64, _int, _int, C.POINTER(_int)], _int),
    "mq_probe_graph_boundary": ([_int, _int, _int, _vp], _int),
}

_LIB = None


def lib():
    """The loaded libmq.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIBRARY)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _LIB = L
    return _LIB


def _check(rc: int):
    if rc != MQ_OK:
        raise MQError(rc, lib().mq_last_error().decode())


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _ptr(t, dtype=None, nbytes=None, what="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return t.data_ptr()


def q4k_bytes(m, k):
    return m * (-(-k // 256)) * Q4K_BLOCK_BYTES


def q8_bytes(n, k):
    return n * (k // 32) * Q8_BLOCK_BYTES


def q4_0_bytes(m, k):
    return m * (k // 32) * Q4_0_BLOCK_BYTES


def version() -> str:
    return lib().mq_version().decode()


def mq_test_set_fault(mask: int):
    _check(lib().mq_test_set_fault(mask))


def mq_time_next_launches(starts, stops):
    """Arm dispatch-timestamp events for this thread's next len(starts) GEMV
    launches (raw hipEvent_t handles as ints); empty lists clear the hook."""
    n = len(starts)
    a, b = (_vp * max(n, 1))(*starts), (_vp * max(n, 1))(*stops)
    _check(lib().mq_time_next_launches(a, b, n))


def mq_probe_grid_barrier(hierarchical, exchange_words, rounds=2000, threads=512, stream=None):
    """Grid-barrier probe (one workgroup per CU): (us per round, mismatched words)."""
    us, bad = C.c_double(), C.c_uint32()
    _check(lib().mq_probe_grid_barrier(int(hierarchical), exchange_words, rounds, threads, C.byref(us), C.byref(bad),
                                       _stream(stream)))
    return us.value, bad.value


def mq_probe_graph_boundary(n_kernels=200, threads=512, reps=10):
    """Microseconds per empty kernel in a graph replay (one workgroup per CU)."""
    us = C.c_double()
    _check(lib().mq_probe_graph_boundary(n_kernels, threads, reps, C.byref(us)))
    return us.value


def mq_probe_stream_read(buf, xor_out=None, workgroups=0, stream=None):
    """Streaming-read probe over the bytes of `buf` (a contiguous device
    tensor whose size is a multiple of 16); returns the uint32 device tensor
    holding the XOR of its 32-bit words."""
    nbytes = buf.numel() * buf.element_size()
    if xor_out is None:
        xor_out = torch.empty(1, dtype=torch.int32, device=buf.device)
    _check(lib().mq_probe_stream_read(_ptr(buf, what="buf"), nbytes, _ptr(xor_out, torch.int32, 4, "xor_out"),
                                      int(workgroups), _stream(stream)))
    return xor_out


def _host_out(out, dtype, shape, nbytes, what="out"):
    """A writable, C-contiguous numpy array of at least nbytes (new if None)."""
    if out is None:
        return np.empty(shape, dtype=dtype)
    if not isinstance(out, np.ndarray) or not out.flags.c_contiguous or not out.flags.writeable:
        raise TypeError(f"{what} must be a writable C-contiguous numpy array")
    if out.nbytes < nbytes:
        raise ValueError(f"{what} holds {out.nbytes} bytes, needs {nbytes}")
    return out


def mq_read_to_host(src, out=None, pageable=False, stream=None):
    """Blocking copy of the device tensor src into host memory through the
    library's pinned buffer (or pageable memory with pageable=True); returns
    out, a numpy array shaped like src when the caller gives none."""
    nbytes = src.numel() * src.element_size()
    dtype = torch.empty(0, dtype=src.dtype).numpy().dtype
    out = _host_out(out, dtype, tuple(src.shape), nbytes)
    flags = MQ_READ_PAGEABLE if pageable else MQ_READ_PINNED
    _check(lib().mq_read_to_host(_ptr(src, what="src"), out.ctypes.data, nbytes, flags, _stream(stream)))
    return out


def mq_readback_stats():
    b, p, q, w = _i64(), _i64(), _i64(), _int()
    _check(lib().mq_readback_stats(C.byref(b), C.byref(p), C.byref(q), C.byref(w)))
    return {"pinned_bytes": b.value, "pinned_reads": p.value, "pageable_reads": q.value, "warned": bool(w.value)}


def mq_readback_release():
    _check(lib().mq_readback_release())


def mq_workspace_stats():
    b, n, r = _i64(), _int(), _int()
    _check(lib().mq_workspace_stats(C.byref(b), C.byref(n), C.byref(r)))
    return {"bytes": b.value, "streams": n.value, "retired": r.value}


def mq_workspace_release():
    _check(lib().mq_workspace_release())


def mq_quantize_q8_0(x, xq=None, stream=None):
    """x: f32 [k] or [n, k] -> uint8 [n*(k/32)*34] q8_0 blocks (written into xq if given)."""
    k = x.shape[-1]
    n = x.numel() // k
    if xq is None:
        xq = torch.empty(q8_bytes(n, k), dtype=torch.uint8, device=x.device)
    _check(lib().mq_quantize_q8_0(_ptr(x, torch.float32, what="x"), _ptr(xq, torch.uint8, q8_bytes(n, k), "xq"),
                                  k, n, _stream(stream)))
    return xq


def mq_gemv_q4k_q8(w, xq, m, k, y=None, stream=None):
    if y is None:
        y = torch.empty(m, dtype=torch.float32, device=w.device)
    _check(lib().mq_gemv_q4k_q8(_ptr(w, torch.uint8, q4k_bytes(m, k), "w"), _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"),
                                _ptr(y, torch.float32, 4 * m, "y"), m, k, _stream(stream)))
    return y


def mq_gemv_q4k_q8_batched(w, xq, m, k, n, y=None, stream=None):
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check(lib().mq_gemv_q4k_q8_batched(_ptr(w, torch.uint8, q4k_bytes(m, k), "w"),
                                        _ptr(xq, torch.uint8, q8_bytes(n, k), "xq"),
                                        _ptr(y, torch.float32, 4 * m * n, "y"), m, k, n, _stream(stream)))
    return y


def mq_debug_gemv_q4k_batched_path(w, xq, m, k, n, path, y=None, stream=None):
    """The batched GEMV forced onto path 0 (vector kernels) or 1 (matrix cores)."""
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check(lib().mq_debug_gemv_q4k_batched_path(_ptr(w, torch.uint8, q4k_bytes(m, k), "w"),
                                                _ptr(xq, torch.uint8, q8_bytes(n, k), "xq"),
                                                _ptr(y, torch.float32, 4 * m * n, "y"), m, k, n, path,
                                                _stream(stream)))
    return y


def mq_gemv_batched_path(m, k, n, weight_format="q4_K"):
    """0 if the batched entry point takes the vector kernels for this shape,
    1 if it takes the matrix cores (host only)."""
    p = _int()
    _check(lib().mq_gemv_batched_path(m, k, n, MQ_FMT_Q4_0 if weight_format == "q4_0" else MQ_FMT_Q4_K,
                                      C.byref(p)))
    return p.value


def mq_gemv_q4k_q8_batched_noalloc(w, xq, m, k, n, y, stream=None):
    """The batched GEMV that allocates nothing: the caller passes y."""
    _check(lib().mq_gemv_q4k_q8_batched_noalloc(_ptr(w, torch.uint8, q4k_bytes(m, k), "w"),
                                                _ptr(xq, torch.uint8, q8_bytes(n, k), "xq"),
                                                _ptr(y, torch.float32, 4 * m * n, "y"), m, k, n, _stream(stream)))
    return y


def mq_gemv_q4_0_q8(w, xq, m, k, y=None, stream=None):
    if y is None:
        y = torch.empty(m, dtype=torch.float32, device=w.device)
    _check(lib().mq_gemv_q4_0_q8(_ptr(w, torch.uint8, q4_0_bytes(m, k), "w"),
                                 _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"),
                                 _ptr(y, torch.float32, 4 * m, "y"), m, k, _stream(stream)))
    return y


def mq_gemv_q4_0_q8_batched(w, xq, m, k, n, y=None, stream=None):
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _check(lib().mq_gemv_q4_0_q8_batched(_ptr(w, torch.uint8, q4_0_bytes(m, k), "w"),
                                         _ptr(xq, torch.uint8, q8_bytes(n, k), "xq"),
                                         _ptr(y, torch.float32, 4 * m * n, "y"), m, k, n, _stream(stream)))
    return y


def mq_gemv_q4k_grouped(w_all, expert_bytes, n_experts, ids, xq, xq_stride_bytes, m, k, y=None,
                        combine=None, y_out=None, want_y=True, stream=None):
    n_sel = ids.numel()
    if y is None and want_y:
        y = torch.empty((n_sel, m), dtype=torch.float32, device=w_all.device)
    if combine is not None and y_out is None:
        y_out = torch.empty(m, dtype=torch.float32, device=w_all.device)
    n_cols = n_sel if xq_stride_bytes else 1
    xq_need = (n_cols - 1) * xq_stride_bytes + q8_bytes(1, k)
    _check(lib().mq_gemv_q4k_grouped(
        _ptr(w_all, torch.uint8, n_experts * expert_bytes, "w_all"), expert_bytes, n_experts,
        _ptr(ids, torch.int32, 4 * n_sel, "ids"), n_sel, _ptr(xq, torch.uint8, xq_need, "xq"), xq_stride_bytes,
        _ptr(y, torch.float32, 4 * n_sel * m, "y"), _ptr(combine, torch.float32, 4 * n_sel, "combine"),
        _ptr(y_out, torch.float32, 4 * m, "y_out"), m, k, _stream(stream)))
    return y, y_out


def mq_gemv_q8_0_q8(w, xq, m, k, y=None, stream=None):
    if y is None:
        y = torch.empty(m, dtype=torch.float32, device=w.device)
    _check(lib().mq_gemv_q8_0_q8(_ptr(w, torch.uint8, q8_bytes(m, k), "w"), _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"),
                                 _ptr(y, torch.float32, 4 * m, "y"), m, k, _stream(stream)))
    return y


def mq_rmsnorm_quantize_q8_0(x, eps=1e-6, xq=None, stream=None):
    k = x.numel()
    if xq is None:
        xq = torch.empty(q8_bytes(1, k), dtype=torch.uint8, device=x.device)
    _check(lib().mq_rmsnorm_quantize_q8_0(_ptr(x, torch.float32, what="x"), _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"),
                                          k, eps, _stream(stream)))
    return xq


def mq_swiglu_quantize_q8_0(gu, inter, n_cols=1, k_pad=None, xq=None, stream=None):
    k_pad = inter if k_pad is None else k_pad
    if xq is None:
        xq = torch.empty(q8_bytes(n_cols, k_pad), dtype=torch.uint8, device=gu.device)
    _check(lib().mq_swiglu_quantize_q8_0(_ptr(gu, torch.float32, 4 * n_cols * 2 * inter, "gu"),
                                         _ptr(xq, torch.uint8, q8_bytes(n_cols, k_pad), "xq"),
                                         inter, n_cols, k_pad, _stream(stream)))
    return xq


def mq_debug_gemv_q4k_q8_isums(w, xq, m, k, stream=None):
    dev = w.device
    y = torch.empty(m, dtype=torch.float32, device=dev)
    isum = torch.empty((m, k // 32), dtype=torch.int32, device=dev)
    ysum = torch.empty(k // 32, dtype=torch.int32, device=dev)
    _check(lib().mq_debug_gemv_q4k_q8_isums(_ptr(w, torch.uint8, q4k_bytes(m, k), "w"),
                                            _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"), _ptr(y), _ptr(isum),
                                            _ptr(ysum), m, k, _stream(stream)))
    return y, isum, ysum


def mq_debug_gemv_q4_0_q8_isums(w, xq, m, k, stream=None):
    dev = w.device
    y = torch.empty(m, dtype=torch.float32, device=dev)
    isum = torch.empty((m, k // 32), dtype=torch.int32, device=dev)
    ysum = torch.empty(k // 32, dtype=torch.int32, device=dev)
    _check(lib().mq_debug_gemv_q4_0_q8_isums(_ptr(w, torch.uint8, q4_0_bytes(m, k), "w"),
                                             _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"), _ptr(y), _ptr(isum),
                                             _ptr(ysum), m, k, _stream(stream)))
    return y, isum, ysum


def mq_debug_gemv_q8_0_q8_isums(w, xq, m, k, stream=None):
    dev = w.device
    y = torch.empty(m, dtype=torch.float32, device=dev)
    isum = torch.empty((m, k // 32), dtype=torch.int32, device=dev)
    _check(lib().mq_debug_gemv_q8_0_q8_isums(_ptr(w, torch.uint8, q8_bytes(m, k), "w"),
                                             _ptr(xq, torch.uint8, q8_bytes(1, k), "xq"), _ptr(y), _ptr(isum),
                                             m, k, _stream(stream)))
    return y, isum


def mq_debug_gate_up_swiglu(w, x, inter, k, n_split=0, part=None, cnt=None, weight_format="q4_K", eps=1e-6,
                            stream=None):
    """The fused gate/up kernel alone: returns (gu f32 [2*inter], g q8_0 bytes)."""
    dev = w.device
    fmt = MQ_FMT_Q4_0 if weight_format == "q4_0" else MQ_FMT_Q4_K
    wb = q4_0_bytes(2 * inter, k) if fmt == MQ_FMT_Q4_0 else q4k_bytes(2 * inter, k)
    gu = torch.empty(2 * inter, dtype=torch.float32, device=dev)
    g = torch.empty(q8_bytes(1, inter), dtype=torch.uint8, device=dev)
    _check(lib().mq_debug_gate_up_swiglu(_ptr(w, torch.uint8, wb, "w"), _ptr(x, torch.float32, 4 * k, "x"), eps,
                                         _ptr(gu), _ptr(g), inter, k, n_split,
                                         _ptr(part, torch.float64, 128 * 8 * n_split, "part"),
                                         _ptr(cnt, torch.int32, 4 * n_split, "cnt"), fmt, _stream(stream)))
    return gu, g


class DecodeChain:
    """One decode step recorded as a hipGraph (mq_chain_create / mq_decode_chain)."""

    def __init__(self, model, weights, x_table, logits=None, flags=0, stream=None):
        L = model.n_layers
        self.L = L
        self.vocab = model.vocab
        self._keep = (weights, x_table)
        arr = lambda key: (_vp * L)(*[_ptr(weights[key][i], torch.uint8, what=key) for i in range(L)])
        self._arrays = [arr("qkv"), arr("o"), arr("gu"), arr("down")]
        self.logits = logits if logits is not None else torch.empty(model.vocab, dtype=torch.float32,
                                                                     device=x_table.device)
        n_inputs = x_table.shape[0]
        fmt = getattr(model, "weight_format", "q4_K")
        if fmt not in ("q4_K", "q4_0"):
            raise ValueError(f"unknown weight format {fmt!r}")
        d = ChainDesc(L, model.hidden, model.qkv_rows, model.inter, model.vocab, *self._arrays,
                      _ptr(weights["lm"], torch.uint8, q8_bytes(model.vocab, model.hidden), "lm"),
                      _ptr(x_table, torch.float32, 4 * n_inputs * model.hidden, "x_table"), n_inputs,
                      _ptr(self.logits, torch.float32, 4 * model.vocab, "logits"), model.eps, flags,
                      MQ_FMT_Q4_0 if fmt == "q4_0" else MQ_FMT_Q4_K, getattr(model, "o_k", 0))
        h = _vp()
        _check(lib().mq_chain_create(C.byref(d), _stream(stream), C.byref(h)))
        self.handle = h
        self.n_stamped = 4 * L + 1 if flags & MQ_SPAN_STAMPS and not flags & MQ_UNFUSED_GLUE else 0

    def step(self, mode=MQ_GRAPH, stream=None):
        _check(lib().mq_decode_chain(self.handle, mode, _stream(stream)))
        return self.logits

    def info(self):
        cap, nodes, step = _int(), _int(), _i64()
        _check(lib().mq_chain_info(self.handle, C.byref(cap), C.byref(nodes), C.byref(step)))
        return {"captured": bool(cap.value), "n_nodes": nodes.value, "step": step.value}

    def reset(self, step=0, stream=None):
        _check(lib().mq_chain_reset(self.handle, step, _stream(stream)))

    def capture_stats(self):
        n, ms = _i64(), C.c_double()
        _check(lib().mq_chain_capture_stats(self.handle, C.byref(n), C.byref(ms)))
        return {"graph_steps": n.value, "capture_ms": ms.value}

    def read_logits(self, out=None, pageable=False, stream=None):
        """Blocking readback of the last step's logits into a numpy f32 [vocab]."""
        vocab = self.vocab
        out = _host_out(out, np.float32, (vocab,), 4 * vocab)
        flags = MQ_READ_PAGEABLE if pageable else MQ_READ_PINNED
        _check(lib().mq_chain_read_logits(self.handle, out.ctypes.data, vocab, flags, _stream(stream)))
        return out

    def host_logits(self):
        """numpy f32 [vocab] view of the chain's pinned host logits (MQ_HOST_LOGITS),
        or None.  It is overwritten by every step: synchronize before reading and
        copy what must outlive the next step.  The memory belongs to the chain:
        the view is invalid once the chain is closed (or collected), so keep the
        chain object alive while the view is used."""
        p = _vp()
        _check(lib().mq_chain_host_logits(self.handle, C.byref(p)))
        if not p.value:
            return None
        return np.ctypeslib.as_array(C.cast(p, C.POINTER(C.c_float)), shape=(self.vocab,))

    def trace(self, stream=None):
        qb, fc = _i64(), _i64()
        _check(lib().mq_chain_trace_sizes(self.handle, C.byref(qb), C.byref(fc)))
        dev = self.logits.device
        q8 = torch.empty(qb.value, dtype=torch.uint8, device=dev)
        f32 = torch.empty(fc.value, dtype=torch.float32, device=dev)
        _check(lib().mq_chain_read_trace(self.handle, _ptr(q8), _ptr(f32), _stream(stream)))
        return q8, f32

    def read_stamps(self, stream=None):
        """MQ_SPAN_STAMPS: numpy uint64 [4*L + 1, 2] of [first wave start, last
        wave end] (100 MHz ticks) of each GEMV kernel's most recent launch, in
        step order (per layer QKV, O, gate/up, down; then the lm_head).
        Blocking."""
        out = np.zeros((self.n_stamped, 2), dtype=np.uint64)
        _check(lib().mq_chain_read_stamps(self.handle, out.ctypes.data, self.n_stamped, _stream(stream)))
        return out

    def clear_stamps(self, stream=None):
        """MQ_SPAN_STAMPS: reset the stamps on the stream (asynchronous)."""
        _check(lib().mq_chain_clear_stamps(self.handle, _stream(stream)))

    def close(self):
        if getattr(self, "handle", None):
            lib().mq_chain_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class MoEChain:
    """Routed-expert FFN tokens, `tokens_per_launch` per step (mq_moe_create / mq_moe_step)."""

    def __init__(self, n_experts, n_sel, hidden, inter, w_gu_all, gu_bytes, w_dn_all, dn_bytes,
                 ids_table, logits_table, x_table, y_table=None, flags=0, stream=None, tokens_per_launch=1):
        n_tokens = ids_table.shape[0]
        self.y_table = y_table if y_table is not None else torch.zeros((n_tokens, hidden), dtype=torch.float32,
                                                                       device=x_table.device)
        self._keep = (w_gu_all, w_dn_all, ids_table, logits_table, x_table)
        d = MoEDesc(n_experts, n_sel, hidden, inter,
                    _ptr(w_gu_all, torch.uint8, n_experts * gu_bytes, "w_gu_all"), gu_bytes,
                    _ptr(w_dn_all, torch.uint8, n_experts * dn_bytes, "w_dn_all"), dn_bytes,
                    _ptr(ids_table, torch.int32, 4 * n_tokens * n_sel, "ids_table"),
                    _ptr(logits_table, torch.float32, 4 * n_tokens * n_sel, "logits_table"),
                    _ptr(x_table, torch.float32, 4 * n_tokens * hidden, "x_table"),
                    _ptr(self.y_table, torch.float32, 4 * n_tokens * hidden, "y_table"), n_tokens, flags,
                    tokens_per_launch)
        h = _vp()
        _check(lib().mq_moe_create(C.byref(d), _stream(stream), C.byref(h)))
        self.handle = h
        self.n_stamped = 4 * L + 1 if flags & MQ_SPAN_STAMPS and not flags & MQ_UNFUSED_GLUE else 0

    def step(self, mode=MQ_GRAPH, stream=None):
        _check(lib().mq_moe_step(self.handle, mode, _stream(stream)))

    def info(self):
        cap, nodes, step = _int(), _int(), _i64()
        _check(lib().mq_chain_info(self.handle, C.byref(cap), C.byref(nodes), C.byref(step)))
        return {"captured": bool(cap.value), "n_nodes": nodes.value, "step": step.value}

    def reset(self, step=0, stream=None):
        _check(lib().mq_chain_reset(self.handle, step, _stream(stream)))

    def read_stamps(self, stream=None):
        """MQ_SPAN_STAMPS: numpy uint64 [4*L + 1, 2] of [first wave start, last
        wave end] (100 MHz ticks) of each GEMV kernel's most recent launch, in
        step order (per layer QKV, O, gate/up, down; then the lm_head).
        Blocking."""
        out = np.zeros((self.n_stamped, 2), dtype=np.uint64)
        _check(lib().mq_chain_read_stamps(self.handle, out.ctypes.data, self.n_stamped, _stream(stream)))
        return out

    def clear_stamps(self, stream=None):
        """MQ_SPAN_STAMPS: reset the stamps on the stream (asynchronous)."""
        _check(lib().mq_chain_clear_stamps(self.handle, _stream(stream)))

    def close(self):
        if getattr(self, "handle", None):
            lib().mq_chain_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
