"""numpy front end of the reference oracle (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use
this package.  The HIP library never imports, links or calls it.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_LIB = None

_u8p = C.POINTER(C.c_uint8)
_u16p = C.POINTER(C.c_uint16)
_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_f32p = C.POINTER(C.c_float)
_f64p = C.POINTER(C.c_double)
_i64 = C.c_int64


class ChainDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("hidden", C.c_int64), ("qkv_rows", C.c_int64),
                ("inter", C.c_int64), ("vocab", C.c_int64),
                ("w_qkv", C.POINTER(_u8p)), ("w_o", C.POINTER(_u8p)),
                ("w_gu", C.POINTER(_u8p)), ("w_down", C.POINTER(_u8p)),
                ("w_lm", _u8p), ("eps", C.c_float), ("weight_format", C.c_int), ("o_k", C.c_int64)]


OREF_Q4K, OREF_Q4_0 = 0, 1


def weight_format_code(model) -> int:
    """The oracle's code for a model's layer-weight format ("q4_K" or "q4_0")."""
    fmt = getattr(model, "weight_format", "q4_K")
    if fmt not in ("q4_K", "q4_0"):
        raise ValueError(f"unknown weight format {fmt!r}")
    return OREF_Q4_0 if fmt == "q4_0" else OREF_Q4K


_SIGS = {
    "oref_f16_to_f32_n": [_u16p, _f32p, _i64],
    "oref_f32_to_f16_n": [_f32p, _u16p, _i64],
    "oref_quantize_q8_0": [_f32p, _i64, _u8p],
    "oref_dequant_q8_0": [_u8p, _i64, _f64p],
    "oref_q4k_scale_min": [_u8p, C.c_int, _i32p, _i32p],
    "oref_dequant_q4k": [_u8p, _i64, _f64p],
    "oref_gemv_q4k": [_u8p, _i64, _i64, _u8p, _f32p, _f64p],
    "oref_gemv_q4k_rows": [_u8p, _i64, _u8p, _i64p, _i64, _f32p, _f64p],
    "oref_gemv_q8_0": [_u8p, _i64, _i64, _u8p, _f32p, _f64p],
    "oref_gemv_q8_0_rows": [_u8p, _i64, _u8p, _i64p, _i64, _f32p, _f64p],
    "oref_isums_q4k": [_u8p, _i64, _i64, _u8p, _i32p, _i32p],
    "oref_isums_q8_0": [_u8p, _i64, _i64, _u8p, _i32p],
    "oref_dequant_q4_0": [_u8p, _i64, _f64p],
    "oref_gemv_q4_0": [_u8p, _i64, _i64, _u8p, _f32p, _f64p],
    "oref_gemv_q4_0_rows": [_u8p, _i64, _u8p, _i64p, _i64, _f32p, _f64p],
    "oref_isums_q4_0": [_u8p, _i64, _i64, _u8p, _i32p],
    "oref_rmsnorm": [_f32p, _i64, C.c_float, _f32p],
    "oref_swiglu": [_f32p, _i64, _f32p],
    "oref_softmax": [_f32p, _i64, _f32p],
    "oref_chain_q8_trace_bytes": [C.POINTER(ChainDesc)],
    "oref_chain_f32_trace_len": [C.POINTER(ChainDesc)],
    "oref_chain": [C.POINTER(ChainDesc), _f32p, _f32p, _u8p, _f32p, _f64p],
    "oref_moe_token": [_u8p, _i64, _u8p, _i64, _i32p, C.c_int, _f32p, _f32p, _i64, _i64,
                       _f32p, _f32p, _f32p],
}
_RESTYPES = {"oref_chain_q8_trace_bytes": C.c_int64, "oref_chain_f32_trace_len": C.c_int64}


def load(path: str | None = None):
    """Load a compiled oracle library (building the default one if absent)."""
    global _LIB
    if path is None:
        if _LIB is not None:
            return _LIB
        path = _build.LIBRARY
        if not os.path.exists(path):
            _build.build()
    lib = C.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, None)
    if path == _build.LIBRARY:
        _LIB = lib
    return lib


def _p(a: np.ndarray | None, t):
    if a is None:
        return C.cast(None, t)
    assert a.flags.c_contiguous
    return a.ctypes.data_as(t)


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


class Oracle:
    """numpy wrappers over one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    # f16
    def f16_to_f32(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
        out = np.empty(h.size, np.float32)
        self.lib.oref_f16_to_f32_n(_p(h, _u16p), _p(out, _f32p), h.size)
        return out

    def f32_to_f16(self, f: np.ndarray) -> np.ndarray:
        f = np.ascontiguousarray(f, dtype=np.float32).ravel()
        out = np.empty(f.size, np.uint16)
        self.lib.oref_f32_to_f16_n(_p(f, _f32p), _p(out, _u16p), f.size)
        return out

    # q8_0
    def quantize_q8_0(self, x: np.ndarray) -> np.ndarray:
        """x: f32 [..., k] -> uint8 [..., k/32*34], each row quantized alone."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        k = x.shape[-1]
        rows = x.reshape(-1, k)
        out = np.empty((rows.shape[0], k // 32 * 34), np.uint8)
        for i in range(rows.shape[0]):
            r = np.ascontiguousarray(rows[i])
            o = out[i]
            self.lib.oref_quantize_q8_0(_p(r, _f32p), k, _p(o, _u8p))
        return out.reshape(*x.shape[:-1], k // 32 * 34)

    def dequant_q8_0(self, blocks: np.ndarray) -> np.ndarray:
        b = _u8(blocks).ravel()
        n = b.size // 34
        out = np.empty(32 * n, np.float64)
        self.lib.oref_dequant_q8_0(_p(b, _u8p), n, _p(out, _f64p))
        return out

    # q4_K
    def scale_min(self, s12: np.ndarray, j: int):
        s = _u8(s12)
        sc, m = C.c_int32(), C.c_int32()
        self.lib.oref_q4k_scale_min(_p(s, _u8p), j, C.byref(sc), C.byref(m))
        return sc.value, m.value

    def dequant_q4k(self, sbs: np.ndarray) -> np.ndarray:
        b = _u8(sbs).ravel()
        n = b.size // 144
        out = np.empty(256 * n, np.float64)
        self.lib.oref_dequant_q4k(_p(b, _u8p), n, _p(out, _f64p))
        return out

    # q4_0
    def dequant_q4_0(self, blocks: np.ndarray) -> np.ndarray:
        b = _u8(blocks).ravel()
        n = b.size // 18
        out = np.empty(32 * n, np.float64)
        self.lib.oref_dequant_q4_0(_p(b, _u8p), n, _p(out, _f64p))
        return out

    # GEMV
    def gemv_q4_0(self, w: np.ndarray, m: int, k: int, xq: np.ndarray, rows=None):
        """Returns (y f32, s_abs f64) for all rows or the listed rows."""
        w, xq = _u8(w), _u8(xq)
        if rows is None:
            y, sa = np.empty(m, np.float32), np.empty(m, np.float64)
            self.lib.oref_gemv_q4_0(_p(w, _u8p), m, k, _p(xq, _u8p), _p(y, _f32p), _p(sa, _f64p))
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            y, sa = np.empty(rows.size, np.float32), np.empty(rows.size, np.float64)
            self.lib.oref_gemv_q4_0_rows(_p(w, _u8p), k, _p(xq, _u8p), _p(rows, _i64p), rows.size,
                                         _p(y, _f32p), _p(sa, _f64p))
        return y, sa

    def isums_q4_0(self, w, m, k, xq):
        w, xq = _u8(w), _u8(xq)
        isum = np.empty((m, k // 32), np.int32)
        self.lib.oref_isums_q4_0(_p(w, _u8p), m, k, _p(xq, _u8p), _p(isum, _i32p))
        return isum

    def gemv_q4k(self, w: np.ndarray, m: int, k: int, xq: np.ndarray, rows=None):
        """Returns (y f32, s_abs f64) for all rows or the listed rows."""
        w, xq = _u8(w), _u8(xq)
        if rows is None:
            y, sa = np.empty(m, np.float32), np.empty(m, np.float64)
            self.lib.oref_gemv_q4k(_p(w, _u8p), m, k, _p(xq, _u8p), _p(y, _f32p), _p(sa, _f64p))
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            y, sa = np.empty(rows.size, np.float32), np.empty(rows.size, np.float64)
            self.lib.oref_gemv_q4k_rows(_p(w, _u8p), k, _p(xq, _u8p), _p(rows, _i64p), rows.size,
                                        _p(y, _f32p), _p(sa, _f64p))
        return y, sa

    def gemv_q8_0(self, w: np.ndarray, m: int, k: int, xq: np.ndarray, rows=None):
        w, xq = _u8(w), _u8(xq)
        if rows is None:
            y, sa = np.empty(m, np.float32), np.empty(m, np.float64)
            self.lib.oref_gemv_q8_0(_p(w, _u8p), m, k, _p(xq, _u8p), _p(y, _f32p), _p(sa, _f64p))
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            y, sa = np.empty(rows.size, np.float32), np.empty(rows.size, np.float64)
            self.lib.oref_gemv_q8_0_rows(_p(w, _u8p), k, _p(xq, _u8p), _p(rows, _i64p), rows.size,
                                         _p(y, _f32p), _p(sa, _f64p))
        return y, sa

    def isums_q4k(self, w, m, k, xq):
        w, xq = _u8(w), _u8(xq)
        isum = np.empty((m, k // 32), np.int32)
        ysum = np.empty(k // 32, np.int32)
        self.lib.oref_isums_q4k(_p(w, _u8p), m, k, _p(xq, _u8p), _p(isum, _i32p), _p(ysum, _i32p))
        return isum, ysum

    def isums_q8_0(self, w, m, k, xq):
        w, xq = _u8(w), _u8(xq)
        isum = np.empty((m, k // 32), np.int32)
        self.lib.oref_isums_q8_0(_p(w, _u8p), m, k, _p(xq, _u8p), _p(isum, _i32p))
        return isum

    # glue
    def rmsnorm(self, x, eps=1e-6):
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty_like(x)
        self.lib.oref_rmsnorm(_p(x, _f32p), x.size, eps, _p(y, _f32p))
        return y

    def swiglu(self, gu):
        gu = np.ascontiguousarray(gu, dtype=np.float32)
        inter = gu.size // 2
        y = np.empty(inter, np.float32)
        self.lib.oref_swiglu(_p(gu, _f32p), inter, _p(y, _f32p))
        return y

    def softmax(self, logits):
        lg = np.ascontiguousarray(logits, dtype=np.float32)
        p = np.empty_like(lg)
        self.lib.oref_softmax(_p(lg, _f32p), lg.size, _p(p, _f32p))
        return p

    # decode step
    def chain(self, model, weights, h0, n_layers=None, traces=False):
        """weights: dict with lists 'qkv','o','gu','down' of uint8 arrays and 'lm'.
        Returns dict(logits, s_abs[, q8_trace, f32_trace])."""
        L = model.n_layers if n_layers is None else n_layers
        keep = []

        def ptrs(lst):
            arr = (_u8p * L)()
            for i in range(L):
                a = _u8(lst[i])
                keep.append(a)
                arr[i] = _p(a, _u8p)
            return arr

        lm = _u8(weights["lm"])
        d = ChainDesc(L, model.hidden, model.qkv_rows, model.inter, model.vocab,
                      ptrs(weights["qkv"]), ptrs(weights["o"]), ptrs(weights["gu"]),
                      ptrs(weights["down"]), _p(lm, _u8p), model.eps, weight_format_code(model),
                      getattr(model, "o_k", 0))
        h0 = np.ascontiguousarray(h0, dtype=np.float32)
        logits = np.empty(model.vocab, np.float32)
        s_abs = np.empty(model.vocab, np.float64)
        q8t = f32t = None
        if traces:
            q8t = np.empty(self.lib.oref_chain_q8_trace_bytes(C.byref(d)), np.uint8)
            f32t = np.empty(self.lib.oref_chain_f32_trace_len(C.byref(d)), np.float32)
        self.lib.oref_chain(C.byref(d), _p(h0, _f32p), _p(logits, _f32p), _p(q8t, _u8p),
                            _p(f32t, _f32p), _p(s_abs, _f64p))
        out = {"logits": logits, "s_abs": s_abs}
        if traces:
            out["q8_trace"], out["f32_trace"] = q8t, f32t
        return out

    # routed experts
    def moe_token(self, w_gu_all, gu_bytes, w_dn_all, dn_bytes, ids, logits, x, hidden, inter):
        w_gu_all, w_dn_all = _u8(w_gu_all), _u8(w_dn_all)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        x = np.ascontiguousarray(x, dtype=np.float32)
        n_sel = ids.size
        y = np.empty(hidden, np.float32)
        ys = np.empty((n_sel, hidden), np.float32)
        c = np.empty(n_sel, np.float32)
        self.lib.oref_moe_token(_p(w_gu_all, _u8p), gu_bytes, _p(w_dn_all, _u8p), dn_bytes,
                                _p(ids, _i32p), n_sel, _p(logits, _f32p), _p(x, _f32p),
                                hidden, inter, _p(y, _f32p), _p(ys, _f32p), _p(c, _f32p))
        return y, ys, c
