"""ctypes binding of the plain-C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU
baseline use it; the GPU library never does.  Every function takes and returns numpy
arrays; inputs come from the seeded generator in ``synth``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

IQ2XS, IQ1M, IQ1S = 1, 2, 4


class QMat(C.Structure):
    _fields_ = [("qtype", C.c_int32), ("rows", C.c_int32), ("cols", C.c_int32), ("pad_", C.c_int32),
                ("s0", C.c_void_p), ("s1", C.c_void_p), ("s2", C.c_void_p)]


class Expert(C.Structure):
    _fields_ = [("gate", QMat), ("up", QMat), ("down", QMat)]


class Grids(C.Structure):
    _fields_ = [("iq2", C.c_uint8 * (512 * 8)), ("iq1", C.c_int8 * (2048 * 8))]

    def iq2_array(self) -> np.ndarray:
        return np.ctypeslib.as_array(self.iq2).reshape(512, 8).copy()

    def iq1_array(self) -> np.ndarray:
        return np.ctypeslib.as_array(self.iq1).reshape(2048, 8).copy()


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = C.CDLL(path)
        P = C.c_void_p
        i32 = C.c_int
        sig = {
            "orc_f16_to_f32": (C.c_float, [C.c_uint16]),
            "orc_set_threads": (None, [i32]),
            "orc_grids_expand": (i32, [P, P, P]),
            "orc_weight": (C.c_float, [P, P, i32, i32]),
            "orc_weight_f64": (C.c_double, [P, P, i32, i32]),
            "orc_dequant": (i32, [P, P, P]),
            "orc_matvec": (i32, [P, P, P, P]),
            "orc_matvec_f64": (i32, [P, P, P, P]),
            "orc_silu": (C.c_float, [C.c_float]),
            "orc_silu_f64": (C.c_double, [C.c_double]),
            "orc_expert_ffn": (i32, [P, P, P, P, P]),
            "orc_expert_ffn_f64": (i32, [P, P, P, P, P]),
            "orc_route": (i32, [P, i32, i32, i32, i32, P, P]),
            "orc_route_f64": (i32, [P, i32, i32, i32, i32, P, P]),
            "orc_group": (i32, [P, i32, i32, i32, P, P, P, P]),
            "orc_accumulate": (i32, [P, P, P, i32, i32, i32, P]),
            "orc_accumulate_f64": (i32, [P, P, P, i32, i32, i32, P]),
            "orc_moe_layer": (i32, [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, P, i32]),
            "orc_moe_layer_f64": (i32, [P, P, P, P, P, P, i32, i32, i32, i32, i32, P, P]),
            "orc_rmsnorm": (i32, [P, i32, i32, C.c_float, P]),
            "orc_rmsnorm_f64": (i32, [P, i32, i32, C.c_double, P]),
            "orc_router": (i32, [P, P, P, i32, i32, i32, P, P]),
            "orc_router_f64": (i32, [P, P, P, i32, i32, i32, P, P]),
            "orc_dot_abs": (i32, [P, P, i32, i32, i32, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _chk(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with {rc}")


def set_threads(n: int) -> None:
    lib().orc_set_threads(n)


def f16_to_f32(h: int) -> float:
    return lib().orc_f16_to_f32(h)


def grids(compact_iq2: np.ndarray, compact_iq1: np.ndarray) -> Grids:
    g = Grids()
    c2 = np.ascontiguousarray(compact_iq2, dtype=np.uint16)
    c1 = np.ascontiguousarray(compact_iq1, dtype=np.uint16)
    _chk(lib().orc_grids_expand(_p(c2), _p(c1), C.byref(g)), "grids_expand")
    return g


def qmat(qtype: int, rows: int, cols: int, streams) -> QMat:
    s = [np.ascontiguousarray(a) for a in streams]
    m = QMat(qtype, rows, cols, 0, s[0].ctypes.data, s[1].ctypes.data, s[2].ctypes.data)
    m._keep = s  # keep the arrays alive while the struct is
    return m


def dequant(m: QMat, g: Grids) -> np.ndarray:
    out = np.empty((m.rows, m.cols), dtype=np.float32)
    _chk(lib().orc_dequant(C.byref(m), C.byref(g), _p(out)), "dequant")
    return out


def weight_f64(m: QMat, g: Grids, r: int, c: int) -> float:
    return lib().orc_weight_f64(C.byref(m), C.byref(g), r, c)


def matvec(m: QMat, g: Grids, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(m.rows, dtype=np.float32)
    _chk(lib().orc_matvec(C.byref(m), C.byref(g), _p(x), _p(y)), "matvec")
    return y


def matvec_f64(m: QMat, g: Grids, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(m.rows, dtype=np.float64)
    _chk(lib().orc_matvec_f64(C.byref(m), C.byref(g), _p(x), _p(y)), "matvec_f64")
    return y


def silu(v: float) -> float:
    return lib().orc_silu(v)


def silu_f64(v: float) -> float:
    return lib().orc_silu_f64(v)


# ------------------------------------------------------------------ experts / layers

class ExpertTable:
    """orc_expert[n] for experts 0..n-1 of a ``synth.Layer`` (keeps the arrays alive)."""

    def __init__(self, layer):
        n = layer.n_experts + layer.has_shared
        self.arr = (Expert * n)()
        self.layer = layer
        H, I = layer.hidden, layer.inter
        for e in range(n):
            b, i = layer.bank_of(e)
            self.arr[e] = Expert(self._mat(b.qtype, I, H, b.gate, i), self._mat(b.qtype, I, H, b.up, i),
                                 self._mat(b.qtype, H, I, b.down, i))

    @staticmethod
    def _mat(qt, rows, cols, streams, i):
        return QMat(qt, rows, cols, 0, *[s[i].ctypes.data for s in streams])

    def expert(self, e: int) -> Expert:
        return self.arr[e]

    def qmat(self, e: int, which: str) -> QMat:
        return getattr(self.arr[e], which)


def expert_ffn(table: ExpertTable, e: int, g: Grids, x: np.ndarray, want_h: bool = False):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(table.layer.hidden, dtype=np.float32)
    h = np.empty(table.layer.inter, dtype=np.float32) if want_h else None
    _chk(lib().orc_expert_ffn(C.byref(table.arr[e]), C.byref(g), _p(x), _p(y), _p(h)), "expert_ffn")
    return (y, h) if want_h else y


def expert_ffn_f64(table: ExpertTable, e: int, g: Grids, x: np.ndarray, want_h: bool = False):
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(table.layer.hidden, dtype=np.float64)
    h = np.empty(table.layer.inter, dtype=np.float64) if want_h else None
    _chk(lib().orc_expert_ffn_f64(C.byref(table.arr[e]), C.byref(g), _p(x), _p(y), _p(h)), "expert_ffn_f64")
    return (y, h) if want_h else y


def route(logits: np.ndarray, k: int, add_shared: bool):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    kp = k + int(bool(add_shared))
    ids = np.empty((T, kp), dtype=np.int32)
    w = np.empty((T, kp), dtype=np.float32)
    _chk(lib().orc_route(_p(logits), T, E, k, int(bool(add_shared)), _p(ids), _p(w)), "route")
    return ids, w


def route_f64(logits: np.ndarray, k: int, add_shared: bool):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    kp = k + int(bool(add_shared))
    ids = np.empty((T, kp), dtype=np.int32)
    w = np.empty((T, kp), dtype=np.float64)
    _chk(lib().orc_route_f64(_p(logits), T, E, k, int(bool(add_shared)), _p(ids), _p(w)), "route_f64")
    return ids, w


def group(ids: np.ndarray, n_ids: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, kp = ids.shape
    counts = np.empty(n_ids, dtype=np.int32)
    offsets = np.empty(n_ids + 1, dtype=np.int32)
    ss = np.empty(T * kp, dtype=np.int32)
    sp = np.empty(T * kp, dtype=np.int32)
    _chk(lib().orc_group(_p(ids), T, kp, n_ids, _p(counts), _p(offsets), _p(ss), _p(sp)), "group")
    return counts, offsets, ss, sp


def accumulate(y: np.ndarray, w: np.ndarray, ids: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """y: [T*kp][H] in slot order; returns a new acc."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, kp = ids.shape
    H = acc.shape[1]
    out = np.array(acc, dtype=np.float32, copy=True)
    y = np.ascontiguousarray(y, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    _chk(lib().orc_accumulate(_p(y), _p(w), _p(ids), T, kp, H, _p(out)), "accumulate")
    return out


def accumulate_f64(y, w, ids, acc):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, kp = ids.shape
    H = acc.shape[1]
    out = np.array(acc, dtype=np.float64, copy=True)
    y = np.ascontiguousarray(y, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    _chk(lib().orc_accumulate_f64(_p(y), _p(w), _p(ids), T, kp, H, _p(out)), "accumulate_f64")
    return out


def moe_layer(table: ExpertTable, g: Grids, x: np.ndarray, k: int, add_shared: bool, logits=None,
              ids=None, w=None, acc=None, n_threads: int = 1):
    """Returns dict(acc, ids, w, y) with y [T*kp][H] in slot order."""
    layer = table.layer
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    E = layer.n_experts
    kp = k + int(bool(add_shared))
    out = np.zeros((T, H), dtype=np.float32) if acc is None else np.array(acc, dtype=np.float32, copy=True)
    ids_out = np.empty((T, kp), dtype=np.int32)
    w_out = np.empty((T, kp), dtype=np.float32)
    y_out = np.empty((T * kp, H), dtype=np.float32)
    lg = None if logits is None else np.ascontiguousarray(logits, dtype=np.float32)
    ii = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    ww = None if w is None else np.ascontiguousarray(w, dtype=np.float32)
    _chk(lib().orc_moe_layer(table.arr, C.byref(g), _p(x), _p(lg), _p(ii), _p(ww), T, E, k,
                             int(bool(add_shared)), H, _p(out), _p(ids_out), _p(w_out), _p(y_out), n_threads),
         "moe_layer")
    return {"acc": out, "ids": ids_out, "w": w_out, "y": y_out}


def moe_layer_f64(table: ExpertTable, g: Grids, x: np.ndarray, k: int, add_shared: bool, logits=None,
                  ids=None, w=None, acc=None):
    layer = table.layer
    x = np.ascontiguousarray(x, dtype=np.float64)
    T, H = x.shape
    E = layer.n_experts
    kp = k + int(bool(add_shared))
    out = np.zeros((T, H), dtype=np.float64) if acc is None else np.array(acc, dtype=np.float64, copy=True)
    y_out = np.empty((T * kp, H), dtype=np.float64)
    lg = None if logits is None else np.ascontiguousarray(logits, dtype=np.float32)
    ii = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    ww = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    _chk(lib().orc_moe_layer_f64(table.arr, C.byref(g), _p(x), _p(lg), _p(ii), _p(ww), T, E, k,
                                 int(bool(add_shared)), H, _p(out), _p(y_out)), "moe_layer_f64")
    return {"acc": out, "y": y_out}


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float32)
    T, H = h.shape
    x = np.empty_like(h)
    _chk(lib().orc_rmsnorm(_p(h), T, H, eps, _p(x)), "rmsnorm")
    return x


def rmsnorm_f64(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float64)
    T, H = h.shape
    x = np.empty_like(h)
    _chk(lib().orc_rmsnorm_f64(_p(h), T, H, eps, _p(x)), "rmsnorm_f64")
    return x


def threads_available() -> int:
    return len(os.sched_getaffinity(0))


def router(x: np.ndarray, wr: np.ndarray, wsg=None):
    """Router projection: (logits [T][E] fp32, shared weight [T] fp32 or None)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    T, H = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, H)
    lg = np.empty((T, E), np.float32)
    sw = None
    if wsg is not None:
        wsg = np.ascontiguousarray(wsg, dtype=np.float32).reshape(H)
        sw = np.empty(T, np.float32)
    _chk(lib().orc_router(_p(x), _p(wr), _p(wsg) if wsg is not None else None, T, H, E, _p(lg),
                          _p(sw) if sw is not None else None), "router")
    return lg, sw


def router_f64(x: np.ndarray, wr: np.ndarray, wsg=None):
    """The router projection summed in double: (logits [T][E], shared weight [T] or None)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    T, H = x.shape
    E = wr.shape[0]
    lg = np.empty((T, E), np.float64)
    sw = None
    if wsg is not None:
        wsg = np.ascontiguousarray(wsg, dtype=np.float32).reshape(H)
        sw = np.empty(T, np.float64)
    _chk(lib().orc_router_f64(_p(x), _p(wr), _p(wsg) if wsg is not None else None, T, H, E, _p(lg),
                              _p(sw) if sw is not None else None), "router_f64")
    return lg, sw


def dot_abs(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_c |x[t][c] * w[e][c]| [T][E]: the scale of the rounding error of each dot."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), np.float64)
    _chk(lib().orc_dot_abs(_p(x), _p(w), T, H, E, _p(out)), "dot_abs")
    return out
