"""Python handle on the fp64 CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU
library never loads it and shares no code with it; the two meet only in the
seeded inputs of ``qmoe_synth``.

Every function here marshals numpy arrays into the C oracle and back; all the
arithmetic lives in the C file.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc -O2 (IEEE semantics: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                               "-I", _HERE, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class OqTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32)]


class OqTail(ctypes.Structure):
    _fields_ = [("norm_shared", ctypes.c_void_p), ("norm_routed", ctypes.c_void_p), ("norm_out", ctypes.c_void_p),
                ("eps", ctypes.c_double), ("layer_scalar", ctypes.c_double)]


class OqRouter(ctypes.Structure):
    _fields_ = [("w", OqTensor), ("router_scale", ctypes.c_void_p), ("per_expert_scale", ctypes.c_void_p),
                ("logit_bias", ctypes.c_void_p), ("top_k", ctypes.c_int32), ("eps", ctypes.c_double)]


class OqPool(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("num_experts", ctypes.c_int32)]


class OqShared(ctypes.Structure):
    _fields_ = [("gate", OqTensor), ("up", OqTensor), ("down", OqTensor)]


def load(path: Optional[str] = None):
    """Load the oracle library (building it first if it is absent)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def using(path: str):
    """Temporarily route every call of this module to another build of the
    oracle (the pin tests use it to show that planted mistakes are caught)."""
    global _lib
    old = _lib
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = old


def _bind(lib):
    P, I32, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    sig = {
        "oq_bf16_to_double": (D, [ctypes.c_uint16]),
        "oq_bf16_round": (ctypes.c_uint16, [D]),
        "oq_code": (I32, [P, I32, I32]),
        "oq_weight": (D, [P, I32, I32]),
        "oq_dequant": (None, [P, P]),
        "oq_matvec": (None, [P, P, P]),
        "oq_gelu_tanh": (D, [D]),
        "oq_router_logits": (None, [P, P, I32, P]),
        "oq_topk": (None, [P, P, I32, P, P]),
        "oq_expert": (None, [P, P, P, P, P]),
        "oq_moe_forward": (I32, [P, I32, I32, P, P, P, P, P, P, P, P]),
        "oq_moe_forward_ex": (I32, [P, I32, I32, P, P, P, P, P, P, P, P, P, P]),
        "oq_layer_tail": (None, [P, P, P, I32, P, P]),
        "oq_qgemv_head": (None, [P, P, I32, D, P, P]),
        "oq_moe_dense_masked": (I32, [P, I32, I32, P, P, P, P]),
        "oq_rmsnorm_bf16": (None, [P, I32, I32, D, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class _Keep:
    """Keeps the numpy buffers behind ctypes structures alive."""

    def __init__(self):
        self.refs = []

    def arr(self, a, dtype):
        a = np.ascontiguousarray(a, dtype=dtype)
        self.refs.append(a)
        return a


def _tensor(qt, keep: _Keep) -> OqTensor:
    c = keep.arr(qt.codes, np.uint32)
    s = keep.arr(qt.scales, np.uint16)
    b = keep.arr(qt.biases, np.uint16)
    return OqTensor(c.ctypes.data, s.ctypes.data, b.ctypes.data, qt.rows, qt.cols, qt.bits, getattr(qt, "group", 64))


def _router(layer, keep: _Keep, top_k: Optional[int] = None, eps: Optional[float] = None) -> OqRouter:
    rs = None if layer.router_scale is None else keep.arr(layer.router_scale, np.float32)
    pes = None if layer.per_expert_scale is None else keep.arr(layer.per_expert_scale, np.float32)
    lb = None if layer.logit_bias is None else keep.arr(layer.logit_bias, np.float32)
    return OqRouter(_tensor(layer.router, keep), _ptr(rs), _ptr(pes), _ptr(lb),
                    layer.cfg.top_k if top_k is None else top_k,
                    layer.cfg.eps if eps is None else eps)


def _pool(layer, keep: _Keep, experts: Optional[Sequence[int]] = None):
    """Pool structure; with ``experts`` only those experts get real tensors
    (the others are never read unless selected, so they must not be)."""
    E = layer.cfg.num_experts
    gate_arr = (OqTensor * E)()
    up_arr = (OqTensor * E)()
    down_arr = (OqTensor * E)()
    sel = range(E) if experts is None else experts
    for e in range(E):
        # shape-only placeholder keeps the shape check meaningful
        for arr, qt in ((gate_arr, layer.gate), (up_arr, layer.up), (down_arr, layer.down)):
            arr[e] = OqTensor(None, None, None, qt.rows, qt.cols, qt.bits, getattr(qt, "group", 64))
    for e in sel:
        gate_arr[e] = _tensor(layer.gate.select(e), keep)
        up_arr[e] = _tensor(layer.up.select(e), keep)
        down_arr[e] = _tensor(layer.down.select(e), keep)
    keep.refs += [gate_arr, up_arr, down_arr]
    return OqPool(ctypes.addressof(gate_arr), ctypes.addressof(up_arr), ctypes.addressof(down_arr), E)


def _shared(layer, keep: _Keep):
    if layer.shared_gate is None:
        return None
    return OqShared(_tensor(layer.shared_gate, keep), _tensor(layer.shared_up, keep),
                    _tensor(layer.shared_down, keep))


# ---------------------------------------------------------------- primitives

def bf16_round(v: float) -> int:
    return int(load().oq_bf16_round(float(v)))


def bf16_to_double(b: int) -> float:
    return float(load().oq_bf16_to_double(int(b)))


def gelu_tanh(z: float) -> float:
    return float(load().oq_gelu_tanh(float(z)))


def code(qt, r: int, c: int) -> int:
    keep = _Keep()
    t = _tensor(qt, keep)
    return int(load().oq_code(ctypes.byref(t), r, c))


def codes(qt) -> np.ndarray:
    """All codes of a matrix as uint8 [rows][cols] (one oracle call per element: small matrices)."""
    keep = _Keep()
    t = _tensor(qt, keep)
    lib = load()
    out = np.empty((qt.rows, qt.cols), dtype=np.uint8)
    for r in range(qt.rows):
        for c in range(qt.cols):
            out[r, c] = lib.oq_code(ctypes.byref(t), r, c)
    return out


def dequant(qt) -> np.ndarray:
    keep = _Keep()
    t = _tensor(qt, keep)
    out = np.empty((qt.rows, qt.cols), dtype=np.float64)
    load().oq_dequant(ctypes.byref(t), out.ctypes.data)
    return out


def matvec(qt, x: np.ndarray) -> np.ndarray:
    keep = _Keep()
    t = _tensor(qt, keep)
    xv = keep.arr(x, np.float64)
    y = np.empty(qt.rows, dtype=np.float64)
    load().oq_matvec(ctypes.byref(t), xv.ctypes.data, y.ctypes.data)
    return y


def expert(gate, up, down, x: np.ndarray) -> np.ndarray:
    keep = _Keep()
    g, u, d = _tensor(gate, keep), _tensor(up, keep), _tensor(down, keep)
    xv = keep.arr(x, np.float64)
    y = np.empty(down.rows, dtype=np.float64)
    load().oq_expert(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), xv.ctypes.data, y.ctypes.data)
    return y


def router_logits(layer, x_bf16_row: np.ndarray, eps: Optional[float] = None) -> np.ndarray:
    keep = _Keep()
    rt = _router(layer, keep, eps=eps)
    xv = keep.arr(x_bf16_row, np.uint16)
    out = np.empty(layer.cfg.num_experts, dtype=np.float64)
    load().oq_router_logits(ctypes.byref(rt), xv.ctypes.data, layer.cfg.hidden, out.ctypes.data)
    return out


def topk(layer, logits: np.ndarray, top_k: Optional[int] = None):
    keep = _Keep()
    rt = _router(layer, keep, top_k=top_k)
    lg = keep.arr(logits, np.float64)
    k = rt.top_k
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    load().oq_topk(ctypes.byref(rt), lg.ctypes.data, lg.size, ids.ctypes.data, w.ctypes.data)
    return ids, w


def rmsnorm_bf16(x_bf16: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, H = x.shape
    out = np.empty_like(x)
    load().oq_rmsnorm_bf16(x.ctypes.data, T, H, eps, out.ctypes.data)
    return out


def _tail(tail, keep: _Keep):
    """OqTail from a dict with optional norm_shared / norm_routed / norm_out
    (float [H]), eps and layer_scalar; None stays None."""
    if tail is None:
        return None
    w = lambda k: None if tail.get(k) is None else keep.arr(tail[k], np.float32).ctypes.data
    return OqTail(w("norm_shared"), w("norm_routed"), w("norm_out"), float(tail.get("eps", 1e-6)),
                  float(tail.get("layer_scalar", 1.0)))


def layer_tail(s: np.ndarray, r: np.ndarray, tail: dict, resid: Optional[np.ndarray] = None) -> np.ndarray:
    """One row through the layer tail: s, r float64 [H], resid bf16 bits [H] or None."""
    keep = _Keep()
    sv, rv = keep.arr(s, np.float64), keep.arr(r, np.float64)
    rs = None if resid is None else keep.arr(resid, np.uint16)
    out = np.empty(sv.size, np.float64)
    tl = _tail(tail, keep)
    load().oq_layer_tail(sv.ctypes.data, rv.ctypes.data, _ptr(rs), sv.size, ctypes.byref(tl), out.ctypes.data)
    return out


def qgemv_head(qt, x_bf16: np.ndarray, softcap: float = 0.0, want_logits: bool = True):
    """Quantized head over token rows x (bf16 bits [T][cols]): (logits [T][rows] or None, argmax [T])."""
    keep = _Keep()
    t = _tensor(qt, keep)
    x = keep.arr(np.atleast_2d(x_bf16), np.uint16)
    T = x.shape[0]
    lg = np.empty((T, qt.rows), np.float64) if want_logits else None
    am = np.empty(T, np.int32)
    load().oq_qgemv_head(ctypes.byref(t), x.ctypes.data, T, float(softcap), _ptr(lg), am.ctypes.data)
    return lg, am


# ---------------------------------------------------------------- the layer

def forward(layer, x_bf16: np.ndarray, threads: int = 1, dense_experts: bool = True,
            tail: Optional[dict] = None, resid: Optional[np.ndarray] = None) -> dict:
    """Whole layer for tokens x (bf16 bits [T][H]).

    ``tail`` (a dict as for ``layer_tail``) passes the two branches through
    the layer tail, with ``resid`` (bf16 bits [T][H], or None for zero) as
    the residual rows.

    Returns ids int32 [T][k], w float64 [T][k], logits float64 [T][E],
    out64 float64 [T][H] and out_bf16 uint16 [T][H].  ``threads`` > 1 splits
    the tokens over that many threads (each runs the same sequential code).
    ``dense_experts=False`` hands the oracle only the experts its own router
    picks (saves marshalling for large pools; the result is identical).
    """
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, H = x.shape
    E, k = layer.cfg.num_experts, layer.cfg.top_k
    res = dict(ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float64),
               logits=np.empty((T, E), np.float64), out64=np.empty((T, H), np.float64),
               out_bf16=np.empty((T, H), np.uint16))
    lib = load()
    keep = _Keep()
    rt = _router(layer, keep)
    experts = None
    if not dense_experts:
        sel = set()
        for t in range(T):
            ids_t, _ = topk(layer, router_logits(layer, x[t]))
            sel.update(int(e) for e in ids_t)
        experts = sorted(sel)
    pool = _pool(layer, keep, experts)
    sh = _shared(layer, keep)
    tl = _tail(tail, keep)
    rs = None if resid is None else keep.arr(resid, np.uint16)

    def run(t0, t1):
        if t1 <= t0:
            return
        rc = lib.oq_moe_forward_ex(x[t0:].ctypes.data, t1 - t0, H, ctypes.byref(rt), ctypes.byref(pool),
                                   None if sh is None else ctypes.byref(sh), None if tl is None else ctypes.byref(tl),
                                   None if rs is None else rs[t0:].ctypes.data,
                                   res["ids"][t0:].ctypes.data, res["w"][t0:].ctypes.data,
                                   res["logits"][t0:].ctypes.data, res["out64"][t0:].ctypes.data,
                                   res["out_bf16"][t0:].ctypes.data)
        if rc != 0:
            raise ValueError("oracle rejected the layer shapes")

    threads = max(1, min(threads, T))
    if threads == 1:
        run(0, T)
    else:
        bounds = np.linspace(0, T, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: run(bounds[i], bounds[i + 1]), range(threads)))
    return res


def dense_masked(layer, x_bf16: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    T, H = x.shape
    keep = _Keep()
    rt = _router(layer, keep)
    pool = _pool(layer, keep)
    sh = _shared(layer, keep)
    out = np.empty((T, H), np.float64)
    rc = load().oq_moe_dense_masked(x.ctypes.data, T, H, ctypes.byref(rt), ctypes.byref(pool),
                                    None if sh is None else ctypes.byref(sh), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the layer shapes")
    return out
