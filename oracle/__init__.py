"""Python loader for the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The oracle shares no
code with the GPU library and never imports it.

All floating-point arrays handed to the oracle are float64 copies of the
exact bf16 / float32 inputs (see ``synth.bf16_bits_to_f64``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("D", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("score", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


class Layer:
    """One layer's inputs in float64 plus its dimensions.

    x, dy: [T, D]; w_gate, w_up: [E, I, D]; w_down: [E, D, I].
    """

    def __init__(self, x, w_gate, w_up, w_down, K: int, score: int, dy=None):
        self.x = _f64(x)
        self.w_gate = _f64(w_gate)
        self.w_up = _f64(w_up)
        self.w_down = _f64(w_down)
        self.dy = None if dy is None else _f64(dy)
        T, D = self.x.shape
        E, I, D2 = self.w_gate.shape
        assert D2 == D and self.w_up.shape == (E, I, D) and self.w_down.shape == (E, D, I)
        self.T, self.D, self.I, self.E, self.K, self.score = T, D, I, E, K, score

    def dims(self, T=None) -> _Dims:
        return _Dims(self.T if T is None else T, self.D, self.I, self.E, self.K, self.score)


def route(logits: np.ndarray, K: int, score: int):
    """Top-K selection and router weights -> (idx int32 [T,K], w float64 [T,K])."""
    lib = _load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    d = _Dims(T, 1, 1, E, K, score)
    idx = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float64)
    _check(lib.moe_oracle_route(ctypes.byref(d), _p(logits), _p(idx), _p(w)), "route")
    return idx, w


def sort(idx: np.ndarray, E: int):
    """Stable sort by expert -> (counts [E], offsets [E+1], sorted_to_flat, flat_to_sorted)."""
    lib = _load()
    idx = _i32(idx)
    T, K = idx.shape
    d = _Dims(T, 1, 1, E, K, 0)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    s2f = np.empty(T * K, dtype=np.int32)
    f2s = np.empty(T * K, dtype=np.int32)
    _check(lib.moe_oracle_sort(ctypes.byref(d), _p(idx), _p(counts), _p(offsets), _p(s2f),
                               _p(f2s)), "sort")
    return counts, offsets, s2f, f2s


def _tokens(tokens):
    if tokens is None:
        return None, 0
    t = np.ascontiguousarray(tokens, dtype=np.int64)
    return t, t.size


def forward(L: Layer, idx, w, tokens=None, want_o: bool = False):
    """y [ntok, D] (and o [ntok, K, D] if want_o) for the given tokens (None = all)."""
    lib = _load()
    idx, w = _i32(idx), _f64(w)
    tok, n = _tokens(tokens)
    n = L.T if tok is None else n
    y = np.empty((n, L.D), dtype=np.float64)
    o = np.empty((n, L.K, L.D), dtype=np.float64) if want_o else None
    d = L.dims()
    _check(lib.moe_oracle_forward(ctypes.byref(d), _p(L.x), _p(L.w_gate), _p(L.w_up),
                                  _p(L.w_down), _p(idx), _p(w), ctypes.c_int64(n), _p(tok),
                                  _p(y), _p(o)), "forward")
    return (y, o) if want_o else y


def backward_tokens(L: Layer, idx, w, tokens=None):
    """dX [ntok, D] and dRouterWeights [ntok, K] for the given tokens (None = all)."""
    lib = _load()
    idx, w = _i32(idx), _f64(w)
    tok, n = _tokens(tokens)
    n = L.T if tok is None else n
    dx = np.empty((n, L.D), dtype=np.float64)
    drw = np.empty((n, L.K), dtype=np.float64)
    d = L.dims()
    _check(lib.moe_oracle_backward_tokens(ctypes.byref(d), _p(L.x), _p(L.w_gate), _p(L.w_up),
                                          _p(L.w_down), _p(idx), _p(w), _p(L.dy),
                                          ctypes.c_int64(n), _p(tok), _p(dx), _p(drw)),
           "backward_tokens")
    return dx, drw


def backward_dw(L: Layer, idx, w, tokens=None):
    """(dW_gate [E,I,D], dW_up [E,I,D], dW_down [E,D,I]) over the given tokens (None = all)."""
    lib = _load()
    idx, w = _i32(idx), _f64(w)
    tok, n = _tokens(tokens)
    n = L.T if tok is None else n
    dwg = np.empty((L.E, L.I, L.D), dtype=np.float64)
    dwu = np.empty((L.E, L.I, L.D), dtype=np.float64)
    dwd = np.empty((L.E, L.D, L.I), dtype=np.float64)
    d = L.dims()
    _check(lib.moe_oracle_backward_dw(ctypes.byref(d), _p(L.x), _p(L.w_gate), _p(L.w_up),
                                      _p(L.w_down), _p(idx), _p(w), _p(L.dy),
                                      ctypes.c_int64(n), _p(tok), _p(dwg), _p(dwu), _p(dwd)),
           "backward_dw")
    return dwg, dwu, dwd


def expert_dw(L: Layer, idx, w, e: int):
    """(dW_gate[e] [I, D], dW_up[e] [I, D], dW_down[e] [D, I]) of one expert,
    summed over all of its routed rows, as the page's backward accumulates an
    expert's weight gradients over all of its token tiles (LigerCute README,
    "LigerMoE design", Backward pass).  Each step is its plain formula, with
    float64 matrix products (a library primitive) for the sums:
      rows r = (t, k) with idx[t, k] = e, in ascending flat slot t*K + k;
      g = x_t W_gate[e]^T,  u = x_t W_up[e]^T,  dA = dY_t W_down[e]   (per row);
      h = silu(g) u;  dG = w dA u sigma(g) (1 + g (1 - sigma(g)));
      dU = w dA silu(g);  Hw = w h   (w = the row's router weight);
      dW_gate = dG^T X,  dW_up = dU^T X,  dW_down = dY^T Hw.
    Needs the layer's dy."""
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    t, k = np.nonzero(idx == e)  # row-major order: ascending flat slot
    X, dY = L.x[t], L.dy[t]
    wr = w[t, k][:, None]
    g = X @ L.w_gate[e].T
    u = X @ L.w_up[e].T
    dA = dY @ L.w_down[e]
    sg = 1.0 / (1.0 + np.exp(-g))
    silu = g * sg
    dG = wr * dA * u * sg * (1.0 + g * (1.0 - sg))
    dU = wr * dA * silu
    Hw = wr * silu * u
    return dG.T @ X, dU.T @ X, dY.T @ Hw


def dw_entries(L: Layer, idx, w, which, e, r, c):
    """Single weight-gradient entries: which 0 = dW_gate[e,r,c], 1 = dW_up, 2 = dW_down."""
    lib = _load()
    idx, w = _i32(idx), _f64(w)
    which, e, r, c = (_i32(np.atleast_1d(v)) for v in (which, e, r, c))
    n = which.size
    out = np.empty(n, dtype=np.float64)
    d = L.dims()
    _check(lib.moe_oracle_dw_entries(ctypes.byref(d), _p(L.x), _p(L.w_gate), _p(L.w_up),
                                     _p(L.w_down), _p(idx), _p(w), _p(L.dy),
                                     ctypes.c_int64(n), _p(which), _p(e), _p(r), _p(c),
                                     _p(out)), "dw_entries")
    return out


def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """Router projection logits = x w_r  (x [T, D], w_r [D, E]) in float64."""
    lib = _load()
    x, w_r = _f64(x), _f64(w_r)
    T, D = x.shape
    D2, E = w_r.shape
    assert D2 == D
    out = np.empty((T, E), dtype=np.float64)
    d = _Dims(T, D, 1, E, 1, 0)
    _check(lib.moe_oracle_router_logits(ctypes.byref(d), _p(x), _p(w_r), _p(out)), "router_logits")
    return out


def router_backward(x: np.ndarray, w_r: np.ndarray, idx, w, drw, score: int):
    """Router backward with the selection fixed -> (dl [T,E], dW_r [D,E], dX_router [T,D])."""
    lib = _load()
    x, w_r, idx, w, drw = _f64(x), _f64(w_r), _i32(idx), _f64(w), _f64(drw)
    T, D = x.shape
    E = w_r.shape[1]
    K = idx.shape[1]
    dl = np.empty((T, E), dtype=np.float64)
    dw_r = np.empty((D, E), dtype=np.float64)
    dx_r = np.empty((T, D), dtype=np.float64)
    d = _Dims(T, D, 1, E, K, score)
    _check(lib.moe_oracle_router_backward(ctypes.byref(d), _p(x), _p(w_r), _p(idx), _p(w),
                                          _p(drw), _p(dl), _p(dw_r), _p(dx_r)), "router_backward")
    return dl, dw_r, dx_r


def threads() -> int:
    """Number of OpenMP threads the oracle's parallel loops use."""
    lib = _load()
    lib.moe_oracle_threads.restype = ctypes.c_int32
    return int(lib.moe_oracle_threads())
