"""CPU oracle for the 4-bit mixture-of-experts layer (ctypes wrapper of moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the product path never imports it,
and it imports nothing from the product package.  See ``moe_oracle.c`` for the
definitions and the passages of the Lily pages they follow.

Parity pins: every function here is pinned by ``tests/test_oracle.py``
(closed forms, brute force and library routines); nothing on the pages gives a
worked numeric example, so no value is pinned to a printed figure.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Q4(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p)]


class _Layer(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32),
                ("top_k", C.c_int32), ("x", C.c_void_p), ("wr_t", C.c_void_p),
                ("rbias", C.c_void_p), ("gate", _Q4), ("up", _Q4), ("down", _Q4),
                ("sh_gate", _Q4), ("sh_up", _Q4), ("sh_down", _Q4)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i32 = C.c_int32
        L.oracle_code.argtypes = [P, i32, i32, i32]
        L.oracle_code.restype = C.c_int
        L.oracle_dequant.argtypes = [P, P, P, i32, i32, P]
        L.oracle_router_logits.argtypes = [P, P, P, i32, i32, i32, P]
        L.oracle_topk.argtypes = [P, i32, i32, i32, P, P]
        L.oracle_routing.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_routing.restype = i32
        L.oracle_expert_act.argtypes = [C.POINTER(_Layer), i32, P, P]
        L.oracle_expert_down.argtypes = [C.POINTER(_Layer), i32, P, P]
        L.oracle_moe_tokens.argtypes = [C.POINTER(_Layer), P, i32, P, P, P]
        L.oracle_rmsnorm_residual.argtypes = [i32, i32, C.c_double, P, P, P, P]
        L.oracle_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def set_threads(n: int):
    """Threads of the oracle's OpenMP loops (for timing the CPU baseline)."""
    lib().oracle_set_threads(int(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def code(q: np.ndarray, K: int, n: int, k: int) -> int:
    q = _c(q, np.uint32)
    return lib().oracle_code(_p(q), K, n, k)


def dequant(q, s, b, N: int, K: int) -> np.ndarray:
    """Dequantised float64 weights [N][K] of one projection."""
    q, s, b = _c(q, np.uint32), _c(s, np.uint16), _c(b, np.uint16)
    assert q.size == N * K // 8 and s.size == b.size == N * K // 64
    w = np.empty((N, K), np.float64)
    lib().oracle_dequant(_p(q), _p(s), _p(b), N, K, _p(w))
    return w


def router_logits(x, wr_t, bias=None) -> np.ndarray:
    x, wr_t = _c(x, np.uint16), _c(wr_t, np.uint16)
    T, H = x.shape
    E = wr_t.shape[0]
    assert wr_t.shape[1] == H and H % 64 == 0
    bias = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(_p(x), _p(wr_t), _p(bias), T, H, E, _p(out))
    return out


def topk(logits, k: int = 8):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_topk(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def routing(ids, E: int, BM: int):
    """Histogram, offsets, stable scatter and block map (see moe_oracle.c)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_token = np.empty(T * k, np.int32)
    tok_row = np.empty((T, k), np.int32)
    max_blocks = -(-T * k // BM) + E
    blocks = np.zeros((max_blocks, 3), np.int32)
    nb = lib().oracle_routing(_p(ids), T, E, k, BM, _p(counts), _p(offsets), _p(row_token),
                              _p(tok_row), _p(blocks))
    return dict(counts=counts, offsets=offsets, row_token=row_token, tok_row=tok_row,
                blocks=blocks[:nb].copy(), num_blocks=nb)


class Layer:
    """Holds the numpy arrays of one layer and the matching C struct."""

    def __init__(self, inp):
        self.inp = inp
        keep = []

        def arr(a, dt):
            a = _c(a, dt)
            keep.append(a)
            return a

        def q4(p):
            return _Q4(arr(p.q, np.uint32).ctypes.data, arr(p.scale, np.uint16).ctypes.data,
                       arr(p.bias, np.uint16).ctypes.data)

        x = arr(inp.x, np.uint16)
        wr = arr(inp.router_wt, np.uint16)
        rb = None if inp.router_bias is None else arr(inp.router_bias, np.float32)
        self.s = _Layer(inp.T, inp.H, inp.I, inp.E, inp.top_k, x.ctypes.data, wr.ctypes.data,
                        None if rb is None else rb.ctypes.data, q4(inp.gate), q4(inp.up),
                        q4(inp.down), q4(inp.sh_gate), q4(inp.sh_up), q4(inp.sh_down))
        self._keep = keep
        self.x = x

    def with_x(self, x):
        """Same weights, another activation matrix (teacher forcing in a stack)."""
        x = _c(x, np.uint16)
        assert x.shape[1] == self.inp.H
        self._keep.append(x)
        self.s.x = x.ctypes.data
        self.s.T = x.shape[0]
        self.x = x
        return self

    def expert_act(self, e: int, t: int) -> np.ndarray:
        a = np.empty(self.inp.I, np.float64)
        xr = np.ascontiguousarray(self.x[t])
        lib().oracle_expert_act(C.byref(self.s), e, _p(xr), _p(a))
        return a

    def expert_down(self, e: int, a) -> np.ndarray:
        a = _c(a, np.float64)
        o = np.empty(self.inp.H, np.float64)
        lib().oracle_expert_down(C.byref(self.s), e, _p(a), _p(o))
        return o

    def tokens(self, tokens: Sequence[int]):
        """y [n][H] float64, ids [n][k], w [n][k] for the listed tokens."""
        tok = _c(list(tokens), np.int32)
        n = tok.size
        k = self.inp.top_k
        y = np.empty((n, self.inp.H), np.float64)
        ids = np.empty((n, k), np.int32)
        w = np.empty((n, k), np.float64)
        lib().oracle_moe_tokens(C.byref(self.s), _p(tok), n, _p(y), _p(ids), _p(w))
        return y, ids, w


def rmsnorm_residual(r, y, eps: float = 1e-6):
    r, y = _c(r, np.float64), _c(y, np.float64)
    T, H = r.shape
    r_out = np.empty_like(r)
    u = np.empty((T, H), np.uint16)
    lib().oracle_rmsnorm_residual(T, H, eps, _p(r), _p(y), _p(r_out), _p(u))
    return r_out, u
