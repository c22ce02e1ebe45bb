"""ctypes front end of the Engram CPU oracle (``engram_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``;
the library under test never imports it.  Every array passed in is read as
is (float32, bf16 bit patterns as uint16, or float64) and every result is
float64 (indices int32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DT_F32, DT_BF16, DT_F64 = 0, 1, 2


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o", _LIB_PATH,
           os.path.join(_HERE, "engram_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_orders", ctypes.c_int32),
        ("orders", ctypes.c_int32 * 4),
        ("heads", ctypes.c_int32),
        ("max_order", ctypes.c_int32),
        ("mult", ctypes.c_void_p),
        ("table_rows", ctypes.c_void_p),
        ("pad_id", ctypes.c_int32),
        ("canon_map", ctypes.c_void_p),
        ("vocab", ctypes.c_int32),
        ("tokens", ctypes.c_void_p),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("tables", ctypes.c_void_p),
        ("hidden", ctypes.c_int32),
        ("w_k", ctypes.c_void_p),
        ("w_v", ctypes.c_void_p),
        ("h", ctypes.c_void_p),
        ("gamma_q", ctypes.c_void_p),
        ("gamma_k", ctypes.c_void_p),
        ("eps", ctypes.c_double),
        ("taps", ctypes.c_int32),
        ("conv_w", ctypes.c_void_p),
        ("fp8_e", ctypes.c_int32),
    ]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(_Problem)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.oracle_hash.argtypes = [P, i64, vp, vp]
    lib.oracle_gather.argtypes = [P, i64, vp, vp]
    lib.oracle_gate_value.argtypes = [P, vp, vp]
    lib.oracle_gate_value.restype = ctypes.c_double
    lib.oracle_conv.argtypes = [P, i64, vp, vp, vp]
    lib.oracle_forward.argtypes = [P, i64, vp, vp, vp, vp, vp, vp]
    lib.oracle_backward_de.argtypes = [P, vp, i64, vp, vp]
    lib.oracle_backward_params.argtypes = [P, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_quantize_rows.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    lib.oracle_table_grad_rows.argtypes = [P, vp, vp, i64, vp, vp, vp]
    lib.oracle_table_grad_dense.argtypes = [P, vp, vp]
    lib.oracle_prefetch_plan.argtypes = [i64, i32, vp, vp, vp, vp]
    lib.oracle_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float64:
        return DT_F64
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data


class Problem:
    """Holds the arrays of one problem and the ctypes struct that points at them.

    Arguments mirror the method's inputs:
      orders, heads, mult [J, max_order] uint64, table_rows [J], pad_id,
      canon_map [V] int32, tokens [B, T] int32, tables: list of J [M_j, D],
      w_k, w_v [d, d_mem] (k_t = W_K e_t), h [B, T, d], conv_w [d, taps],
      gamma_q / gamma_k [d] or None, eps.
    Arrays are kept referenced for the lifetime of the object.
    """

    def __init__(self, *, orders, heads, mult, table_rows, pad_id, canon_map, tokens, tables,
                 w_k=None, w_v=None, h=None, conv_w=None, gamma_q=None, gamma_k=None, eps=1e-6,
                 fp8=False):
        J = len(orders) * heads
        assert len(orders) <= 4 and J <= 64 and len(tables) == J
        self.orders = tuple(int(o) for o in orders)
        self.heads = int(heads)
        self.J = J
        self.mult = np.ascontiguousarray(mult, dtype=np.uint64).reshape(J, -1)
        self.max_order = self.mult.shape[1]
        assert self.max_order >= max(self.orders)
        self.table_rows = np.ascontiguousarray(table_rows, dtype=np.int64)
        self.canon_map = np.ascontiguousarray(canon_map, dtype=np.int32)
        self.tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        assert self.tokens.ndim == 2
        self.B, self.T = self.tokens.shape
        self.tables = [np.ascontiguousarray(t) for t in tables]
        self.dim = self.tables[0].shape[1]
        for j, t in enumerate(self.tables):
            assert t.shape == (int(self.table_rows[j]), self.dim) and t.dtype == self.tables[0].dtype
        self._tab_ptrs = (ctypes.c_void_p * J)(*[t.ctypes.data for t in self.tables])
        self.d_mem = J * self.dim
        self.w_k = None if w_k is None else np.ascontiguousarray(w_k)
        self.w_v = None if w_v is None else np.ascontiguousarray(w_v)
        if fp8 and self.w_k is not None:
            # the FP8 projection reads each weight row in e4m3 with its own scale
            self.w_k = quantize_rows(self.w_k)[2]
            self.w_v = quantize_rows(self.w_v)[2]
        self.hidden = 0 if self.w_k is None else self.w_k.shape[0]
        if self.w_k is not None:
            assert self.w_k.shape == (self.hidden, self.d_mem) and self.w_v.shape == self.w_k.shape
            assert self.w_k.dtype == self.w_v.dtype
        self.h = None if h is None else np.ascontiguousarray(h)
        if self.h is not None:
            assert self.h.shape == (self.B, self.T, self.hidden)
        self.conv_w = None if conv_w is None else np.ascontiguousarray(conv_w, dtype=np.float64)
        self.taps = 0 if self.conv_w is None else self.conv_w.shape[1]
        assert self.taps <= 16
        self.gamma_q = None if gamma_q is None else np.ascontiguousarray(gamma_q, dtype=np.float64)
        self.gamma_k = None if gamma_k is None else np.ascontiguousarray(gamma_k, dtype=np.float64)
        self.eps = float(eps)
        self.pad_id = int(pad_id)
        s = _Problem()
        s.num_orders = len(self.orders)
        for i, o in enumerate(self.orders):
            s.orders[i] = o
        s.heads = self.heads
        s.max_order = self.max_order
        s.mult = _ptr(self.mult)
        s.table_rows = _ptr(self.table_rows)
        s.pad_id = self.pad_id
        s.canon_map = _ptr(self.canon_map)
        s.vocab = self.canon_map.size
        s.tokens = _ptr(self.tokens)
        s.B, s.T = self.B, self.T
        s.dim = self.dim
        s.dtype = _dt(self.tables[0])
        s.w_dtype = _dt(self.w_k) if self.w_k is not None else 0
        s.act_dtype = _dt(self.h) if self.h is not None else 0
        s.tables = ctypes.cast(self._tab_ptrs, ctypes.c_void_p)
        s.hidden = self.hidden
        s.w_k, s.w_v, s.h = _ptr(self.w_k), _ptr(self.w_v), _ptr(self.h)
        s.gamma_q, s.gamma_k = _ptr(self.gamma_q), _ptr(self.gamma_k)
        s.eps = self.eps
        s.taps = self.taps
        s.conv_w = _ptr(self.conv_w)
        s.fp8_e = 1 if fp8 else 0
        self._s = s

    @classmethod
    def from_inputs(cls, inp, *, widen_weights: bool = True, **over):
        """Problem over the arrays of a ``synth.Inputs``.

        widen_weights: hand the projection weights over as float64 (an exact
        widening of the bf16/f32 values) so the slow inner products skip the
        per-element decode.
        """
        wl = inp.wl
        w_k, w_v = inp.w_k, inp.w_v
        if widen_weights:
            w_k, w_v = _widen(w_k), _widen(w_v)
        kw = dict(orders=wl.orders, heads=wl.heads, mult=inp.multipliers, table_rows=inp.table_rows,
                  pad_id=wl.pad_id, canon_map=inp.canon_map, tokens=inp.tokens, tables=inp.tables,
                  w_k=w_k, w_v=w_v, h=inp.hidden, conv_w=inp.conv_w, eps=wl.rms_eps)
        kw.update(over)
        return cls(**kw)

    @property
    def ref(self):
        return ctypes.byref(self._s)

    # ------------------------------------------------------------ entries
    def all_positions(self) -> np.ndarray:
        return np.arange(self.B * self.T, dtype=np.int64)

    def hash(self, pos=None) -> np.ndarray:
        pos = self.all_positions() if pos is None else np.ascontiguousarray(pos, dtype=np.int64)
        out = np.empty((pos.size, self.J), np.int32)
        _load().oracle_hash(self.ref, pos.size, _ptr(pos), _ptr(out))
        return out

    def gather(self, idx: np.ndarray) -> np.ndarray:
        idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1, self.J)
        out = np.empty((idx.shape[0], self.d_mem), np.float64)
        _load().oracle_gather(self.ref, idx.shape[0], _ptr(idx), _ptr(out))
        return out

    def gate_value(self, h: np.ndarray, k: np.ndarray) -> float:
        h = np.ascontiguousarray(h, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        assert h.size == self.hidden and k.size == self.hidden
        return _load().oracle_gate_value(self.ref, _ptr(h), _ptr(k))

    def conv(self, vt: np.ndarray):
        vt = np.ascontiguousarray(vt, dtype=np.float64)
        T = vt.shape[0]
        assert vt.shape == (T, self.hidden)
        z = np.empty_like(vt)
        y = np.empty_like(vt)
        _load().oracle_conv(self.ref, T, _ptr(vt), _ptr(z), _ptr(y))
        return z, y

    def forward(self, pos=None, *, want=("y",)):
        """Dict of float64 arrays at flat positions `pos` (default: all)."""
        pos = self.all_positions() if pos is None else np.ascontiguousarray(pos, dtype=np.int64)
        n = pos.size
        d = self.hidden
        out = {}
        shapes = {"y": (n, d), "alpha": (n,), "k": (n, d), "v": (n, d), "e": (n, self.d_mem)}
        for key in want:
            out[key] = np.empty(shapes[key], np.float64)
        _load().oracle_forward(self.ref, n, _ptr(pos), _ptr(out.get("y")), _ptr(out.get("alpha")),
                               _ptr(out.get("k")), _ptr(out.get("v")), _ptr(out.get("e")))
        return out

    def backward_de(self, dy: np.ndarray, pos=None) -> np.ndarray:
        dy = np.ascontiguousarray(dy)
        assert dy.shape == (self.B, self.T, self.hidden) and _dt(dy) == _dt(self.h)
        pos = self.all_positions() if pos is None else np.ascontiguousarray(pos, dtype=np.int64)
        out = np.empty((pos.size, self.d_mem), np.float64)
        _load().oracle_backward_de(self.ref, _ptr(dy), pos.size, _ptr(pos), _ptr(out))
        return out

    def backward_params(self, dy: np.ndarray, pos=None,
                        want=("w_k", "w_v", "conv_w", "gamma_q", "gamma_k", "h")) -> dict:
        """Parameter and hidden-state gradients of L = sum <G, Y> (float64).

        w_k, w_v [d, d_mem], conv_w [d, taps], gamma_q, gamma_k [d]: summed
        over the positions `pos` (default: all, the full gradients); h
        [npos, d]: per position, the gate's part of dL/dh_t."""
        dy = np.ascontiguousarray(dy)
        assert dy.shape == (self.B, self.T, self.hidden) and _dt(dy) == _dt(self.h)
        pos = self.all_positions() if pos is None else np.ascontiguousarray(pos, dtype=np.int64)
        d, dm = self.hidden, self.d_mem
        shapes = {"w_k": (d, dm), "w_v": (d, dm), "conv_w": (d, self.taps), "gamma_q": (d,),
                  "gamma_k": (d,), "h": (pos.size, d)}
        out = {k: np.empty(shapes[k], np.float64) for k in want}
        _load().oracle_backward_params(self.ref, _ptr(dy), pos.size, _ptr(pos), _ptr(out.get("w_k")),
                                       _ptr(out.get("w_v")), _ptr(out.get("conv_w")),
                                       _ptr(out.get("gamma_q")), _ptr(out.get("gamma_k")),
                                       _ptr(out.get("h")))
        return out

    def table_grad_rows(self, dy: np.ndarray, idx_all: np.ndarray, rows_j, rows_r):
        """dE_j[r] for the requested (j, r) pairs -> ([n, D] float64, #positions used)."""
        dy = np.ascontiguousarray(dy)
        assert dy.shape == (self.B, self.T, self.hidden) and _dt(dy) == _dt(self.h)
        idx_all = np.ascontiguousarray(idx_all, dtype=np.int32)
        assert idx_all.shape == (self.B * self.T, self.J)
        rj = np.ascontiguousarray(rows_j, dtype=np.int32)
        rr = np.ascontiguousarray(rows_r, dtype=np.int32)
        out = np.empty((rj.size, self.dim), np.float64)
        npos = _load().oracle_table_grad_rows(self.ref, _ptr(dy), _ptr(idx_all), rj.size, _ptr(rj),
                                              _ptr(rr), _ptr(out))
        return out, npos

    def table_grad_dense(self, dy: np.ndarray) -> list:
        dy = np.ascontiguousarray(dy)
        assert dy.shape == (self.B, self.T, self.hidden) and _dt(dy) == _dt(self.h)
        grads = [np.empty((int(m), self.dim), np.float64) for m in self.table_rows]
        ptrs = (ctypes.c_void_p * self.J)(*[g.ctypes.data for g in grads])
        _load().oracle_table_grad_dense(self.ref, _ptr(dy), ctypes.cast(ptrs, ctypes.c_void_p))
        return grads


def e4m3_decode(code: int) -> float:
    """Value of an OCP E4M3 code (0..255; the NaN codes decode as their bit pattern says)."""
    return float(_load().oracle_e4m3_decode(code))


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code, ties to even, saturating at 448."""
    return int(_load().oracle_e4m3_encode(float(x)))


def quantize_rows(x: np.ndarray):
    """Per-row E4M3 quantization of a 2-D array (bf16 bits, fp32 or fp64):
    (codes uint8, scales float32, dequantized float64), scale = max|row| / 448
    and codes of x / scale, both in fp32."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty(rows, np.float32)
    deq = np.empty((rows, cols), np.float64)
    _load().oracle_quantize_rows(_ptr(x), _dt(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(deq))
    return codes, scales, deq


def prefetch_plan(idx: np.ndarray):
    """(uniq [sum counts] int32, counts [J] int64, inv [N, J] int32) for idx [N, J]."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, J = idx.shape
    uniq = np.empty(max(N * J, 1), np.int32)
    counts = np.empty(J, np.int64)
    inv = np.empty((N, J), np.int32)
    _load().oracle_prefetch_plan(N, J, _ptr(idx), _ptr(uniq), _ptr(counts), _ptr(inv))
    return uniq[: int(counts.sum())].copy(), counts, inv


def _widen(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) or fp32 values as float64, exactly."""
    return _widen(a)
