"""Seeded synthetic inputs shared by tests, the bench and ``__graft_entry__``.

This module draws the arrays both sides consume (token streams, the
canonical-id surjection, hash multipliers, table values, projection weights,
hidden states, conv taps, upstream gradients).  It contains no step of the
Engram computation itself.  The counter-based generator lives in ``gen.c``
(splitmix64, element-indexed; Box-Muller normals) and is compiled to
``libsynth.so`` by ``__graft_entry__.build()``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .workloads import WORKLOADS, Workload, get_workload, primes_from  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream numbers (the seed of a stream is 1000 * config_index + stream)
S_TOKENS, S_CANON, S_MULT, S_TABLES, S_WK, S_WV, S_HIDDEN, S_CONV, S_DY = range(1, 10)


def build(verbose: bool = False) -> str:
    import subprocess
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", _LIB_PATH,
           os.path.join(_HERE, "gen.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.synth_u64.argtypes = [u64, u64, i64, vp]
    lib.synth_unit.argtypes = [u64, u64, i64, vp]
    lib.synth_normal_f64.argtypes = [u64, u64, i64, dbl, vp]
    lib.synth_normal_f32.argtypes = [u64, u64, i64, dbl, vp]
    lib.synth_normal_bf16.argtypes = [u64, u64, i64, dbl, vp]
    lib.synth_zipf_cdf.argtypes = [i64, dbl, vp]
    lib.synth_zipf.argtypes = [u64, u64, i64, i64, vp, vp]
    for f in (lib.synth_u64, lib.synth_unit, lib.synth_normal_f64, lib.synth_normal_f32,
              lib.synth_normal_bf16, lib.synth_zipf_cdf, lib.synth_zipf):
        f.restype = None
    _lib = lib
    return lib


def seed_of(cfg_index: int, stream: int) -> int:
    return 1000 * cfg_index + stream


# ---------------------------------------------------------------- raw streams
def u64_stream(seed: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(seed, offset, n, out.ctypes.data)
    return out


def unit_stream(seed: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_unit(seed, offset, n, out.ctypes.data)
    return out


def normal_stream(seed: int, n: int, stdev: float, dtype: str, offset: int = 0,
                  out: np.ndarray | None = None) -> np.ndarray:
    """N(0, stdev^2) values; dtype 'f64', 'f32' or 'bf16' (bf16 as uint16 bits)."""
    lib = _load()
    if dtype == "f64":
        out = np.empty(n, np.float64) if out is None else out
        lib.synth_normal_f64(seed, offset, n, stdev, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, np.float32) if out is None else out
        lib.synth_normal_f32(seed, offset, n, stdev, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, np.uint16) if out is None else out
        lib.synth_normal_bf16(seed, offset, n, stdev, out.ctypes.data)
    else:
        raise ValueError(dtype)
    assert out.size == n and out.flags.c_contiguous
    return out


def zipf_tokens(seed: int, n: int, vocab: int, s: float, offset: int = 0) -> np.ndarray:
    """Elements offset .. offset+n-1 of the token stream (later batches of one
    stream continue it)."""
    lib = _load()
    cdf = np.empty(vocab, np.float64)
    lib.synth_zipf_cdf(vocab, s, cdf.ctypes.data)
    out = np.empty(n, np.int32)
    lib.synth_zipf(seed, offset, n, vocab, cdf.ctypes.data, out.ctypes.data)
    return out


def repeat_tokens(seed: int, n: int, vocab: int, s: float, offset: int = 0, p_copy: float = 0.5,
                  seg: int = 4, reach: int = 8) -> np.ndarray:
    """A token stream with local repetition: the Zipf stream cut into segments
    of `seg` tokens, each of which (with probability p_copy) is replaced by a
    copy of one of the `reach` segments before it, so short N-grams recur
    within a few dozen tokens, as phrases do in text.  Segments are counted
    from the stream start, so consecutive batches (offsets that are multiples
    of seg) continue one stream."""
    assert offset % seg == 0
    out = zipf_tokens(seed, n, vocab, s, offset=offset)
    nseg = n // seg
    s0 = offset // seg
    u = unit_stream(seed + 7919, nseg, offset=s0)
    r = (u64_stream(seed + 7920, nseg, offset=s0) % np.uint64(reach)).astype(np.int64)
    for i in range(nseg):
        src = i - 1 - int(r[i])
        if u[i] < p_copy and src >= 0:
            out[i * seg:(i + 1) * seg] = out[src * seg:(src + 1) * seg]
    return out


def random_surjection(seed: int, vocab: int, canon_vocab: int) -> np.ndarray:
    """Seeded surjection [0,vocab) -> [0,canon_vocab).

    A seeded permutation pi (argsort of stream values) sends pi[i] -> i for
    i < canon_vocab, so every canonical id has a preimage; every other raw id
    goes to a uniformly drawn canonical id.
    """
    keys = u64_stream(seed, vocab)
    perm = np.argsort(keys, kind="stable")
    out = np.empty(vocab, np.int32)
    out[perm[:canon_vocab]] = np.arange(canon_vocab, dtype=np.int32)
    rest = vocab - canon_vocab
    if rest:
        extra = u64_stream(seed, rest, offset=vocab) % np.uint64(canon_vocab)
        out[perm[canon_vocab:]] = extra.astype(np.int32)
    return out


# ------------------------------------------------------------- per workload
class Inputs:
    """All arrays of one workload, drawn lazily from the seeded streams."""

    def __init__(self, wl: Workload):
        self.wl = wl
        self._cache = {}

    def _get(self, key, fn):
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    def drop(self, key):
        self._cache.pop(key, None)

    @property
    def tokens(self) -> np.ndarray:  # int32 [B, T]
        wl = self.wl
        return self._get("tokens", lambda: zipf_tokens(
            seed_of(wl.cfg, S_TOKENS), wl.B * wl.T, wl.vocab, wl.zipf_s).reshape(wl.B, wl.T))

    @property
    def canon_map(self) -> np.ndarray:  # int32 [V]
        wl = self.wl
        return self._get("canon", lambda: random_surjection(
            seed_of(wl.canon_cfg, S_CANON), wl.vocab, wl.canon_vocab))

    @property
    def multipliers(self) -> np.ndarray:  # uint64 [J, max_order], odd
        wl = self.wl
        return self._get("mult", lambda: (u64_stream(
            seed_of(wl.cfg, S_MULT), wl.J * wl.max_order) | np.uint64(1)).reshape(wl.J, wl.max_order))

    @property
    def table_rows(self) -> np.ndarray:  # int64 [J]
        return self._get("rows", lambda: np.asarray(self.wl.rows, dtype=np.int64))

    def table_offsets(self) -> np.ndarray:
        """Element offset of table j inside the table stream."""
        rows = self.table_rows
        return np.concatenate([[0], np.cumsum(rows * self.wl.dim)[:-1]]).astype(np.int64)

    def table(self, j: int) -> np.ndarray:
        """Table j as [M_j, D] (float32, or uint16 bf16 bits)."""
        wl = self.wl

        def mk():
            n = int(self.table_rows[j]) * wl.dim
            a = normal_stream(seed_of(wl.cfg, S_TABLES), n, wl.table_std, wl.dtype,
                              offset=int(self.table_offsets()[j]))
            return a.reshape(int(self.table_rows[j]), wl.dim)
        return self._get(("table", j), mk)

    @property
    def tables(self) -> list:
        return [self.table(j) for j in range(self.wl.J)]

    def _weight(self, stream):
        wl = self.wl
        return normal_stream(seed_of(wl.cfg, stream), wl.hidden * wl.d_mem, wl.w_std,
                             wl.dtype).reshape(wl.hidden, wl.d_mem)

    @property
    def w_k(self) -> np.ndarray:  # [d, d_mem]: k_t = W_K e_t
        return self._get("wk", lambda: self._weight(S_WK))

    @property
    def w_v(self) -> np.ndarray:  # [d, d_mem]
        return self._get("wv", lambda: self._weight(S_WV))

    @property
    def hidden(self) -> np.ndarray:  # [B, T, d]
        wl = self.wl
        return self._get("h", lambda: normal_stream(
            seed_of(wl.cfg, S_HIDDEN), wl.B * wl.T * wl.hidden, 1.0, wl.dtype).reshape(wl.B, wl.T, wl.hidden))

    def w_k_branch(self, m: int) -> np.ndarray:  # [d, d_mem] W_K of branch m (branch 0 = w_k)
        if m == 0:
            return self.w_k
        wl = self.wl
        n = wl.hidden * wl.d_mem
        return self._get(("wk", m), lambda: normal_stream(
            seed_of(wl.cfg, S_WK), n, wl.w_std, wl.dtype, offset=m * n).reshape(wl.hidden, wl.d_mem))

    def hidden_branch(self, m: int) -> np.ndarray:  # [B, T, d] of branch m (branch 0 = hidden)
        if m == 0:
            return self.hidden
        wl = self.wl
        n = wl.B * wl.T * wl.hidden
        return self._get(("h", m), lambda: normal_stream(
            seed_of(wl.cfg, S_HIDDEN), n, 1.0, wl.dtype, offset=m * n).reshape(wl.B, wl.T, wl.hidden))

    @property
    def conv_w(self) -> np.ndarray:  # float32 [d, taps]; tap i multiplies position t-i
        wl = self.wl
        return self._get("conv", lambda: normal_stream(
            seed_of(wl.cfg, S_CONV), wl.hidden * wl.taps, wl.conv_std, "f32").reshape(wl.hidden, wl.taps))

    @property
    def dy(self) -> np.ndarray:  # [B, T, d]
        wl = self.wl
        return self._get("dy", lambda: normal_stream(
            seed_of(wl.cfg, S_DY), wl.B * wl.T * wl.hidden, 1.0, wl.dtype).reshape(wl.B, wl.T, wl.hidden))


    def dy_branch(self, m: int) -> np.ndarray:  # [B, T, d] upstream gradient of branch m's Y
        if m == 0:
            return self.dy
        wl = self.wl
        n = wl.B * wl.T * wl.hidden
        return self._get(("dy", m), lambda: normal_stream(
            seed_of(wl.cfg, S_DY), n, 1.0, wl.dtype, offset=m * n).reshape(wl.B, wl.T, wl.hidden))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def as_float(a: np.ndarray) -> np.ndarray:
    """float view of an input array: bf16 bits -> float32, float arrays unchanged."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else a
