"""Python binding of libengram.so, the MI355X (gfx950) Engram library.

Argument marshalling only: every step of the hot path runs in the HIP
kernels behind the C ABI declared in ``include/engram.h``.  PyTorch is used
for device memory and streams.  The functions keep the C names; tensors are
passed by pointer, the current torch stream is used when no stream is given.
Importing works without a GPU (the library only needs the HIP runtime to
load); calling a device entry point needs one.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")

ENGRAM_OK, ENGRAM_E_INVALID, ENGRAM_E_UNSUPPORTED, ENGRAM_E_WORKSPACE, ENGRAM_E_HIP, ENGRAM_E_SCRATCH = range(6)
ENGRAM_NOALLOC_SCRATCH_BYTES = 64 << 20
ENGRAM_F32, ENGRAM_BF16 = 0, 1
ENGRAM_MAX_ORDERS = 4
ENGRAM_MAX_TABLES = 32
ENGRAM_MAX_BRANCHES = 8
ENGRAM_FLAG_FUSED_GATHER = 1
ENGRAM_FLAG_FP8_PROJ = 2
ENGRAM_FLAG_CHECK_IDS = 4
ENGRAM_FLAG_GATHER_DEDUP = 8
ENGRAM_PLAN_REUSE = 1
ENGRAM_GRAD_SORTED_SPARSE, ENGRAM_GRAD_SORTED_DENSE, ENGRAM_GRAD_ATOMIC_DENSE = 0, 1, 2
ENGRAM_OP_FORWARD, ENGRAM_OP_BACKWARD, ENGRAM_OP_BACKWARD_PARAMS, ENGRAM_OP_SHARD = 0, 1, 2, 3
ENGRAM_SHARD_MAX_GPUS = 64

_vp = ctypes.c_void_p


class engram_config(ctypes.Structure):
    _fields_ = [
        ("vocab", ctypes.c_int32),
        ("canon_vocab", ctypes.c_int32),
        ("num_orders", ctypes.c_int32),
        ("orders", ctypes.c_int32 * ENGRAM_MAX_ORDERS),
        ("heads", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("conv_kernel", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("pad_id", ctypes.c_int32),
        ("table_rows", _vp),
        ("multipliers", _vp),
        ("flags", ctypes.c_uint32),
        ("branches", ctypes.c_int32),
        ("bad_ids", _vp),
    ]


class engram_params(ctypes.Structure):
    _fields_ = [
        ("canon_map", _vp),
        ("tables", _vp * ENGRAM_MAX_TABLES),
        ("w_kv", _vp),
        ("gamma_q", _vp),
        ("gamma_k", _vp),
        ("conv_w", _vp),
    ]


class engram_saved(ctypes.Structure):
    _fields_ = [("idx", _vp), ("stats", _vp), ("k", _vp), ("v", _vp), ("e", _vp)]


class engram_compact(ctypes.Structure):
    _fields_ = [
        ("capacity_rows", ctypes.c_int64),
        ("total_rows", ctypes.c_int64),
        ("counts", _vp),
        ("uniq_host", _vp),
        ("inverse_host", _vp),
        ("staging_host", _vp),
        ("rows_dev", _vp),
        ("inverse_dev", _vp),
        ("ready_event", _vp),
        ("flags", ctypes.c_uint32),
        ("ring_rows", ctypes.c_int64),
        ("ring_pos", _vp),
        ("ring_head", ctypes.c_int64),
        ("ring_hits", ctypes.c_int64),
        ("consumed_event", _vp),
    ]


class engram_table_grad(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("keys", _vp),
        ("rows", _vp),
        ("count", _vp),
        ("dense", _vp * ENGRAM_MAX_TABLES),
    ]


class engram_param_grad(ctypes.Structure):
    _fields_ = [
        ("w_kv", _vp),
        ("conv_w", _vp),
        ("gamma_q", _vp),
        ("gamma_k", _vp),
        ("hidden", _vp),
    ]


class EngramError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {engram_status_string(status)} (status {status})")
        self.status = status


EXPORTS = ("engram_workspace_size", "engram_status_string", "engram_hash_indices", "engram_forward",
           "engram_forward_noalloc",
           "engram_backward_table_grad", "engram_backward", "engram_prefetch_plan",
           "engram_shard_requests", "engram_shard_serve", "engram_shard_grads", "engram_shard_reduce",
           "engram_quantize_fp8", "engram_device_copy",
           "engram_profile_enable",
           "engram_profile_reset", "engram_profile_read")

_lib = None


def lib():
    """The loaded libengram.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hashed_gram_embedding_canon_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    C, P, S, K, G, PG = (ctypes.POINTER(engram_config), ctypes.POINTER(engram_params),
                         ctypes.POINTER(engram_saved), ctypes.POINTER(engram_compact),
                         ctypes.POINTER(engram_table_grad), ctypes.POINTER(engram_param_grad))
    L.engram_workspace_size.argtypes = [C, i64, i64, i32]
    L.engram_workspace_size.restype = sz
    L.engram_status_string.argtypes = [ctypes.c_int]
    L.engram_status_string.restype = ctypes.c_char_p
    L.engram_hash_indices.argtypes = [C, _vp, _vp, i64, i64, _vp, _vp]
    L.engram_forward.argtypes = [C, P, _vp, _vp, i64, i64, _vp, S, K, _vp, sz, _vp]
    L.engram_forward_noalloc.argtypes = [C, P, _vp, _vp, i64, i64, _vp, S, K, _vp]
    L.engram_backward_table_grad.argtypes = [C, P, _vp, _vp, i64, i64, S, G, _vp, sz, _vp]
    L.engram_backward.argtypes = [C, P, _vp, _vp, i64, i64, S, G, PG, _vp, sz, _vp]
    L.engram_prefetch_plan.argtypes = [C, _vp, _vp, i64, i64, _vp, K, _vp]
    L.engram_shard_requests.argtypes = [C, i32, _vp, i64, _vp, _vp, _vp, _vp, sz, _vp]
    L.engram_quantize_fp8.argtypes = [_vp, i32, i64, i32, _vp, _vp, _vp]
    L.engram_device_copy.argtypes = [_vp, _vp, sz, _vp]
    L.engram_shard_serve.argtypes = [C, i32, _vp, _vp, i64, _vp, _vp]
    L.engram_shard_grads.argtypes = [C, i32, _vp, _vp, _vp, i64, _vp, _vp, _vp, _vp, sz, _vp]
    L.engram_shard_reduce.argtypes = [C, i32, _vp, _vp, _vp, _vp, i32, _vp]
    L.engram_profile_enable.argtypes = [i32]
    L.engram_profile_enable.restype = None
    L.engram_profile_reset.argtypes = []
    L.engram_profile_reset.restype = None
    L.engram_profile_read.argtypes = [ctypes.c_char_p, sz, _vp, _vp, i32]
    L.engram_profile_read.restype = i32
    for name in ("engram_hash_indices", "engram_forward", "engram_forward_noalloc",
                 "engram_backward_table_grad",
                 "engram_backward", "engram_prefetch_plan", "engram_shard_requests",
                 "engram_shard_serve", "engram_shard_grads", "engram_shard_reduce",
                 "engram_quantize_fp8", "engram_device_copy"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


# ------------------------------------------------------------------ helpers
def _ptr(x) -> int | None:
    """Address of a torch tensor, numpy array, raw int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != ENGRAM_OK:
        raise EngramError(status, where)


class Config:
    """engram_config plus the host arrays it points at (kept alive here)."""

    def __init__(self, *, vocab, canon_vocab, orders, heads, dim, hidden, table_rows, multipliers,
                 dtype=ENGRAM_BF16, conv_kernel=4, rms_eps=1e-6, pad_id=0, flags=0, branches=1,
                 bad_ids=None):
        import numpy as np
        self.table_rows = np.ascontiguousarray(table_rows, dtype=np.int64)
        self.multipliers = np.ascontiguousarray(multipliers, dtype=np.uint64)
        c = engram_config()
        c.vocab, c.canon_vocab = int(vocab), int(canon_vocab)
        c.num_orders = len(orders)
        for i, o in enumerate(orders):
            c.orders[i] = int(o)
        c.heads, c.dim, c.hidden = int(heads), int(dim), int(hidden)
        c.conv_kernel, c.dtype = int(conv_kernel), int(dtype)
        c.rms_eps, c.pad_id = float(rms_eps), int(pad_id)
        c.table_rows = self.table_rows.ctypes.data
        c.multipliers = self.multipliers.ctypes.data
        c.flags = int(flags)
        c.branches = int(branches)
        c.bad_ids = _ptr(bad_ids)
        self.c = c
        self.branches = max(1, int(branches))
        self.J = len(orders) * int(heads)
        self.d_mem = self.J * int(dim)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def make_params(*, canon_map, tables, w_kv, conv_w, gamma_q=None, gamma_k=None) -> engram_params:
    p = engram_params()
    p.canon_map = _ptr(canon_map)
    for j, t in enumerate(tables):
        p.tables[j] = _ptr(t)
    p.w_kv = _ptr(w_kv)
    p.gamma_q = _ptr(gamma_q)
    p.gamma_k = _ptr(gamma_k)
    p.conv_w = _ptr(conv_w)
    return p


def make_saved(*, idx=None, stats=None, k=None, v=None, e=None) -> engram_saved:
    s = engram_saved()
    s.idx, s.stats, s.k, s.v, s.e = _ptr(idx), _ptr(stats), _ptr(k), _ptr(v), _ptr(e)
    return s


# ------------------------------------------------------------ entry points
def engram_workspace_size(cfg: Config, B: int, T: int, op: int) -> int:
    return int(lib().engram_workspace_size(cfg.ref, B, T, op))


def engram_status_string(status: int) -> str:
    return lib().engram_status_string(status).decode()


def engram_hash_indices(cfg: Config, canon_map, tokens, idx, *, B: int, T: int, stream=None):
    _check(lib().engram_hash_indices(cfg.ref, _ptr(canon_map), _ptr(tokens), B, T, _ptr(idx),
                                     _stream(stream)), "engram_hash_indices")


def engram_forward(cfg: Config, params: engram_params, tokens, hidden, y, *, B: int, T: int,
                   saved: engram_saved | None = None, compact: engram_compact | None = None,
                   workspace=None, ws_bytes: int | None = None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().engram_forward(cfg.ref, ctypes.byref(params), _ptr(tokens), _ptr(hidden), B, T,
                                _ptr(y), ctypes.byref(saved) if saved is not None else None,
                                ctypes.byref(compact) if compact is not None else None,
                                _ptr(workspace), ws_bytes, _stream(stream)), "engram_forward")


def engram_forward_noalloc(cfg: Config, params: engram_params, tokens, hidden, y, *, B: int, T: int,
                           saved: engram_saved | None = None, compact: engram_compact | None = None,
                           stream=None):
    _check(lib().engram_forward_noalloc(cfg.ref, ctypes.byref(params), _ptr(tokens), _ptr(hidden), B,
                                        T, _ptr(y), ctypes.byref(saved) if saved is not None else None,
                                        ctypes.byref(compact) if compact is not None else None,
                                        _stream(stream)), "engram_forward_noalloc")


def engram_backward_table_grad(cfg: Config, params: engram_params, hidden, dy, *, B: int, T: int,
                               saved: engram_saved, out: engram_table_grad, workspace=None,
                               ws_bytes: int | None = None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().engram_backward_table_grad(cfg.ref, ctypes.byref(params), _ptr(hidden), _ptr(dy),
                                            B, T, ctypes.byref(saved) if saved is not None else None,
                                            ctypes.byref(out), _ptr(workspace), ws_bytes,
                                            _stream(stream)), "engram_backward_table_grad")


def make_param_grad(*, w_kv=None, conv_w=None, gamma_q=None, gamma_k=None,
                    hidden=None) -> engram_param_grad:
    g = engram_param_grad()
    g.w_kv, g.conv_w, g.gamma_q, g.gamma_k, g.hidden = (_ptr(w_kv), _ptr(conv_w), _ptr(gamma_q),
                                                        _ptr(gamma_k), _ptr(hidden))
    return g


def engram_backward(cfg: Config, params: engram_params, hidden, dy, *, B: int, T: int,
                    saved: engram_saved, table_out: engram_table_grad | None = None,
                    param_out: engram_param_grad | None = None, workspace=None,
                    ws_bytes: int | None = None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().engram_backward(cfg.ref, ctypes.byref(params), _ptr(hidden), _ptr(dy), B, T,
                                 ctypes.byref(saved) if saved is not None else None,
                                 ctypes.byref(table_out) if table_out is not None else None,
                                 ctypes.byref(param_out) if param_out is not None else None,
                                 _ptr(workspace), ws_bytes, _stream(stream)), "engram_backward")


def _ws_bytes(workspace, ws_bytes):
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return ws_bytes


def engram_quantize_fp8(src, dtype: int, rows: int, cols: int, codes, scales, *, stream=None):
    _check(lib().engram_quantize_fp8(_ptr(src), dtype, rows, cols, _ptr(codes), _ptr(scales),
                                     _stream(stream)), "engram_quantize_fp8")


def engram_shard_requests(cfg: Config, G: int, idx, N: int, send_ids, send_counts, inverse, *,
                          workspace=None, ws_bytes: int | None = None, stream=None):
    _check(lib().engram_shard_requests(cfg.ref, G, _ptr(idx), N, _ptr(send_ids), _ptr(send_counts),
                                       _ptr(inverse), _ptr(workspace), _ws_bytes(workspace, ws_bytes),
                                       _stream(stream)), "engram_shard_requests")


def engram_shard_serve(cfg: Config, G: int, shard_tables, ids, n: int, rows_out, *, stream=None):
    tabs = (ctypes.c_void_p * len(shard_tables))(*[_ptr(t) for t in shard_tables])
    _check(lib().engram_shard_serve(cfg.ref, G, ctypes.cast(tabs, ctypes.c_void_p), _ptr(ids), n,
                                    _ptr(rows_out), _stream(stream)), "engram_shard_serve")


def engram_shard_grads(cfg: Config, G: int, keys, rows, count, capacity: int, send_ids, send_rows,
                       send_counts, *, workspace=None, ws_bytes: int | None = None, stream=None):
    _check(lib().engram_shard_grads(cfg.ref, G, _ptr(keys), _ptr(rows), _ptr(count), capacity,
                                    _ptr(send_ids), _ptr(send_rows), _ptr(send_counts),
                                    _ptr(workspace), _ws_bytes(workspace, ws_bytes), _stream(stream)),
           "engram_shard_grads")


def engram_shard_reduce(cfg: Config, G: int, shard_grads, ids, rows, counts_host, *, stream=None):
    grads = (ctypes.c_void_p * len(shard_grads))(*[_ptr(t) for t in shard_grads])
    counts = (ctypes.c_int64 * len(counts_host))(*[int(c) for c in counts_host])
    _check(lib().engram_shard_reduce(cfg.ref, G, ctypes.cast(grads, ctypes.c_void_p), _ptr(ids),
                                     _ptr(rows), ctypes.cast(counts, ctypes.c_void_p), len(counts_host),
                                     _stream(stream)), "engram_shard_reduce")


def engram_prefetch_plan(cfg: Config, canon_map_host, tokens_host, *, B: int, T: int,
                         host_tables=None, plan: engram_compact, side_stream=None):
    tabs = None
    if host_tables is not None:
        tabs = (_vp * len(host_tables))(*[_ptr(t) for t in host_tables])
    ss = None
    if host_tables is not None:
        ss = _stream(side_stream)
    _check(lib().engram_prefetch_plan(cfg.ref, _ptr(canon_map_host), _ptr(tokens_host), B, T,
                                      ctypes.cast(tabs, _vp) if tabs is not None else None,
                                      ctypes.byref(plan), ss), "engram_prefetch_plan")


def engram_device_copy(dst, src, nbytes: int, *, stream=None):
    _check(lib().engram_device_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "engram_device_copy")


def engram_profile_enable(on: bool):
    lib().engram_profile_enable(1 if on else 0)


def engram_profile_reset():
    lib().engram_profile_reset()


def engram_profile_read(max_entries: int = 64) -> dict:
    """{kernel name: (launches, total ms)} of the launches timed since the last read."""
    import numpy as np
    names = ctypes.create_string_buffer(64 * max_entries)
    cnt = np.zeros(max_entries, np.int64)
    ms = np.zeros(max_entries, np.float64)
    n = lib().engram_profile_read(names, len(names), cnt.ctypes.data, ms.ctypes.data, max_entries)
    if n < 0:
        raise EngramError(ENGRAM_E_HIP, "engram_profile_read")
    out = {}
    parts = names.raw.split(b"\0")
    for i in range(n):
        out[parts[i].decode()] = (int(cnt[i]), float(ms[i]))
    return out
