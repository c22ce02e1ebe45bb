"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/engram.h declares, validates arguments before any
GPU work, sizes workspaces, and its host prefetch planner (which runs the
same hash as the device kernel) matches the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def eg():
    import hashed_gram_embedding_canon_amd as eg
    if not os.path.exists(eg.LIB_PATH):
        pytest.fail("libengram.so is not built: run __graft_entry__.build()")
    eg.lib()
    return eg


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "engram.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(eg):
    names = _declared_functions()
    assert len(names) == 17, names
    L = ctypes.CDLL(eg.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(eg.EXPORTS)


def test_status_strings(eg):
    assert eg.engram_status_string(0) == "ok"
    for s in range(1, 6):
        assert eg.engram_status_string(s) not in ("ok", "unknown status")
    assert eg.engram_status_string(99) == "unknown status"


def _cfg(eg, **over):
    wl = synth.get_workload("tiny")
    inp = synth.Inputs(wl)
    kw = dict(vocab=wl.vocab, canon_vocab=wl.canon_vocab, orders=wl.orders, heads=wl.heads,
              dim=wl.dim, hidden=wl.hidden, table_rows=inp.table_rows, multipliers=inp.multipliers,
              dtype=eg.ENGRAM_F32, conv_kernel=4)
    kw.update(over)
    return eg.Config(**kw)


def test_workspace_sizes(eg):
    cfg = _cfg(eg)
    f = eg.engram_workspace_size(cfg, 2, 100, eg.ENGRAM_OP_FORWARD)
    b = eg.engram_workspace_size(cfg, 2, 100, eg.ENGRAM_OP_BACKWARD)
    assert f > 200 * 256 * 4 and b > f  # e alone is N*d_mem*4 bytes
    bp = eg.engram_workspace_size(cfg, 2, 100, eg.ENGRAM_OP_BACKWARD_PARAMS)
    assert bp > b  # the rows gathered again, dW slices and per-block sums on top
    assert eg.engram_workspace_size(cfg, 2, 100, 7) == 0
    assert eg.engram_workspace_size(_cfg(eg, hidden=200), 2, 100, 0) == 0
    assert eg.engram_workspace_size(cfg, -1, 100, 0) == 0


FAKE = 1 << 20  # a 16-byte aligned non-null address; validation fails before any use


def _fwd(eg, cfg, **over):
    p = eg.make_params(canon_map=FAKE, tables=[FAKE] * cfg.J, w_kv=FAKE, conv_w=FAKE)
    kw = dict(tokens=FAKE, hidden=FAKE, B=2, T=8, y=FAKE, workspace=FAKE, ws_bytes=1 << 40)
    kw.update(over)
    return eg.lib().engram_forward(cfg.ref, ctypes.byref(p), kw["tokens"], kw["hidden"], kw["B"],
                                   kw["T"], kw["y"], None, None, kw["workspace"], kw["ws_bytes"], None)


def test_forward_validation(eg):
    bad_orders = _cfg(eg, orders=(3, 2))
    assert _fwd(eg, bad_orders) == eg.ENGRAM_E_INVALID
    assert _fwd(eg, _cfg(eg, orders=(2, 5))) == eg.ENGRAM_E_INVALID
    assert _fwd(eg, _cfg(eg, dtype=7)) == eg.ENGRAM_E_UNSUPPORTED
    assert _fwd(eg, _cfg(eg, hidden=300)) == eg.ENGRAM_E_UNSUPPORTED
    assert _fwd(eg, _cfg(eg, dim=6)) == eg.ENGRAM_E_UNSUPPORTED  # 24-byte rows
    assert _fwd(eg, _cfg(eg, conv_kernel=9)) == eg.ENGRAM_E_UNSUPPORTED
    assert _fwd(eg, _cfg(eg, heads=9)) == eg.ENGRAM_E_UNSUPPORTED  # J = 18 -> d_mem 576
    cfg = _cfg(eg)
    assert _fwd(eg, cfg, hidden=None) == eg.ENGRAM_E_INVALID
    assert _fwd(eg, cfg, y=FAKE + 4) == eg.ENGRAM_E_INVALID  # misaligned
    assert _fwd(eg, cfg, B=-1) == eg.ENGRAM_E_INVALID
    assert _fwd(eg, cfg, workspace=None) == eg.ENGRAM_E_WORKSPACE
    assert _fwd(eg, cfg, ws_bytes=1000) == eg.ENGRAM_E_WORKSPACE
    assert _fwd(eg, cfg, B=0) == eg.ENGRAM_OK  # empty batch: nothing to do
    assert _fwd(eg, cfg, T=0) == eg.ENGRAM_OK
    rows = np.array([10007] * 7 + [0], np.int64)
    assert _fwd(eg, _cfg(eg, table_rows=rows)) == eg.ENGRAM_E_INVALID
    # the FP8 projection: bf16 only, d_mem <= 4096, not with the fused gather
    fp8 = eg.ENGRAM_FLAG_FP8_PROJ
    assert _fwd(eg, _cfg(eg, flags=fp8)) == eg.ENGRAM_E_UNSUPPORTED  # fp32
    assert _fwd(eg, _cfg(eg, flags=fp8 | eg.ENGRAM_FLAG_FUSED_GATHER,
                         dtype=eg.ENGRAM_BF16)) == eg.ENGRAM_E_UNSUPPORTED
    wide = dict(dtype=eg.ENGRAM_BF16, flags=fp8, heads=8, dim=512,
                table_rows=np.full(16, 10007, np.int64), multipliers=np.ones((16, 3), np.uint64))
    assert _fwd(eg, _cfg(eg, **wide)) == eg.ENGRAM_E_UNSUPPORTED  # d_mem 8192
    assert eg.engram_workspace_size(_cfg(eg, **dict(wide, dim=256)), 2, 8, 0) > 0  # d_mem 4096


def test_id_check_validation(eg):
    """ENGRAM_FLAG_CHECK_IDS needs a 4-byte aligned device counter; without one
    the call is rejected on the host, before any GPU work."""
    chk = eg.ENGRAM_FLAG_CHECK_IDS
    L = eg.lib()
    for bad in (None, FAKE + 2):
        cfg = _cfg(eg, flags=chk, bad_ids=bad)
        assert _fwd(eg, cfg) == eg.ENGRAM_E_INVALID
        assert L.engram_hash_indices(cfg.ref, FAKE, FAKE, 2, 8, FAKE, None) == eg.ENGRAM_E_INVALID
        assert eg.engram_workspace_size(cfg, 2, 8, eg.ENGRAM_OP_FORWARD) == 0
    ok = _cfg(eg, flags=chk, bad_ids=FAKE + 4)
    assert eg.engram_workspace_size(ok, 2, 8, eg.ENGRAM_OP_FORWARD) == \
        eg.engram_workspace_size(_cfg(eg), 2, 8, eg.ENGRAM_OP_FORWARD)
    assert _fwd(eg, ok, B=0) == eg.ENGRAM_OK  # no tokens: nothing queued, no sync
    assert _fwd(eg, _cfg(eg, flags=16)) == eg.ENGRAM_E_INVALID  # unknown flag bit


def test_gather_dedup_shape_limit(eg):
    """The LDS dedup gather stages a 16-token tile's rows (at most 64 KB)."""
    dd = eg.ENGRAM_FLAG_GATHER_DEDUP
    assert eg.engram_workspace_size(_cfg(eg, flags=dd), 2, 8, eg.ENGRAM_OP_FORWARD) > 0  # 16 KB
    assert _fwd(eg, _cfg(eg, flags=dd, dim=256)) == eg.ENGRAM_E_UNSUPPORTED  # 128 KB


def test_noalloc_forward_host_checks(eg):
    """The allocation-free forward validates like engram_forward and refuses an
    input whose scratch exceeds its fixed array, before any GPU work."""
    L = eg.lib()
    cfg = _cfg(eg)
    p = eg.make_params(canon_map=FAKE, tables=[FAKE] * cfg.J, w_kv=FAKE, conv_w=FAKE)

    def call(cfg, B, T, hidden=FAKE):
        return L.engram_forward_noalloc(cfg.ref, ctypes.byref(p), FAKE, hidden, B, T, FAKE, None, None,
                                        None)
    assert call(_cfg(eg, orders=(3, 2)), 2, 8) == eg.ENGRAM_E_INVALID
    assert call(cfg, 2, 8, hidden=None) == eg.ENGRAM_E_INVALID
    assert call(cfg, 0, 8) == eg.ENGRAM_OK
    per_tok = eg.engram_workspace_size(cfg, 1, 1024, eg.ENGRAM_OP_FORWARD) / 1024
    too_many = int(eg.ENGRAM_NOALLOC_SCRATCH_BYTES / per_tok) + 4096
    assert call(cfg, 1, too_many) == eg.ENGRAM_E_SCRATCH
    assert "scratch" in eg.engram_status_string(eg.ENGRAM_E_SCRATCH)


def test_backward_and_hash_validation(eg):
    cfg = _cfg(eg)
    L = eg.lib()
    p = eg.make_params(canon_map=FAKE, tables=[FAKE] * cfg.J, w_kv=FAKE, conv_w=FAKE)
    out = eg.engram_table_grad()
    out.mode = 5
    assert L.engram_backward_table_grad(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, None,
                                        ctypes.byref(out), FAKE, 1 << 40, None) == eg.ENGRAM_E_INVALID
    out.mode = eg.ENGRAM_GRAD_SORTED_SPARSE
    out.keys = out.rows = out.count = FAKE
    # saved tensors are required
    assert L.engram_backward_table_grad(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, None,
                                        ctypes.byref(out), FAKE, 1 << 40, None) == eg.ENGRAM_E_INVALID
    sv = eg.make_saved(idx=FAKE, stats=FAKE, k=FAKE, v=FAKE)
    assert L.engram_backward_table_grad(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, ctypes.byref(sv),
                                        ctypes.byref(out), FAKE, 16, None) == eg.ENGRAM_E_WORKSPACE
    out.mode = eg.ENGRAM_GRAD_ATOMIC_DENSE  # dense pointers missing
    assert L.engram_backward_table_grad(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, ctypes.byref(sv),
                                        ctypes.byref(out), FAKE, 1 << 40, None) == eg.ENGRAM_E_INVALID
    # engram_backward: at least one output; parameter grads need d_mem % 256 == 0
    out.mode = eg.ENGRAM_GRAD_SORTED_SPARSE
    assert L.engram_backward(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, ctypes.byref(sv), None,
                             None, FAKE, 1 << 40, None) == eg.ENGRAM_E_INVALID
    pg = eg.make_param_grad(w_kv=FAKE, conv_w=FAKE)
    assert L.engram_backward(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, ctypes.byref(sv), None,
                             ctypes.byref(pg), FAKE, 16, None) == eg.ENGRAM_E_WORKSPACE
    pg_bad = eg.make_param_grad(w_kv=FAKE + 4)
    assert L.engram_backward(cfg.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, ctypes.byref(sv), None,
                             ctypes.byref(pg_bad), FAKE, 1 << 40, None) == eg.ENGRAM_E_INVALID
    odd = _cfg(eg, dim=40)  # d_mem = 320
    assert L.engram_backward(odd.ref, ctypes.byref(p), FAKE, FAKE, 2, 8, ctypes.byref(sv), None,
                             ctypes.byref(pg), FAKE, 1 << 40, None) == eg.ENGRAM_E_UNSUPPORTED
    assert L.engram_hash_indices(cfg.ref, None, FAKE, 2, 8, FAKE, None) == eg.ENGRAM_E_INVALID
    assert L.engram_hash_indices(cfg.ref, FAKE, FAKE, 0, 8, FAKE, None) == eg.ENGRAM_OK


def _plan(eg, cfg, tokens, canon, J):
    N = tokens.size
    cap = N * J
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(max(cap, 1), np.int32)
    inv = np.zeros((N, J), np.int32)
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host, plan.inverse_host = counts.ctypes.data, uniq.ctypes.data, inv.ctypes.data
    eg.engram_prefetch_plan(cfg, canon, tokens, B=tokens.shape[0], T=tokens.shape[1], plan=plan)
    return uniq[: plan.total_rows], counts, inv


@pytest.mark.parametrize("name,B,T", [("tiny", 1, 512), ("tiny", 3, 77), ("small", 2, 1500)])
def test_host_plan_matches_oracle(eg, oracle_lib, name, B, T):
    """Host planner (same hash code as the device kernel) vs the oracle: bit-exact."""
    wl = synth.get_workload(name).with_shape(B, T)
    inp = synth.Inputs(wl)
    cfg = eg.Config(vocab=wl.vocab, canon_vocab=wl.canon_vocab, orders=wl.orders, heads=wl.heads,
                    dim=wl.dim, hidden=wl.hidden, table_rows=inp.table_rows,
                    multipliers=inp.multipliers, dtype=eg.ENGRAM_BF16 if wl.dtype == "bf16" else 0)
    tabs = [np.zeros((int(m), 1), np.float32) for m in inp.table_rows]  # rows are not read
    p = oracle_lib.Problem(orders=wl.orders, heads=wl.heads, mult=inp.multipliers,
                           table_rows=inp.table_rows, pad_id=wl.pad_id, canon_map=inp.canon_map,
                           tokens=inp.tokens, tables=tabs)
    idx = p.hash()
    u_ref, c_ref, inv_ref = oracle_lib.prefetch_plan(idx)
    u, c, inv = _plan(eg, cfg, inp.tokens, inp.canon_map, wl.J)
    assert np.array_equal(c, c_ref)
    assert np.array_equal(u, u_ref)
    base = np.concatenate([[0], np.cumsum(c_ref)[:-1]])
    assert np.array_equal(inv, inv_ref + base[None, :].astype(np.int32))


def test_host_plan_adversarial_multipliers(eg, oracle_lib):
    """Multipliers near 2^64 and large ids stress the 64-bit wrap and the mod-prime reduction."""
    V = 1 << 17
    J = 4
    rows = np.array([2147483647, 4450003, 13, 1000003], np.int64)  # includes 2^31-1
    mult = np.array([[2**64 - 1, 2**63 + 1, 3], [2**64 - 3, 1, 2**62 + 7], [5, 7, 2**64 - 5],
                     [2**63 - 1, 2**64 - 7, 9]], dtype=np.uint64)
    tokens = (synth.u64_stream(3, 2 * 300) % np.uint64(V)).astype(np.int32).reshape(2, 300)
    tokens[0, :4] = V - 1
    canon = np.arange(V, dtype=np.int32)
    cfg = eg.Config(vocab=V, canon_vocab=V, orders=(2, 3), heads=2, dim=64, hidden=256,
                    table_rows=rows, multipliers=mult, dtype=eg.ENGRAM_BF16)
    tabs = [np.zeros((1, 1), np.float32)] * J
    # a hash-only oracle problem: tables are never read by hash()
    p = oracle_lib.Problem(orders=(2, 3), heads=2, mult=mult, table_rows=[1] * J, pad_id=0,
                           canon_map=canon, tokens=tokens, tables=tabs)
    p.table_rows[:] = rows  # the hash reads M_j through this array
    idx = p.hash()
    u_ref, c_ref, inv_ref = oracle_lib.prefetch_plan(idx)
    u, c, inv = _plan(eg, cfg, tokens, canon, J)
    assert np.array_equal(c, c_ref) and np.array_equal(u, u_ref)
    # brute force of a few positions with Python integers
    for (b, t) in ((0, 0), (0, 3), (1, 299)):
        ctx = [int(tokens[b, t - i]) if t - i >= 0 else 0 for i in range(3)]
        j = 0
        for n in (2, 3):
            for _ in range(2):
                x = 0
                for i in range(n):
                    x ^= (int(mult[j, i]) * ctx[i]) % (1 << 64)
                assert idx[b * 300 + t, j] == x % int(rows[j])
                j += 1


def test_row_ring_validation(eg):
    """The HBM row ring is checked on the host before any copy is queued."""
    cfg = _cfg(eg)
    N, J = 2 * 8, cfg.J
    tokens = np.ones((2, 8), np.int32)
    canon = np.zeros(cfg.c.vocab, np.int32)
    cap = N * J
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(cap, np.int32)
    inv = np.zeros((N, J), np.int32)
    pos = np.full(10, -1, np.int64)
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host, plan.inverse_host = counts.ctypes.data, uniq.ctypes.data, inv.ctypes.data
    plan.staging_host = plan.rows_dev = plan.inverse_dev = FAKE
    tabs = (ctypes.c_void_p * J)(*([FAKE] * J))
    L = eg.lib()
    for R, p, head in ((2 * cap - 1, pos, 0), (2 * cap, None, 0), (2 * cap, pos, -1), (1 << 31, pos, 0)):
        plan.ring_rows, plan.ring_head = R, head
        plan.ring_pos = None if p is None else p.ctypes.data
        assert L.engram_prefetch_plan(cfg.ref, canon.ctypes.data, tokens.ctypes.data, 2, 8, tabs,
                                      ctypes.byref(plan), None) == eg.ENGRAM_E_INVALID


def test_shard_validation(eg):
    """Sharded exchange calls reject bad GPU counts, buffers and workspaces on the host."""
    cfg = _cfg(eg)
    L = eg.lib()
    for G in (0, eg.ENGRAM_SHARD_MAX_GPUS + 1):
        assert L.engram_shard_requests(cfg.ref, G, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                       None) == eg.ENGRAM_E_INVALID
        assert L.engram_shard_serve(cfg.ref, G, FAKE, FAKE, 4, FAKE, None) == eg.ENGRAM_E_INVALID
    assert L.engram_shard_requests(cfg.ref, 4, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 64,
                                   None) == eg.ENGRAM_E_WORKSPACE
    assert L.engram_shard_requests(cfg.ref, 4, None, 16, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                   None) == eg.ENGRAM_E_INVALID
    assert L.engram_shard_grads(cfg.ref, 4, FAKE, FAKE + 4, FAKE, 16, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                None) == eg.ENGRAM_E_INVALID  # misaligned rows
    counts = (ctypes.c_int64 * 2)(3, -1)
    assert L.engram_shard_reduce(cfg.ref, 4, FAKE, FAKE, FAKE, counts, 2, None) == eg.ENGRAM_E_INVALID
    # shards of 2^27 rows or more cannot be named by a request id
    big = _cfg(eg, table_rows=np.array([(1 << 27) + 1] * 8, np.int64))
    assert L.engram_shard_serve(big.ref, 1, FAKE, FAKE, 4, FAKE, None) == eg.ENGRAM_E_UNSUPPORTED
    assert eg.engram_workspace_size(cfg, 2, 100, eg.ENGRAM_OP_SHARD) > 0


def test_device_copy_validation(eg):
    L = eg.lib()
    assert L.engram_device_copy(FAKE, FAKE + 16, 24, None) == eg.ENGRAM_E_INVALID  # not 16-byte pieces
    assert L.engram_device_copy(FAKE + 8, FAKE, 32, None) == eg.ENGRAM_E_INVALID   # misaligned
    assert L.engram_device_copy(None, FAKE, 32, None) == eg.ENGRAM_E_INVALID
    assert L.engram_device_copy(FAKE, FAKE, 0, None) == eg.ENGRAM_OK


def test_profile_api_without_launches(eg):
    eg.engram_profile_enable(True)
    eg.engram_profile_reset()
    assert eg.engram_profile_read() == {}
    eg.engram_profile_enable(False)


def test_quantize_fp8_validation(eg):
    L = eg.lib()
    q = lambda *a: L.engram_quantize_fp8(*a, None)  # noqa: E731
    assert q(FAKE, 7, 4, 64, FAKE, FAKE) == eg.ENGRAM_E_UNSUPPORTED        # dtype
    assert q(FAKE, eg.ENGRAM_BF16, -1, 64, FAKE, FAKE) == eg.ENGRAM_E_INVALID
    assert q(FAKE, eg.ENGRAM_BF16, 4, 60, FAKE, FAKE) == eg.ENGRAM_E_INVALID  # cols % 8
    assert q(FAKE, eg.ENGRAM_BF16, 4, 0, FAKE, FAKE) == eg.ENGRAM_E_INVALID
    assert q(None, eg.ENGRAM_BF16, 4, 64, FAKE, FAKE) == eg.ENGRAM_E_INVALID
    assert q(FAKE + 8, eg.ENGRAM_BF16, 4, 64, FAKE, FAKE) == eg.ENGRAM_E_INVALID  # src alignment
    assert q(FAKE, eg.ENGRAM_BF16, 4, 64, FAKE + 4, FAKE) == eg.ENGRAM_E_INVALID  # codes alignment
    assert q(FAKE, eg.ENGRAM_BF16, 0, 64, FAKE, FAKE) == eg.ENGRAM_OK         # nothing to do
