"""GPU parity of the table-gradient backward against the oracle.

Bar: relative L2 <= 1e-3 of the table gradients (fp32 accumulation), for
the sorted segmented reduction (sparse and dense outputs) and the atomic
variant; the sparse keys must be exactly the distinct (table, row) pairs,
ascending; sorted and atomic results agree to the same bound.
"""
import dataclasses

import numpy as np
import pytest

import synth
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


def _fwd_bwd(torch, wl, modes):
    import hashed_gram_embedding_canon_amd as eg
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    dy = H.to_dev(inp.dy)
    out = {m: dp.backward(bufs, dy, m) for m in modes}
    torch.cuda.synchronize()
    return inp, dp, bufs, out


def _sparse_to_dict(res, D):
    n = int(res["count"].item())
    keys = res["keys"][:n].cpu().numpy()
    rows = res["rows"][:n].cpu().numpy().astype(np.float64)
    return keys, rows


@pytest.mark.parametrize("dtype,B,T,hidden", [("f32", 1, 512, 256), ("f32", 3, 77, 256), ("bf16", 2, 300, 256),
                                              ("bf16", 1, 200, 4096)])
def test_tiny_table_grads(torch, oracle_lib, dtype, B, T, hidden):
    """hidden 4096: 1024 lanes per workgroup in the elementwise backward."""
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype=dtype, hidden=hidden).with_shape(B, T)
    print(f"[tiny bwd {dtype}] B={B} T={T} d={hidden}", flush=True)
    modes = (eg.ENGRAM_GRAD_SORTED_SPARSE, eg.ENGRAM_GRAD_SORTED_DENSE, eg.ENGRAM_GRAD_ATOMIC_DENSE)
    inp, dp, bufs, out = _fwd_bwd(torch, wl, modes)
    p = H.oracle_problem(inp)
    ref = p.table_grad_dense(inp.dy)
    idx = p.hash()
    # sparse: keys are exactly the distinct (j, row) pairs in ascending order
    keys, rows = _sparse_to_dict(out[eg.ENGRAM_GRAD_SORTED_SPARSE], wl.dim)
    want = np.unique(np.concatenate([(np.int64(j) << 32) | idx[:, j].astype(np.int64)
                                     for j in range(wl.J)]))
    assert np.array_equal(keys, want)
    ref_rows = np.stack([ref[int(k >> 32)][int(k & 0xFFFFFFFF)] for k in keys])
    err = H.rel_l2(rows, ref_rows)
    assert err <= 1e-3, err
    for mode in (eg.ENGRAM_GRAD_SORTED_DENSE, eg.ENGRAM_GRAD_ATOMIC_DENSE):
        dense = out[mode]["dense"]
        got = np.concatenate([d.cpu().numpy().astype(np.float64).ravel() for d in dense])
        refc = np.concatenate([r.ravel() for r in ref])
        err = H.rel_l2(got, refc)
        assert err <= 1e-3, (mode, err)
    # sorted and atomic agree
    a = np.concatenate([d.cpu().numpy().ravel() for d in out[eg.ENGRAM_GRAD_ATOMIC_DENSE]["dense"]])
    s = np.concatenate([d.cpu().numpy().ravel() for d in out[eg.ENGRAM_GRAD_SORTED_DENSE]["dense"]])
    assert H.rel_l2(a.astype(np.float64), s.astype(np.float64)) <= 1e-3


def test_sorted_path_is_deterministic(torch):
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype="bf16").with_shape(2, 300)
    inp, dp, bufs, out = _fwd_bwd(torch, wl, (eg.ENGRAM_GRAD_SORTED_SPARSE,))
    again = dp.backward(bufs, H.to_dev(inp.dy), eg.ENGRAM_GRAD_SORTED_SPARSE)
    torch.cuda.synchronize()
    r1, r2 = out[eg.ENGRAM_GRAD_SORTED_SPARSE], again
    n = int(r1["count"].item())
    assert n == int(r2["count"].item())
    assert torch.equal(r1["keys"][:n], r2["keys"][:n]) and torch.equal(r1["rows"][:n], r2["rows"][:n])


def test_table_grads_one_digit_sort(torch, oracle_lib):
    """Tables of 251 rows: one 8-bit digit pass sorts the row ids (the first
    pass, which reads idx itself, is also the last).  Every key exact, every
    row against the oracle; most rows are hit by several tokens."""
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), rows=(251,) * 8).with_shape(2, 512)
    print("[tiny bwd] 8 tables of 251 rows, B=2 T=512", flush=True)
    modes = (eg.ENGRAM_GRAD_SORTED_SPARSE, eg.ENGRAM_GRAD_SORTED_DENSE)
    inp, dp, bufs, out = _fwd_bwd(torch, wl, modes)
    p = H.oracle_problem(inp)
    ref = p.table_grad_dense(inp.dy)
    idx = p.hash()
    assert idx.max() < 251
    keys, rows = _sparse_to_dict(out[eg.ENGRAM_GRAD_SORTED_SPARSE], wl.dim)
    want = np.unique(np.concatenate([(np.int64(j) << 32) | idx[:, j].astype(np.int64)
                                     for j in range(wl.J)]))
    assert np.array_equal(keys, want)
    ref_rows = np.stack([ref[int(k >> 32)][int(k & 0xFFFFFFFF)] for k in keys])
    err = H.rel_l2(rows, ref_rows)
    dense = out[eg.ENGRAM_GRAD_SORTED_DENSE]["dense"]
    err_d = H.rel_l2(np.concatenate([d.cpu().numpy().astype(np.float64).ravel() for d in dense]),
                     np.concatenate([r.ravel() for r in ref]))
    print(f"  {len(keys)} keys for {idx.size} lookups: rel L2 {err:.2e} (dense {err_d:.2e})", flush=True)
    assert err <= 1e-3 and err_d <= 1e-3, (err, err_d)


def test_table_grads_one_long_segment_per_table(torch, oracle_lib):
    """A constant token stream: past the first few positions every table's
    keys are one segment of nearly N elements, summed by a whole block of lane
    groups.  Every key exact, every row against the oracle."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("tiny").with_shape(1, 20000)
    print("[tiny bwd] constant tokens B=1 T=20000", flush=True)
    inp = synth.Inputs(wl)
    tok = np.full((wl.B, wl.T), 7, np.int32)
    dp = H.DeviceProblem(inp, tokens=tok)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    dy = H.to_dev(inp.dy)
    sparse = dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_SPARSE)
    dense = dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_DENSE)["dense"]
    torch.cuda.synchronize()
    keys, rows = _sparse_to_dict(sparse, wl.dim)
    p = H.oracle_problem(inp, tokens=tok)
    idx = p.hash()
    want = np.unique(np.concatenate([(np.int64(j) << 32) | idx[:, j].astype(np.int64)
                                     for j in range(wl.J)]))
    assert np.array_equal(keys, want)
    longest = max(np.unique(idx[:, j], return_counts=True)[1].max() for j in range(wl.J))
    assert longest >= wl.T - 4, longest
    ref = p.table_grad_dense(inp.dy)
    ref_rows = np.stack([ref[int(k >> 32)][int(k & 0xFFFFFFFF)] for k in keys])
    err = H.rel_l2(rows, ref_rows)
    worst = max(H.rel_l2(rows[i], ref_rows[i]) for i in range(len(keys)))
    print(f"  {len(keys)} keys, longest segment {longest}: rel L2 {err:.2e}, worst row {worst:.2e}",
          flush=True)
    assert err <= 1e-3 and worst <= 1e-3, (err, worst)
    got = np.concatenate([d.cpu().numpy().astype(np.float64).ravel() for d in dense])
    assert H.rel_l2(got, np.concatenate([r.ravel() for r in ref])) <= 1e-3


def test_table_grads_many_sort_blocks(torch, oracle_lib):
    """270000 tokens: more than 64 sort blocks per table, where a separate
    scan kernel writes the digit offsets.  Every key exact; every row against
    the atomic scatter; sampled rows (the 8 most-hit keys and 200 seeded
    random ones) against the oracle."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("tiny").with_shape(1, 270000)
    print("[tiny bwd] B=1 T=270000", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    dy = H.to_dev(inp.dy)
    sparse = dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_SPARSE)
    atomic = dp.backward(bufs, dy, eg.ENGRAM_GRAD_ATOMIC_DENSE)["dense"]
    torch.cuda.synchronize()
    keys, rows = _sparse_to_dict(sparse, wl.dim)
    p = H.oracle_problem(inp)
    idx = p.hash()
    all_keys = np.concatenate([(np.int64(j) << 32) | idx[:, j].astype(np.int64) for j in range(wl.J)])
    uk, cnt = np.unique(all_keys, return_counts=True)
    assert np.array_equal(keys, uk)
    kj = (keys >> 32).astype(np.int64)
    kr = (keys & 0xFFFFFFFF).astype(np.int64)
    a = np.concatenate([atomic[j].cpu().numpy().astype(np.float64)[kr[kj == j]] for j in range(wl.J)])
    err_a = H.rel_l2(rows, a)
    picked = set(int(k) for k in uk[np.argsort(-cnt, kind="stable")[:8]])
    picked.update(int(keys[int(q)]) for q in synth.u64_stream(23, 200) % np.uint64(len(keys)))
    sel = sorted(picked)
    rj = np.array([k >> 32 for k in sel], np.int32)
    rr = np.array([k & 0xFFFFFFFF for k in sel], np.int32)
    ref, npos = p.table_grad_rows(inp.dy, idx, rj, rr)
    key_pos = {int(k): i for i, k in enumerate(keys)}
    got = np.stack([rows[key_pos[k]] for k in sel])
    err = H.rel_l2(got, ref)
    print(f"  {len(keys)} keys; sorted vs atomic rel L2 {err_a:.2e}; {len(sel)} sampled rows "
          f"({npos} positions) vs oracle {err:.2e}", flush=True)
    assert err_a <= 1e-3 and err <= 1e-3, (err_a, err)


def test_engram27b_table_grads_sampled(torch, oracle_lib):
    """27B-scale shapes: every key exact; against the oracle, the rows of the
    64 most-hit keys (the longest segments), the most-hit row of every table
    and 24 seeded random keys."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("engram27b_bwd")
    print("[engram27b_bwd] forward + sorted and atomic backward", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    dy = H.to_dev(inp.dy)
    sparse = dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_SPARSE)
    torch.cuda.synchronize()
    keys, rows = _sparse_to_dict(sparse, wl.dim)
    p = H.oracle_problem(inp)
    idx = p.hash()
    assert np.array_equal(bufs["idx"].cpu().numpy(), idx)
    want = np.unique(np.concatenate([(np.int64(j) << 32) | idx[:, j].astype(np.int64)
                                     for j in range(wl.J)]))
    assert np.array_equal(keys, want)
    # pick rows: the 64 most-hit keys, the most-hit row of every table, seeded random keys
    all_keys = np.concatenate([(np.int64(j) << 32) | idx[:, j].astype(np.int64) for j in range(wl.J)])
    uk, cnt = np.unique(all_keys, return_counts=True)
    picked = set(int(k) for k in uk[np.argsort(-cnt, kind="stable")[:64]])
    for j in range(wl.J):
        vals, c = np.unique(idx[:, j], return_counts=True)
        picked.add((j << 32) | int(vals[np.argmax(c)]))
    picks = synth.u64_stream(21, 24) % np.uint64(len(keys))
    picked.update(int(keys[int(q)]) for q in picks)
    sel = [(k >> 32, k & 0xFFFFFFFF) for k in sorted(picked)]
    rj = np.array([s[0] for s in sel], np.int32)
    rr = np.array([s[1] for s in sel], np.int32)
    ref, npos = p.table_grad_rows(inp.dy, idx, rj, rr)
    print(f"  oracle used {npos} positions", flush=True)
    key_pos = {int(k): i for i, k in enumerate(keys)}
    got = np.stack([rows[key_pos[(int(j) << 32) | int(r)]] for j, r in zip(rj, rr)])
    err = H.rel_l2(got, ref)
    print(f"  rel L2 = {err:.3e}", flush=True)
    assert err <= 1e-3, err
    # rows hit once or twice, under a bound of their own: the heavy segments
    # above dominate a pooled norm, so an error confined to the light rows
    # (most rows of a Zipf stream) would hide there
    rng_pick = synth.u64_stream(22, 4096)
    light = []
    for hits, want_n in ((1, 384), (2, 256)):
        cand = uk[cnt == hits]
        sel_i = np.unique(rng_pick % np.uint64(len(cand)))[:want_n]
        light.append(cand[sel_i.astype(np.int64)])
    light = np.concatenate(light)
    lj = (light >> 32).astype(np.int32)
    lr = (light & 0xFFFFFFFF).astype(np.int32)
    ref_l, npos_l = p.table_grad_rows(inp.dy, idx, lj, lr)
    got_l = np.stack([rows[key_pos[int(k)]] for k in light])
    err_l = H.rel_l2(got_l, ref_l)
    worst = max(H.rel_l2(got_l[i], ref_l[i]) for i in range(len(light)))
    print(f"  {len(light)} single/double-hit rows ({npos_l} positions): rel L2 = {err_l:.3e}, "
          f"worst row {worst:.3e}", flush=True)
    assert len(light) >= 512 and err_l <= 1e-3, err_l
    # the atomic variant agrees with the sorted one on every key (on the GPU)
    dense = dp.backward(bufs, dy, eg.ENGRAM_GRAD_ATOMIC_DENSE)["dense"]
    torch.cuda.synchronize()
    n = int(sparse["count"].item())
    skeys = sparse["keys"][:n]
    srows = sparse["rows"][:n]
    num = torch.zeros((), dtype=torch.float64, device="cuda")
    den = torch.zeros((), dtype=torch.float64, device="cuda")
    for j in range(wl.J):
        m = (skeys >> 32) == j
        r = (skeys[m] & 0xFFFFFFFF).long()
        a = dense[j][r].double()
        b = srows[m].double()
        num += ((a - b) ** 2).sum()
        den += (b ** 2).sum()
    err_all = float((num / den).sqrt())
    print(f"  atomic vs sorted over all {n} keys: rel L2 = {err_all:.3e}", flush=True)
    assert err_all <= 1e-3, err_all


def test_training_backward_concurrent_streams(torch):
    """Training backward (sparse table gradients and every parameter gradient)
    of single-sequence slices issued on three streams at once equals the same
    calls made one after another on one stream, bit for bit."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("small").with_shape(6, 4096)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    saved = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(saved)
    dy = H.to_dev(inp.dy)
    T, J, D, d = dp.T, wl.J, wl.dim, wl.hidden
    n_ws = eg.engram_workspace_size(dp.cfg, 1, T, eg.ENGRAM_OP_BACKWARD_PARAMS)

    def run(streams):
        ws = [torch.empty(n_ws, dtype=torch.uint8, device="cuda") for _ in streams]
        # every output exists (and count is zeroed, a kernel on the default
        # stream) before the event that the side streams wait for
        outs = [{"keys": torch.empty(T * J, dtype=torch.int64, device="cuda"),
                 "rows": torch.empty(T * J, D, dtype=torch.float32, device="cuda"),
                 "count": torch.zeros(1, dtype=torch.int64, device="cuda"),
                 "w_kv": torch.empty(2 * d, wl.d_mem, dtype=torch.float32, device="cuda"),
                 "conv_w": torch.empty(d, wl.taps, dtype=torch.float32, device="cuda"),
                 "gamma_q": torch.empty(d, dtype=torch.float32, device="cuda"),
                 "gamma_k": torch.empty(d, dtype=torch.float32, device="cuda"),
                 "hidden": torch.empty(1, T, d, dtype=dp.tdtype, device="cuda")} for _ in range(dp.B)]
        ev = torch.cuda.Event()
        ev.record()
        for st in streams:
            st.wait_event(ev)
        for b in range(dp.B):
            rows = slice(b * T, (b + 1) * T)
            o = outs[b]
            tg = eg.engram_table_grad()
            tg.mode = eg.ENGRAM_GRAD_SORTED_SPARSE
            tg.keys, tg.rows, tg.count = o["keys"].data_ptr(), o["rows"].data_ptr(), o["count"].data_ptr()
            pg = eg.make_param_grad(**{k: o[k] for k in ("w_kv", "conv_w", "gamma_q", "gamma_k", "hidden")})
            sv = eg.make_saved(**{k: t[rows] for k, t in saved.items()})
            eg.engram_backward(dp.cfg, dp.params, dp.hidden[b:b + 1], dy[b:b + 1], B=1, T=T, saved=sv,
                               table_out=tg, param_out=pg, workspace=ws[b % len(streams)],
                               stream=streams[b % len(streams)])
        torch.cuda.synchronize()
        return outs

    serial = run([torch.cuda.current_stream()])
    for rep in range(2):
        conc = run([torch.cuda.Stream() for _ in range(3)])
        for b, (x, y) in enumerate(zip(serial, conc)):
            n = int(x["count"].item())
            assert n == int(y["count"].item()), (rep, b)
            assert torch.equal(x["keys"][:n], y["keys"][:n]) and torch.equal(x["rows"][:n], y["rows"][:n]), (rep, b)
            for k in ("w_kv", "conv_w", "gamma_q", "gamma_k", "hidden"):
                assert torch.equal(x[k], y[k]), (rep, b, k)
        print(f"  rep {rep}: {dp.B} slices identical", flush=True)
