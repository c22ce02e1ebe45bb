"""Host-resident tables: the prefetch plan gathers the distinct rows into
pinned staging and copies them on a side stream; the compact-mode forward
must be bit-identical to the forward that reads the tables in HBM."""
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


@pytest.mark.parametrize("name,B,T", [("tiny", 2, 300), ("small", 2, 2048)])
def test_compact_forward_bit_identical(torch, oracle_lib, name, B, T):
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload(name).with_shape(B, T)
    print(f"[prefetch {name}] B={B} T={T}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    y_ref = dp.forward()
    N, J = dp.N, wl.J
    cap = N * J
    es = 2 if wl.dtype == "bf16" else 4
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(cap, np.int32)
    inv_h = torch.empty(N, J, dtype=torch.int32, pin_memory=True)
    staging = torch.empty(cap * wl.dim * es, dtype=torch.uint8, pin_memory=True)
    rows_dev = torch.empty(cap * wl.dim * es, dtype=torch.uint8, device="cuda")
    inv_dev = torch.empty(N, J, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()  # creates the underlying hipEvent; the planner re-records it on `side`
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host = counts.ctypes.data, uniq.ctypes.data
    plan.inverse_host, plan.staging_host = inv_h.data_ptr(), staging.data_ptr()
    plan.rows_dev, plan.inverse_dev = rows_dev.data_ptr(), inv_dev.data_ptr()
    plan.ready_event = ev.cuda_event
    host_tables = [inp.table(j) for j in range(J)]
    eg.engram_prefetch_plan(dp.cfg, inp.canon_map, inp.tokens, B=B, T=T, host_tables=host_tables,
                            plan=plan, side_stream=side)
    bufs = dp.alloc_saved(("idx",))
    y = dp.forward(bufs, compact=plan)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    # the plan agrees with the oracle's sorted-unique rows and inverse map
    p = H.oracle_problem(inp)
    u_ref, c_ref, inv_ref = oracle_lib.prefetch_plan(p.hash())
    assert np.array_equal(counts, c_ref)
    assert np.array_equal(uniq[: plan.total_rows], u_ref)
    base = np.concatenate([[0], np.cumsum(c_ref)[:-1]]).astype(np.int32)
    assert np.array_equal(bufs["idx"].cpu().numpy(), inv_ref + base[None, :])


def test_plan_ahead_then_reuse(torch, oracle_lib):
    """Indices planned ahead (no host tables), then gather + copy only
    (ENGRAM_PLAN_REUSE): same compact forward as the HBM forward."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("small").with_shape(2, 2048)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    y_ref = dp.forward()
    N, J = dp.N, wl.J
    cap = N * J
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(cap, np.int32)
    inv_h = torch.empty(N, J, dtype=torch.int32, pin_memory=True)
    staging = torch.empty(cap * wl.dim * 2, dtype=torch.uint8, pin_memory=True)
    rows_dev = torch.empty(cap * wl.dim * 2, dtype=torch.uint8, device="cuda")
    inv_dev = torch.empty(N, J, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host = counts.ctypes.data, uniq.ctypes.data
    plan.inverse_host, plan.staging_host = inv_h.data_ptr(), staging.data_ptr()
    plan.rows_dev, plan.inverse_dev = rows_dev.data_ptr(), inv_dev.data_ptr()
    plan.ready_event = ev.cuda_event
    eg.engram_prefetch_plan(dp.cfg, inp.canon_map, inp.tokens, B=dp.B, T=dp.T, host_tables=None,
                            plan=plan, side_stream=side)
    assert plan.total_rows == int(counts.sum()) > 0
    plan.flags = eg.ENGRAM_PLAN_REUSE
    host_tables = [inp.table(j) for j in range(J)]
    eg.engram_prefetch_plan(dp.cfg, inp.canon_map, inp.tokens, B=dp.B, T=dp.T,
                            host_tables=host_tables, plan=plan, side_stream=side)
    y = dp.forward(compact=plan)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    # a reused plan whose rows fall outside the tables is rejected on the host
    uniq[0] = int(inp.table_rows[0])
    with pytest.raises(eg.EngramError):
        eg.engram_prefetch_plan(dp.cfg, inp.canon_map, inp.tokens, B=dp.B, T=dp.T,
                                host_tables=host_tables, plan=plan, side_stream=side)


@pytest.mark.parametrize("name,B,T,batches,ahead", [("tiny", 2, 300, 6, False), ("tiny", 2, 300, 6, True),
                                                    ("small", 2, 2048, 4, True)])
def test_row_ring_across_batches(torch, name, B, T, batches, ahead):
    """HBM row ring over successive batches of one token stream, planned in
    the copying call or ahead of it: the compact forward stays bit-identical
    to the HBM forward, every inverse entry points at a ring row holding its
    table row, rows found in the ring are not copied again, and the ring
    wraps."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload(name).with_shape(B, T)
    print(f"[row ring {name}] B={B} T={T} batches={batches}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    N, J = dp.N, wl.J
    cap = N * J
    R = 2 * cap + cap // 2
    es = 2 if wl.dtype == "bf16" else 4
    rb = wl.dim * es
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(cap, np.int32)
    inv_h = torch.empty(N, J, dtype=torch.int32, pin_memory=True)
    staging = torch.empty(cap * rb, dtype=torch.uint8, pin_memory=True)
    ring = torch.zeros(R * rb, dtype=torch.uint8, device="cuda")
    inv_dev = torch.empty(N, J, dtype=torch.int32, device="cuda")
    ring_pos = np.full(int(inp.table_rows.sum()), -1, np.int64)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host = counts.ctypes.data, uniq.ctypes.data
    plan.inverse_host, plan.staging_host = inv_h.data_ptr(), staging.data_ptr()
    plan.rows_dev, plan.inverse_dev = ring.data_ptr(), inv_dev.data_ptr()
    plan.ready_event = ev.cuda_event
    plan.ring_rows, plan.ring_pos, plan.ring_head = R, ring_pos.ctypes.data, 0
    host_tables = [inp.table(j) for j in range(J)]
    tables_u8 = [np.ascontiguousarray(t).view(np.uint8).reshape(t.shape[0], rb) for t in host_tables]
    hits_total = 0
    for k in range(batches):
        tok = synth.zipf_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                                offset=k * N).reshape(B, T)
        dp.tokens_host = tok
        dp.tokens = H.to_dev(tok)
        y_ref = dp.forward()
        head0 = plan.ring_head
        plan.flags = 0
        if ahead:
            eg.engram_prefetch_plan(dp.cfg, inp.canon_map, tok, B=B, T=T, host_tables=None, plan=plan)
            plan.flags = eg.ENGRAM_PLAN_REUSE
        eg.engram_prefetch_plan(dp.cfg, inp.canon_map, tok, B=B, T=T, host_tables=host_tables,
                                plan=plan, side_stream=side)
        y = dp.forward(compact=plan)
        idx = dp.hash()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), k
        assert plan.ring_head - head0 == plan.total_rows  # the misses, all copied
        hits_total += plan.ring_hits if k else 0
        if k == 0:
            assert plan.ring_hits == 0
        # ring row of every (token, table) holds that table row, byte for byte
        ringh = ring.cpu().numpy().reshape(R, rb)
        inv = inv_dev.cpu().numpy()
        idxh = idx.cpu().numpy()
        for j in range(J):
            assert np.array_equal(ringh[inv[:, j]], tables_u8[j][idxh[:, j]]), (k, j)
        print(f"  batch {k}: {plan.total_rows} rows copied, {plan.ring_hits} found in the ring, "
              f"head {plan.ring_head}", flush=True)
    assert hits_total > 0
    assert plan.ring_head > R  # wrapped


def _pinned_tables(torch, inp, J):
    """The host tables copied into pinned host memory (as a serving host would hold them)."""
    out = []
    for j in range(J):
        t = np.ascontiguousarray(inp.table(j))
        p = torch.empty(t.nbytes, dtype=torch.uint8, pin_memory=True)
        p.numpy()[:] = t.view(np.uint8).reshape(-1)
        out.append(p)
    return out


def _host_plan(torch, eg, N, J, rb, ring_rows=0):
    cap = N * J
    st = {"counts": np.zeros(J, np.int64), "uniq": np.zeros(cap, np.int32),
          "inv_h": torch.empty(N, J, dtype=torch.int32, pin_memory=True),
          "staging": torch.empty(cap * rb, dtype=torch.uint8, pin_memory=True),
          "rows": torch.zeros(max(ring_rows, cap) * rb, dtype=torch.uint8, device="cuda"),
          "inv_dev": torch.empty(N, J, dtype=torch.int32, device="cuda"),
          "side": torch.cuda.Stream(), "ev": torch.cuda.Event()}
    st["ev"].record()
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host = st["counts"].ctypes.data, st["uniq"].ctypes.data
    plan.inverse_host, plan.staging_host = st["inv_h"].data_ptr(), st["staging"].data_ptr()
    plan.rows_dev, plan.inverse_dev = st["rows"].data_ptr(), st["inv_dev"].data_ptr()
    plan.ready_event = st["ev"].cuda_event
    return plan, st


def test_host_tables_at_the_100b_widths(torch, oracle_lib):
    """The host-table path at the widths of the 100B-parameter table
    ("DeepSeek AI II", system-efficiency part; the QbitAI mirror's host
    offload): D = 128, d = 4096, 4 x 8192 tokens, 16 pinned host tables of
    ~1M x 128 rows.  The plan is bit-exact against the oracle's, the compact
    forward is bit-identical to the forward over the same tables in HBM and
    within the bf16 bar of the oracle at 1024 sampled positions; then the
    HBM row ring over three more batches at the same widths."""
    import dataclasses

    import hashed_gram_embedding_canon_amd as eg
    from synth.workloads import primes_from
    wl = dataclasses.replace(synth.get_workload("host100b"), rows=tuple(primes_from(1_000_003, 16)),
                             B=4, T=8192)
    print(f"[host tables, 100B widths] B={wl.B} T={wl.T} D={wl.dim} d={wl.hidden}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    N, J, rb = dp.N, wl.J, wl.dim * 2
    host_tables = _pinned_tables(torch, inp, J)
    plan, st = _host_plan(torch, eg, N, J, rb)
    eg.engram_prefetch_plan(dp.cfg, inp.canon_map, inp.tokens, B=wl.B, T=wl.T, host_tables=host_tables,
                            plan=plan, side_stream=st["side"])
    bufs = dp.alloc_saved(("idx",))
    y = dp.forward(bufs, compact=plan)
    y_ref = dp.forward()
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    p = H.oracle_problem(inp)
    u_ref, c_ref, inv_ref = oracle_lib.prefetch_plan(p.hash())
    assert np.array_equal(st["counts"], c_ref)
    assert np.array_equal(st["uniq"][: plan.total_rows], u_ref)
    base = np.concatenate([[0], np.cumsum(c_ref)[:-1]]).astype(np.int32)
    assert np.array_equal(bufs["idx"].cpu().numpy(), inv_ref + base[None, :])
    pos = H.sample_positions(wl.B, wl.T, 1024, seed=41)
    ref = p.forward(pos, want=("y",))["y"]
    err = H.rel_max_err(H.to_host_f64(y).reshape(-1, wl.hidden)[pos], ref)
    print(f"  compact forward vs oracle at {pos.size} positions: {err:.3e}", flush=True)
    assert err <= 1e-2
    del st, plan
    # HBM row ring at the same widths, three more batches of the stream
    cap = N * J
    R = 2 * cap + cap // 4
    plan, st = _host_plan(torch, eg, N, J, rb, ring_rows=R)
    ring_pos = np.full(int(inp.table_rows.sum()), -1, np.int64)
    plan.ring_rows, plan.ring_pos, plan.ring_head = R, ring_pos.ctypes.data, 0
    tables_u8 = [h.numpy().reshape(-1, rb) for h in host_tables]
    hits = 0
    for k in range(1, 4):
        tok = synth.zipf_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                                offset=k * N).reshape(wl.B, wl.T)
        dp.tokens_host, dp.tokens = tok, H.to_dev(tok)
        y_ref = dp.forward()
        plan.flags = 0
        eg.engram_prefetch_plan(dp.cfg, inp.canon_map, tok, B=wl.B, T=wl.T, host_tables=host_tables,
                                plan=plan, side_stream=st["side"])
        y = dp.forward(compact=plan)
        idx = dp.hash()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), k
        hits += plan.ring_hits
        ringh = st["rows"].cpu().numpy().reshape(R, rb)
        inv = st["inv_dev"].cpu().numpy()
        idxh = idx.cpu().numpy()
        for j in range(J):
            assert np.array_equal(ringh[inv[:, j]], tables_u8[j][idxh[:, j]]), (k, j)
        print(f"  ring batch {k}: {plan.total_rows} rows copied, {plan.ring_hits} found in the ring",
              flush=True)
    assert hits > 0


@pytest.mark.parametrize("ring", [False, True])
def test_forward_overlaps_next_plan_copy(torch, ring):
    """A forward on plan k queued behind long work on the compute stream, and
    the copies of plan k+1 queued at once on the side stream: with
    consumed_event the copies wait until the forward has read inverse_dev and
    rows_dev, so both forwards equal the forwards over the tables in HBM."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("small").with_shape(2, 2048)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    N, J, rb = dp.N, wl.J, wl.dim * 2
    cap = N * J
    R = 2 * cap + cap // 2 if ring else 0
    plan, st = _host_plan(torch, eg, N, J, rb, ring_rows=R)
    ring_pos = np.full(int(inp.table_rows.sum()), -1, np.int64)
    if ring:
        plan.ring_rows, plan.ring_pos, plan.ring_head = R, ring_pos.ctypes.data, 0
    consumed = torch.cuda.Event()
    consumed.record()
    plan.consumed_event = consumed.cuda_event
    host_tables = [inp.table(j) for j in range(J)]
    toks = [synth.zipf_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                              offset=k * N).reshape(dp.B, dp.T) for k in range(3)]
    refs = []
    for tok in toks:
        dp.tokens = H.to_dev(tok)
        refs.append(dp.forward())
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty_like(a)
    outs = []
    for k, tok in enumerate(toks):
        plan.flags = 0
        eg.engram_prefetch_plan(dp.cfg, inp.canon_map, tok, B=dp.B, T=dp.T, host_tables=host_tables,
                                plan=plan, side_stream=st["side"])
        for _ in range(12):  # the forward waits behind ~10 ms of other work
            torch.matmul(a, b, out=c)
        y = torch.empty_like(refs[0])
        dp.forward(compact=plan, y=y)
        outs.append(y)
    torch.cuda.synchronize()
    for k in range(3):
        assert torch.equal(outs[k], refs[k]), k
