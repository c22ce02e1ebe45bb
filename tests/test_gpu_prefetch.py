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
