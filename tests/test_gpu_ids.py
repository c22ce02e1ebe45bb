"""GPU test of the token-id check (ENGRAM_FLAG_CHECK_IDS) through the C ABI.

Indices depend on the token ids alone ("DeepSeek AI II", section "DeepSeek
Engram"), so an id outside [0, vocab) has no canonical id.  With the check
the kernels never index canon_map out of bounds: every bad id is counted,
read as canonical pad_id, and the call returns ENGRAM_E_INVALID.  The
expected outputs come from the oracle run on the same tokens with each bad
id replaced by a raw id whose canonical id is pad_id (which is what the
kernels compute).  No test here lets a kernel read out of bounds: the bad
ids only ever reach the guarded path.
"""
import dataclasses

import numpy as np
import pytest

import synth
from synth.workloads import primes_from
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


def _workloads():
    tiny = synth.get_workload("tiny").with_shape(2, 256)
    # the 27B row width (160-byte rows: a token's pieces straddle the blocks of
    # the fused hash + gather kernel) over small tables, ragged length
    w27 = dataclasses.replace(synth.get_workload("engram27b"), rows=tuple(primes_from(20011, 16)),
                              B=2, T=700)
    return [tiny, w27]


def _bad_tokens(inp, wl):
    tok = np.array(inp.tokens, dtype=np.int32, copy=True)
    bad = [(0, 17, wl.vocab), (1, 100, -5), (1, wl.T - 1, wl.vocab + 12345), (0, 0, -1)]
    for b, t, x in bad:
        tok[b, t] = x
    # a raw id whose canonical id is pad_id stands for a bad id in the oracle
    sub = int(np.flatnonzero(inp.canon_map == wl.pad_id)[0])
    ref_tok = tok.copy()
    for b, t, _ in bad:
        ref_tok[b, t] = sub
    return tok, ref_tok, len(bad)


@pytest.mark.parametrize("wi", [0, 1])
def test_bad_ids_are_counted_and_rejected(torch, oracle_lib, wi):
    import hashed_gram_embedding_canon_amd as eg
    wl = _workloads()[wi]
    print(f"[ids] {wl.name} B={wl.B} T={wl.T}", flush=True)
    inp = synth.Inputs(wl)
    tok, ref_tok, nbad = _bad_tokens(inp, wl)
    dp = H.DeviceProblem(inp, tokens=tok)
    counter = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    dp.cfg = eg.Config(vocab=wl.vocab, canon_vocab=wl.canon_vocab, orders=wl.orders, heads=wl.heads,
                       dim=wl.dim, hidden=wl.hidden, table_rows=inp.table_rows,
                       multipliers=inp.multipliers, dtype=dp.dtype_code, conv_kernel=wl.taps,
                       rms_eps=wl.rms_eps, pad_id=wl.pad_id, flags=eg.ENGRAM_FLAG_CHECK_IDS,
                       bad_ids=counter)
    p = H.oracle_problem(inp, tokens=ref_tok)
    idx_ref = p.hash()
    # engram_hash_indices
    with pytest.raises(eg.EngramError) as ex:
        dp.hash()
    assert ex.value.status == eg.ENGRAM_E_INVALID
    assert int(counter[0].item()) == nbad
    idx = torch.empty(dp.N, wl.J, dtype=torch.int32, device="cuda")
    with pytest.raises(eg.EngramError):
        eg.engram_hash_indices(dp.cfg, dp.canon, dp.tokens, idx, B=dp.B, T=dp.T)
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    # engram_forward (fused hash + gather): every index and Y as the oracle
    bufs = dp.alloc_saved(("idx", "stats"))
    with pytest.raises(eg.EngramError) as ex:
        y = torch.empty(dp.B, dp.T, wl.hidden, dtype=dp.tdtype, device="cuda")
        eg.engram_forward(dp.cfg, dp.params, dp.tokens, dp.hidden, y, B=dp.B, T=dp.T,
                          saved=eg.make_saved(**bufs), workspace=dp.workspace(eg.ENGRAM_OP_FORWARD))
    assert ex.value.status == eg.ENGRAM_E_INVALID
    assert int(counter[0].item()) == nbad
    assert np.array_equal(bufs["idx"].cpu().numpy(), idx_ref)
    pos = H.sample_positions(dp.B, dp.T, 256, seed=5)
    ref = p.forward(pos, want=("y",))["y"]
    got = H.to_host_f64(y).reshape(-1, wl.hidden)[pos]
    tol = 1e-5 if wl.dtype == "f32" else 1e-2
    assert H.rel_max_err(got, ref) <= tol


def test_valid_ids_pass_the_check_unchanged(torch):
    import hashed_gram_embedding_canon_amd as eg
    wl = _workloads()[1]
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    y0 = dp.forward()
    idx0 = dp.hash()
    counter = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    dp.cfg = eg.Config(vocab=wl.vocab, canon_vocab=wl.canon_vocab, orders=wl.orders, heads=wl.heads,
                       dim=wl.dim, hidden=wl.hidden, table_rows=inp.table_rows,
                       multipliers=inp.multipliers, dtype=dp.dtype_code, conv_kernel=wl.taps,
                       rms_eps=wl.rms_eps, pad_id=wl.pad_id, flags=eg.ENGRAM_FLAG_CHECK_IDS,
                       bad_ids=counter)
    y1 = dp.forward()
    idx1 = dp.hash()
    torch.cuda.synchronize()
    assert int(counter[0].item()) == 0
    assert torch.equal(y0, y1) and torch.equal(idx0, idx1)
