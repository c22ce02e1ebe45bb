"""GPU test of engram_forward_noalloc (the allocation-free forward) through
the C ABI: two calls in a row, the second with a smaller input, each
compared with engram_forward on the same inputs (which uses a caller
workspace).  Both run the same kernels, so the outputs must be identical bit
for bit -- stricter than the forward's tolerance against the oracle."""
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


def _small_tables(name):
    wl = synth.get_workload(name)
    if name == "tiny":
        return wl
    return dataclasses.replace(wl, rows=tuple(primes_from(30011, wl.J)))


def _pair(torch, eg, wl, saved_keys):
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    ref_bufs = dp.alloc_saved(saved_keys)
    y_ref = dp.forward(ref_bufs)
    bufs = dp.alloc_saved(saved_keys)
    for b in bufs.values():
        b.fill_(-7)
    y = torch.full_like(y_ref, float("nan"))
    eg.engram_forward_noalloc(dp.cfg, dp.params, dp.tokens, dp.hidden, y, B=dp.B, T=dp.T,
                              saved=eg.make_saved(**bufs) if bufs else None)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    for k in saved_keys:
        assert torch.equal(bufs[k], ref_bufs[k]), k
    return dp


@pytest.mark.parametrize("name,shapes", [("tiny", [(2, 256), (1, 77)]),
                                         ("small", [(2, 1024), (1, 300)]),
                                         ("engram27b", [(2, 1500), (1, 333)])])
def test_noalloc_matches_forward_twice(torch, name, shapes):
    import hashed_gram_embedding_canon_amd as eg
    base = _small_tables(name)
    for i, (B, T) in enumerate(shapes):
        wl = base.with_shape(B, T)
        print(f"[noalloc] {name} call {i}: B={B} T={T}", flush=True)
        _pair(torch, eg, wl, ("idx", "stats") if i == 0 else ())


def test_noalloc_refuses_oversized_input(torch):
    import hashed_gram_embedding_canon_amd as eg
    wl = _small_tables("engram27b").with_shape(1, 64)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    per_tok = eg.engram_workspace_size(dp.cfg, 1, 1024, eg.ENGRAM_OP_FORWARD) / 1024
    T = int(eg.ENGRAM_NOALLOC_SCRATCH_BYTES / per_tok) + 2048
    y = torch.empty(1, T, wl.hidden, dtype=dp.tdtype, device="cuda")
    with pytest.raises(eg.EngramError) as ex:
        # the host refuses before any kernel reads the (too short) inputs
        eg.engram_forward_noalloc(dp.cfg, dp.params, dp.tokens, dp.hidden, y, B=1, T=T)
    assert ex.value.status == eg.ENGRAM_E_SCRATCH
