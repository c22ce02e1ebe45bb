"""GPU parity of the forward with the LDS dedup of repeated rows inside a
gather tile (ENGRAM_FLAG_GATHER_DEDUP): the same indices, gathered rows and
outputs as the forward without it, bit for bit, on the i.i.d. Zipf stream and
on a stream with local repetition (where a tile holds many repeated rows),
and the gathered rows exactly the oracle's."""
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


def _wl(name, B, T):
    wl = synth.get_workload(name)
    if name != "tiny":
        wl = dataclasses.replace(wl, rows=tuple(primes_from(20011, wl.J)))
    return wl.with_shape(B, T)


@pytest.mark.parametrize("name,B,T", [("tiny", 2, 300), ("small", 3, 257), ("engram27b", 2, 1000),
                                      ("engram40b", 1, 700)])
@pytest.mark.parametrize("stream", ["zipf", "repeat"])
def test_dedup_gather_matches_plain(torch, oracle_lib, name, B, T, stream):
    import hashed_gram_embedding_canon_amd as eg
    wl = _wl(name, B, T)
    print(f"[dedup {name} {stream}] B={B} T={T}", flush=True)
    inp = synth.Inputs(wl)
    tok = None
    if stream == "repeat":
        tok = synth.repeat_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), B * T - (B * T) % 4, wl.vocab,
                                  wl.zipf_s)
        tok = np.concatenate([tok, np.zeros((B * T) % 4, np.int32)]).reshape(B, T)
    plain = H.DeviceProblem(inp, tokens=tok)
    dd = H.DeviceProblem(inp, tokens=tok, flags=eg.ENGRAM_FLAG_GATHER_DEDUP)
    b0 = plain.alloc_saved(("idx", "stats", "e"))
    b1 = dd.alloc_saved(("idx", "stats", "e"))
    y0 = plain.forward(b0)
    y1 = dd.forward(b1)
    y2 = dd.forward()  # e in the workspace
    torch.cuda.synchronize()
    assert torch.equal(b0["idx"], b1["idx"])
    assert torch.equal(b0["e"], b1["e"])
    assert torch.equal(y0, y1) and torch.equal(y0, y2)
    assert torch.equal(b0["stats"], b1["stats"])
    p = H.oracle_problem(inp, tokens=plain.tokens_host)
    pos = H.sample_positions(B, T, 128, seed=3)
    ref = p.forward(pos, want=("e",))["e"]
    assert np.array_equal(H.to_host_f64(b1["e"])[pos], ref)
