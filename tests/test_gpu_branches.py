"""GPU parity of the multi-branch forward ("DeepSeek AI II", section
"DeepSeek Engram", multi-branch integration): one projection GEMM over
[W_K^(0); ...; W_K^(M-1); W_V], a gate and an output per branch, v shared.
Each branch is checked against the single-branch oracle on its own W_K and
hidden state."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


@pytest.mark.parametrize("dtype,M,B,T", [("f32", 3, 2, 300), ("bf16", 2, 3, 77), ("f32", 1, 1, 64),
                                         ("bf16", 4, 1, 513)])
def test_tiny_branches_full(torch, oracle_lib, dtype, M, B, T):
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype=dtype, branches=M).with_shape(B, T)
    print(f"[branches tiny {dtype}] M={M} B={B} T={T}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    y = dp.forward(bufs)
    torch.cuda.synchronize()
    ys = y.reshape(M, -1, wl.hidden) if M > 1 else y.reshape(1, -1, wl.hidden)
    stats = bufs["stats"].reshape(M, -1, 4)
    for m in range(M):
        p = H.oracle_problem(inp, branch=m)
        if m == 0:
            assert np.array_equal(bufs["idx"].cpu().numpy(), p.hash())
        ref = p.forward(want=("y", "alpha"))
        err = H.rel_max_err(H.to_host_f64(ys[m]), ref["y"])
        a_err = float(np.abs(stats[m, :, 0].cpu().numpy() - ref["alpha"]).max())
        print(f"  branch {m}: max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
        assert err <= TOL[dtype], (m, err)
        assert a_err <= (1e-5 if dtype == "f32" else 1e-2), (m, a_err)


def test_one_branch_matches_default_config(torch):
    """branches = 1 and the default (0) run the same kernels: identical Y."""
    wl = synth.get_workload("tiny").with_shape(2, 300)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    y1 = dp.forward()
    dp.cfg.c.branches = 0
    y0 = dp.forward()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_small_bf16_branches_sampled(torch, oracle_lib):
    wl = dataclasses.replace(synth.get_workload("small"), branches=3).with_shape(2, 2048)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("stats",))
    y = dp.forward(bufs).reshape(3, -1, wl.hidden)
    torch.cuda.synchronize()
    pos = H.sample_positions(dp.B, dp.T, 128, seed=21)
    for m in range(3):
        p = H.oracle_problem(inp, branch=m)
        ref = p.forward(pos, want=("y", "alpha"))
        got = H.to_host_f64(y[m][torch.as_tensor(pos, device=y.device)])
        err = H.rel_max_err(got, ref["y"])
        print(f"  small branch {m}: max-abs-err/max|ref| = {err:.3e}", flush=True)
        assert err <= TOL["bf16"], (m, err)


def test_backward_rejects_branches(torch):
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), branches=2).with_shape(1, 64)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    with pytest.raises(eg.EngramError, match="status 2"):
        dp.backward(bufs, H.to_dev(inp.dy), eg.ENGRAM_GRAD_SORTED_SPARSE)
